"""GPU parity of the ternary-sketch channel screen: the load-time sketch bit-exact against the
oracle (codes, FP16 scales and rho, decided in the same fp32 operation order), and the screened
layer's kept ids exactly and y within tolerance, at small ragged shapes and at the full
40-layer-stack shapes."""
import numpy as np
import pytest

from gpu_common import CH_MARGIN_REL, MARGIN, TOL_BF16, HostLayer, cuda_ok, rel_err
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O
from oracle import sketch_oracle as S

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]

MODES = {"gate_dnorm": 0, "router_weighted": 1}


def _layer(wl, layer=0):
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=1)
    return M.Layer(desc, T.device_layer(wl, layer))


def _build(L, wl, layer=0):
    import torch
    signs = torch.from_numpy(T.rotation_signs(wl, layer)).cuda()
    buf = L.build_sketch(signs)
    torch.cuda.synchronize()
    return buf, signs


def _nbp(wl):
    """Row stride of the FP16 scales and rho: H/128 rounded up to a multiple of 8."""
    return (wl.H // 128 + 7) // 8 * 8


def _regions(wl):
    """Byte offsets of the sketch buffer's regions (the header's layout)."""
    rows = wl.E * wl.I
    al = lambda n: (n + 255) // 256 * 256
    cb, sb = rows * (wl.H // 16) * 4, rows * _nbp(wl) * 2
    o, offs = 0, []
    for n in (cb, cb, sb, sb, sb, sb):
        offs.append((o, n))
        o = al(o + n)
    return offs


def _unpack(buf, wl, rows):
    """codes [len(rows)][H] int8 and alpha, rho (FP16 bit patterns) of G and V for the rows."""
    b = buf.cpu().numpy()
    offs = _regions(wl)
    out = []
    for t in range(2):
        o, n = offs[t]
        words = b[o:o + n].view(np.uint32).reshape(wl.E * wl.I, wl.H // 16)[rows]
        fields = (words[:, :, None] >> (2 * np.arange(16, dtype=np.uint32))[None, None, :]) & 3
        assert not np.any(fields == 2), "invalid 2-bit code"
        codes = np.where(fields == 3, -1, fields).astype(np.int8).reshape(len(rows), wl.H)
        oa, na = offs[2 + t]
        orr, nr = offs[4 + t]
        nb = wl.H // 128
        alpha = b[oa:oa + na].view(np.uint16).reshape(wl.E * wl.I, _nbp(wl))[rows]
        rho = b[orr:orr + nr].view(np.uint16).reshape(wl.E * wl.I, _nbp(wl))[rows]
        assert not np.any(alpha[:, nb:]) and not np.any(rho[:, nb:]), "padding not zero"
        alpha, rho = alpha[:, :nb], rho[:, :nb]
        out.append((codes, alpha, rho))
    return out


def _check_rows(buf, wl, hl, signs_np, rows):
    got = _unpack(buf, wl, rows)
    by_expert = {}
    for r in rows:
        by_expert.setdefault(int(r) // wl.I, []).append(int(r) % wl.I)
    pos = {int(r): i for i, r in enumerate(rows)}
    for e, js in by_expert.items():
        G, V, _ = hl.expert(e)
        for t, W in enumerate((G, V)):
            ref_c, ref_a, ref_r = S.sketch_rows(O._row(W, js[0]) if len(js) == 1 else
                                                _rows(W, js), signs_np)
            for q, j in enumerate(js):
                i = pos[e * wl.I + j]
                assert np.array_equal(got[t][0][i], ref_c[q]), (e, j, t)
                assert np.array_equal(got[t][1][i], ref_a[q].view(np.uint16)), (e, j, t)
                assert np.array_equal(got[t][2][i], ref_r[q].view(np.uint16)), (e, j, t)


def _rows(W, js):
    if isinstance(W, tuple):
        return ("bf16", W[1][js])
    return np.asarray(W)[js]


SMALL = [
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=171, H=384, E=9, k=3, I=40, n_shared=1,
              I_shared=24, layers=1),
    T.reduced(WORKLOADS["tiny_f32"], wid=172, H=256, E=6, k=2, I=16, n_shared=1,
              I_shared=8, shared_dtype="f32"),
    T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=173, H=2048, E=24, k=8, I=96, n_shared=1,
              I_shared=64, layers=1),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}I{w.I}{w.expert_dtype}")
def test_sketch_build_bit_exact(wl):
    L = _layer(wl)
    hl = HostLayer(wl)
    buf, _ = _build(L, wl)
    _check_rows(buf, wl, hl, T.rotation_signs(wl, 0), np.arange(wl.E * wl.I))


def test_sketch_build_full_size_sampled():
    """H=2048, E=256, I=768 (the stack's layer 3): 96 sampled rows of G and V, bit-exact."""
    import torch
    wl = WORKLOADS["qwen35_a3b_sparse"]
    L = _layer(wl, 3)
    hl = HostLayer(wl, 3)
    buf, _ = _build(L, wl, 3)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(wl.E * wl.I, 96, replace=False))
    _check_rows(buf, wl, hl, T.rotation_signs(wl, 3), rows)
    L.close()
    del L, buf
    torch.cuda.empty_cache()


def _pick(wl, hl, token, keep, mode, signs_np, sk_cache, layer=0):
    """First redraw of x with a top-k router margin and a K-th/(K+1)-th sketch-score margin."""
    dn = {}

    def dnorm_of(e):
        if e not in dn:
            dn[e] = O.down_norms(hl.expert(e)[2])
        return dn[e]

    def sketch_of(e):
        if e not in sk_cache:
            G, V, _ = hl.expert(e)
            sk_cache[e] = (S.sketch_rows(G, signs_np), S.sketch_rows(V, signs_np))
        return sk_cache[e]

    for a in range(64):
        x = T.x(wl, token, layer, a)
        logits = O.router_logits(x, hl.router)[0]
        if O.topk_margin(logits, wl.k) < MARGIN:
            continue
        ids, w = O.route(logits[None], wl.k)
        s, _, _ = S.sketch_scores(x, ids[0], w[0], sketch_of, dnorm_of, signs_np, mode)
        srt = np.sort(s.ravel())[::-1]
        if 0 < keep < srt.size and srt[keep - 1] - srt[keep] < CH_MARGIN_REL * srt[0]:
            continue
        return x, ids[0], w[0], dnorm_of, sketch_of
    raise RuntimeError("no margin-satisfying draw")


def _screen(L, x_np, keep, mode, ids=None, w=None):
    """The screened layer on the GPU; with ids and w the routing is given (no router inside:
    every workgroup scans z itself instead of sharing the scans)."""
    import torch
    x = torch.from_numpy(np.asarray(x_np, dtype=np.float32)).cuda().reshape(1, -1)
    y = torch.empty_like(x)
    kept = torch.full((max(keep, 1),), -1, dtype=torch.int32, device="cuda")
    kw = {}
    if ids is not None:
        kw = dict(ids=torch.from_numpy(np.asarray(ids, dtype=np.int32)).cuda().reshape(1, -1),
                  w=torch.from_numpy(np.asarray(w, dtype=np.float32)).cuda().reshape(1, -1))
    L.channel_select(x, keep, kept, y=y, mode=mode, sketch=True, **kw)
    assert L.check() == 0
    return kept.cpu().numpy()[:keep], y.cpu().numpy()[0]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"H{w.H}E{w.E}I{w.I}{w.expert_dtype}")
def test_sketch_screen_small(wl, mode):
    L = _layer(wl)
    hl = HostLayer(wl)
    _build(L, wl)
    signs_np = T.rotation_signs(wl, 0)
    cache = {}
    n = wl.k * wl.I
    for tok, keep in enumerate([1, n // 8, n // 3 + 1, n - 1, n, 0]):
        x, ids, w, dnorm_of, sketch_of = _pick(wl, hl, tok, keep, mode, signs_np, cache)
        kept_ref, y_ref = S.sketch_select_token(x, ids, w, hl.expert, sketch_of, dnorm_of, keep,
                                                signs_np, hl.shared, mode)
        kept, y = _screen(L, x, keep, MODES[mode])
        assert kept.tolist() == kept_ref.tolist(), (tok, keep)
        assert rel_err(y, y_ref) <= TOL_BF16, (tok, keep, rel_err(y, y_ref))


@pytest.mark.parametrize("wl", SMALL[:2], ids=lambda w: f"H{w.H}E{w.E}I{w.I}{w.expert_dtype}")
def test_sketch_screen_given_routing(wl):
    """Routing passed in (the oracle's top-k ids and softmax weights): the path where each
    workgroup scans every block of z itself."""
    L = _layer(wl)
    hl = HostLayer(wl)
    _build(L, wl)
    signs_np = T.rotation_signs(wl, 0)
    cache = {}
    n = wl.k * wl.I
    for tok, keep in enumerate([1, n // 3 + 1, n - 1]):
        x, ids, w, dnorm_of, sketch_of = _pick(wl, hl, 40 + tok, keep, "router_weighted",
                                               signs_np, cache)
        kept_ref, y_ref = S.sketch_select_token(x, ids, w, hl.expert, sketch_of, dnorm_of, keep,
                                                signs_np, hl.shared, "router_weighted")
        kept, y = _screen(L, x, keep, 1, ids=ids, w=w)
        assert kept.tolist() == kept_ref.tolist(), (tok, keep)
        assert rel_err(y, y_ref) <= TOL_BF16, (tok, keep, rel_err(y, y_ref))


@pytest.mark.parametrize("keep", [799, 1106])
def test_sketch_screen_full_size(keep):
    """The stack's shapes (H=2048, E=256, k=8, I=768, one shared expert), eq.-1 scores."""
    import torch
    wl = WORKLOADS["qwen35_a3b_sparse"]
    L = _layer(wl, 1)
    hl = HostLayer(wl, 1)
    _build(L, wl, 1)
    signs_np = T.rotation_signs(wl, 1)
    cache = {}
    for tok in (0, 7):
        x, ids, w, dnorm_of, sketch_of = _pick(wl, hl, tok, keep, "router_weighted", signs_np,
                                               cache, layer=1)
        kept_ref, y_ref = S.sketch_select_token(x, ids, w, hl.expert, sketch_of, dnorm_of, keep,
                                                signs_np, hl.shared, "router_weighted")
        kept, y = _screen(L, x, keep, 1)
        assert kept.tolist() == kept_ref.tolist(), tok
        err = rel_err(y, y_ref)
        print(f"sketch screen keep {keep} token {tok}: max|dy|/||y||inf = {err:.3e}")
        assert err <= TOL_BF16
    L.close()
    del L
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ stage 3: the reader
def _basis(wl, hl):
    """U from the layer's stacked down columns (every routed channel), by the oracle."""
    return S.recovery_basis((hl.expert(e)[2] for e in range(wl.E)), wl.H)


def _reader(L, x_np, keep, mode):
    import torch
    x = torch.from_numpy(np.asarray(x_np, dtype=np.float32)).cuda().reshape(1, -1)
    y = torch.empty_like(x)
    kept = torch.full((max(keep, 1),), -1, dtype=torch.int32, device="cuda")
    L.channel_select(x, keep, kept, y=y, mode=mode, reader=True)
    assert L.check() == 0
    return kept.cpu().numpy()[:keep], y.cpu().numpy()[0]


@pytest.mark.parametrize("wl", SMALL[:2], ids=lambda w: f"H{w.H}E{w.E}I{w.I}{w.expert_dtype}")
def test_reader_recovery_small(wl):
    import torch
    L = _layer(wl)
    hl = HostLayer(wl)
    _build(L, wl)
    U = _basis(wl, hl)
    L.build_recovery(torch.from_numpy(U.astype(np.float32)).cuda())
    coeffs = {}

    def coeffs_of(e):
        if e not in coeffs:
            coeffs[e] = S.recovery_coeffs(hl.expert(e)[2], U.astype(np.float32))
        return coeffs[e]

    signs_np = T.rotation_signs(wl, 0)
    cache = {}
    n = wl.k * wl.I
    for tok, keep in enumerate([1, n // 8, n // 3 + 1, n]):
        x, ids, w, dnorm_of, sketch_of = _pick(wl, hl, 50 + tok, keep, "router_weighted",
                                               signs_np, cache)
        kept_ref, y_ref = S.reader_token(x, ids, w, hl.expert, sketch_of, dnorm_of, keep,
                                         signs_np, U.astype(np.float32), coeffs_of, hl.shared,
                                         "router_weighted")
        kept, y = _reader(L, x, keep, 1)
        assert kept.tolist() == kept_ref.tolist(), (tok, keep)
        assert rel_err(y, y_ref) <= TOL_BF16, (tok, keep, rel_err(y, y_ref))


def test_reader_recovery_full_size():
    """The stack's shapes: U of the layer's 196,608 down columns, keep 799."""
    import torch
    wl = WORKLOADS["qwen35_a3b_sparse"]
    L = _layer(wl, 4)
    hl = HostLayer(wl, 4)
    _build(L, wl, 4)
    U = _basis(wl, hl).astype(np.float32)
    L.build_recovery(torch.from_numpy(U).cuda())
    signs_np = T.rotation_signs(wl, 4)
    cache, coeffs = {}, {}

    def coeffs_of(e):
        if e not in coeffs:
            coeffs[e] = S.recovery_coeffs(hl.expert(e)[2], U)
        return coeffs[e]

    x, ids, w, dnorm_of, sketch_of = _pick(wl, hl, 3, 799, "router_weighted", signs_np, cache,
                                           layer=4)
    kept_ref, y_ref = S.reader_token(x, ids, w, hl.expert, sketch_of, dnorm_of, 799, signs_np,
                                     U, coeffs_of, hl.shared, "router_weighted")
    kept, y = _reader(L, x, 799, 1)
    assert kept.tolist() == kept_ref.tolist()
    err = rel_err(y, y_ref)
    print(f"reader keep 799: max|dy|/||y||inf = {err:.3e}")
    assert err <= TOL_BF16
    L.close()
    del L
    torch.cuda.empty_cache()
