"""Property test (hypothesis) of the HIP path against the oracle over random small shapes:
batch-1 layer (with the launch's own routing read back), batched layer, and the channel-sparse
layer at a random keep count.  Shapes respect the descriptor rules (H a multiple of 32, I and
I_s multiples of 8); every draw is margin-checked so that the oracle's routing and keep set are
unique."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from gpu_common import (CH_MARGIN_REL, MARGIN, TOL_BF16, HostLayer, cuda_ok, pick_attempt,
                        rel_err)
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]

SETTINGS = settings(max_examples=24, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow,
                                           HealthCheck.function_scoped_fixture])


@st.composite
def shapes(draw):
    E = draw(st.integers(1, 48))
    k = draw(st.integers(1, min(E, 8)))
    ns = draw(st.integers(0, 2))
    return dict(H=32 * draw(st.integers(1, 24)), E=E, k=k, I=8 * draw(st.integers(1, 16)),
                ns=ns, Is=8 * draw(st.integers(1, 8)) if ns else 0,
                f32=draw(st.booleans()), B=draw(st.integers(2, 6)),
                keep_frac=draw(st.floats(0.0, 1.0)), wid=draw(st.integers(200, 239)))


def _workload(p):
    base = WORKLOADS["tiny_f32" if p["f32"] else "qwen35_a3b_bf16"]
    kw = dict(wid=p["wid"], H=p["H"], E=p["E"], k=p["k"], I=p["I"], n_shared=p["ns"],
              I_shared=p["Is"], layers=1)
    if p["f32"]:
        kw["shared_dtype"] = "f32"
    return T.reduced(base, **kw)


@SETTINGS
@given(shapes())
def test_random_shapes_match_oracle(p):
    import torch
    import routed_expert_ffn_route_amd as M
    wl = _workload(p)
    print(f"case {p}", flush=True)
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=p["B"])
    L = M.Layer(desc, T.device_layer(wl, 0))
    hl = HostLayer(wl)
    try:
        xs = np.stack([np.asarray(pick_attempt(wl, b, host_router=hl.router)[1],
                                  dtype=np.float32).reshape(-1) for b in range(p["B"])])
        refs = [O.moe_layer_token(x, hl.router, hl.expert, wl.k, hl.shared) for x in xs]
        # batch 1: y and the launch's own routing
        xd = torch.from_numpy(xs[:1].copy()).cuda()
        yd = torch.empty_like(xd)
        L.forward(xd, yd, B=1)
        assert L.check() == 0
        assert rel_err(yd.cpu().numpy()[0], refs[0][0]) <= TOL_BF16
        ids = torch.empty((1, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, wl.k), dtype=torch.float32, device="cuda")
        L.routing(ids, w, B=1)
        assert ids.cpu().numpy()[0].tolist() == refs[0][1].tolist()
        assert np.max(np.abs(w.cpu().numpy()[0] - refs[0][2])) <= 1e-6
        # the batch (the batched layer takes bf16 experts; fp32 ones are refused as documented,
        # except at B = 2, which runs token by token on the batch-1 kernel)
        xb = torch.from_numpy(xs).cuda()
        yb = torch.empty_like(xb)
        if p["f32"] and p["B"] > 2:
            with pytest.raises(M.MoeError) as ei:
                L.forward(xb, yb, B=p["B"])
            assert ei.value.status == M.MOE_ERR_UNSUPPORTED
        else:
            L.forward(xb, yb, B=p["B"])
            assert L.check() == 0
            yb = yb.cpu().numpy()
            for b in range(p["B"]):
                assert rel_err(yb[b], refs[b][0]) <= TOL_BF16, b
            if p["B"] <= 2:  # token by token: each launch's own routing, in its row
                idb = torch.empty((p["B"], wl.k), dtype=torch.int32, device="cuda")
                wb = torch.empty((p["B"], wl.k), dtype=torch.float32, device="cuda")
                L.routing(idb, wb, B=p["B"])
                for b in range(p["B"]):
                    assert idb.cpu().numpy()[b].tolist() == refs[b][1].tolist(), b
                    assert np.max(np.abs(wb.cpu().numpy()[b] - refs[b][2])) <= 1e-6, b
        # channel-sparse layer at a random keep count (token 0, when its K-th score is unique)
        n = wl.k * wl.I
        keep = int(round(p["keep_frac"] * n))
        x0 = xs[0].astype(np.float64)
        ids0, w0 = refs[0][1], refs[0][2]
        dn = {int(e): O.down_norms(hl.expert(int(e))[2]) for e in ids0}
        s, _ = O.channel_scores(x0, ids0, w0, hl.expert, dn.__getitem__)
        srt = np.sort(s.ravel())[::-1]
        if 0 < keep < n and srt[keep - 1] - srt[keep] < CH_MARGIN_REL * srt[0]:
            return
        kept_ref, y_ref = O.channel_select_token(x0, ids0, w0, hl.expert, dn.__getitem__,
                                                 keep, hl.shared)
        kept = torch.full((max(keep, 1),), -1, dtype=torch.int32, device="cuda")
        y = torch.empty_like(xd)
        L.channel_select(xd, keep, kept, y=y)
        assert L.check() == 0
        assert kept.cpu().numpy()[:keep].tolist() == kept_ref.tolist()
        y = y.cpu().numpy()[0]
        if np.max(np.abs(y_ref)) == 0.0:  # nothing kept and no shared experts
            assert not np.any(y)
        else:
            assert rel_err(y, y_ref) <= TOL_BF16
    finally:
        L.close()
