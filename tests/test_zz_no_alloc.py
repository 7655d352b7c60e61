"""GPU check of moe_ffn_forward_noalloc (the layer on the library's static scratch) against
moe_ffn_forward (a handle with its own workspace) through the C ABI: the same kernels, so
the outputs must be bit-identical, and within the oracle's tolerance.  Two calls in a row,
the second with a smaller input (fewer tokens, a smaller layer), then the first again."""
import numpy as np
import pytest

from gpu_common import HostLayer, TOL_BF16, cuda_ok, pick_attempt, rel_err
from synth import tensors as T
from synth.workloads import WORKLOADS
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]

BIG = T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=171, H=2048, E=64, k=8, I=256, n_shared=1,
                I_shared=256, layers=1)
SMALL = T.reduced(WORKLOADS["qwen35_a3b_bf16"], wid=172, H=1024, E=32, k=4, I=128,
                  n_shared=1, I_shared=64, layers=1)


def _case(wl, B):
    import torch
    import routed_expert_ffn_route_amd as M
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared,
                       router_dtype=wl.router_dtype, expert_dtype=wl.expert_dtype,
                       shared_dtype=wl.shared_dtype, max_batch=B)
    tensors = T.device_layer(wl, 0)
    hl = HostLayer(wl)
    xs = [pick_attempt(wl, b, host_router=hl.router)[1] for b in range(B)]
    x = torch.from_numpy(np.stack(xs).astype(np.float32)).cuda()
    return M, desc, tensors, hl, x


@pytest.mark.parametrize("order", ["big_then_small", "small_then_big"])
def test_noalloc_matches_handle_path(order):
    import torch
    cases = [(BIG, 3), (SMALL, 1), (BIG, 3)] if order == "big_then_small" else \
            [(SMALL, 2), (BIG, 1), (SMALL, 1)]
    for wl, B in cases:
        M, desc, tensors, hl, x = _case(wl, B)
        y_ref = torch.empty((B, wl.H), dtype=torch.float32, device="cuda")
        L = M.Layer(desc, tensors)
        L.forward(x, y_ref)
        assert L.check() == 0
        y = torch.full((B, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        M.forward_noalloc(desc, tensors, x, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), (wl.wid, B)
        xc = x.cpu().numpy()
        for b in range(B):
            y_o, _, _ = O.moe_layer_token(xc[b], hl.router, hl.expert, wl.k, hl.shared)
            assert rel_err(y[b].cpu().numpy(), y_o) <= TOL_BF16
        L.close()


def test_noalloc_rejects_oversized_layer():
    import routed_expert_ffn_route_amd as M
    import torch
    wl = WORKLOADS["qwen35_a3b_bf16"]
    desc = M.make_desc(wl.H, wl.E, wl.k, wl.I, wl.n_shared, wl.I_shared, max_batch=4096)
    x = torch.zeros((1, wl.H), dtype=torch.float32, device="cuda")
    y = torch.zeros_like(x)
    fake = {n: x for n in ("router", "gate", "up", "down_t", "sh_gate", "sh_up", "sh_down_t")}
    with pytest.raises(M.MoeError) as ei:
        M.forward_noalloc(desc, fake, x, y)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
