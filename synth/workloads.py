"""The five synthetic workloads and the stream-id scheme that names each tensor.

Shapes follow the pages' models: a tiny fp32 layer; a 40-layer bf16 stack shaped like
Qwen3.5-35B-A3B (256 experts, 8 routed, one shared expert; the model catalogue on
"Mixture of Experts Changes the Arithmetic", section "Two Numbers Instead of One");
its channel-sparse variant keeping a fixed count of channels per token (the top-k keep
rule of the arXiv:2610.37386 review, section "Background: channels and keep rules");
the 64-expert, top-3, 8192x8192-per-expert batch sweep of the "501B of which 23B"
post, section 3[B]; and a large-expert-count MXFP4 layer shaped like the Kimi K3 row of
the same model catalogue (896 experts, 16 routed, two shared).

Every tensor is a stream of the counter-based generator; its stream id packs
(workload, tensor kind, layer, sub-index) so that any element can be regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

KIND = {
    "router": 1, "gate": 2, "up": 3, "down_t": 4,
    "sh_gate": 5, "sh_up": 6, "sh_down_t": 7,
    "x": 8, "logits": 9, "linear": 10, "signs": 11,
}


def stream_id(wid: int, kind: str, layer: int = 0, sub: int = 0) -> int:
    assert 0 <= wid < 256 and 0 <= layer < 65536 and 0 <= sub < 2**32
    return (wid << 56) | (KIND[kind] << 48) | (layer << 32) | sub


def x_sub(token: int, attempt: int = 0, case: int = 0) -> int:
    """Sub-index of the activation vector of one token (attempt = margin redraw count,
    case = an independent draw of the whole batch)."""
    assert 0 <= attempt < 64 and 0 <= token < 2**20 and 0 <= case < 64
    return (case << 26) | (token << 6) | attempt


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    kind: str                 # "swiglu" (G, V, D per expert) or "linear" (one matrix)
    H: int
    E: int
    k: int
    I: int                    # channels per expert (linear: output width)
    n_shared: int
    I_shared: int
    layers: int
    router_dtype: str | None  # None: routed from supplied logits
    expert_dtype: str         # "f32" | "bf16" | "mxfp4"
    shared_dtype: str | None
    tokens: int
    batches: tuple
    sigma_router: float
    sigma_gate: float
    sigma_up: float
    sigma_down: float
    sigma_x: float = 1.0
    sigma_logits: float = 1.0
    seed: int = 0
    weights_wid: int = -1     # workload whose weight streams this one reuses (-1: itself)
    keep_fracs: tuple = field(default_factory=tuple)

    @property
    def wwid(self) -> int:
        return self.wid if self.weights_wid < 0 else self.weights_wid

    def keep_counts(self) -> tuple:
        # Fixed keep count per token: nearest integer of f * k * I (half rounds up).
        return tuple(int(math.floor(f * self.k * self.I + 0.5)) for f in self.keep_fracs)


WORKLOADS = {
    "tiny_f32": Workload(
        wid=1, name="tiny_f32", kind="swiglu", H=512, E=16, k=2, I=256, n_shared=0,
        I_shared=0, layers=1, router_dtype="f32", expert_dtype="f32", shared_dtype=None,
        tokens=64, batches=(1,), sigma_router=1 / math.sqrt(512),
        sigma_gate=1 / math.sqrt(512), sigma_up=1 / math.sqrt(512),
        sigma_down=1 / math.sqrt(256)),
    "qwen35_a3b_bf16": Workload(
        wid=2, name="qwen35_a3b_bf16", kind="swiglu", H=2048, E=256, k=8, I=768,
        n_shared=1, I_shared=768, layers=40, router_dtype="bf16", expert_dtype="bf16",
        shared_dtype="bf16", tokens=256, batches=(1,), sigma_router=0.02,
        sigma_gate=0.02, sigma_up=0.02, sigma_down=0.02),
    "qwen35_a3b_sparse": Workload(
        wid=3, name="qwen35_a3b_sparse", kind="swiglu", H=2048, E=256, k=8, I=768,
        n_shared=1, I_shared=768, layers=40, router_dtype="bf16", expert_dtype="bf16",
        shared_dtype="bf16", tokens=256, batches=(1,), sigma_router=0.02,
        sigma_gate=0.02, sigma_up=0.02, sigma_down=0.02, weights_wid=2,
        keep_fracs=(0.13, 0.18)),
    "linear_e64_k3": Workload(
        wid=4, name="linear_e64_k3", kind="linear", H=8192, E=64, k=3, I=8192,
        n_shared=0, I_shared=0, layers=1, router_dtype=None, expert_dtype="bf16",
        shared_dtype=None, tokens=2048, batches=(1, 4, 16, 64, 256, 2048),
        sigma_router=0.0, sigma_gate=1 / math.sqrt(8192), sigma_up=0.0, sigma_down=0.0),
    "mxfp4_e896_k16": Workload(
        wid=5, name="mxfp4_e896_k16", kind="swiglu", H=7168, E=896, k=16, I=2048,
        n_shared=2, I_shared=2048, layers=8, router_dtype="bf16", expert_dtype="mxfp4",
        shared_dtype="bf16", tokens=128, batches=(1, 16), sigma_router=0.02,
        sigma_gate=0.02, sigma_up=0.02, sigma_down=0.02),
}
