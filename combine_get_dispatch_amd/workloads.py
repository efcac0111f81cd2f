"""Seeded synthetic workloads for the MoE dispatch / combine path.

This module only draws inputs: routing (top-k expert ids and their weights),
activations, expert outputs and gradients. It holds none of the
dispatch/combine arithmetic (no counting, scanning, packing, quantization or
reduction); both the GPU path and the CPU oracle consume the same bytes.

The five workloads restate the shapes the DeepEP pages report on
(blog.hotdry.top DeepEP notes, section 1 "两种内核设计"; czhn.yksolo.com launch
report, normal-kernel and low-latency-kernel setups): hidden 7168, top-8
experts, 4096 tokens per batch with top-4 groups for the normal kernels and
128 tokens per batch for the low-latency ones, FP8 dispatch with BF16 combine;
plus a tiny case, a skewed-routing case and a large case with backward. The
pages measure on these synthetic shapes, not on a dataset, so no dataset is
stood in for. Random numbers come from numpy's PCG64 (one independent
SeedSequence child per array) or, for large perf-only tensors, from torch's
seeded device generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    T: int            # source tokens on the GPU (all simulated source ranks)
    H: int            # hidden size
    E: int            # experts
    R: int            # simulated expert-parallel ranks
    k: int            # experts per token
    use_fp8: bool     # FP8 e4m3 dispatch (else BF16)
    routing: str      # uniform | softmax_topk | group_limited | zipf
    n_groups: int = 8
    topk_groups: int = 4
    zipf_s: float = 1.2
    hot_frac: float = 0.0
    hot_scale: float = 100.0
    backward: bool = False
    desc: str = ""

    @property
    def N(self) -> int:
        return self.T * self.k

    @property
    def G(self) -> int:
        return self.H // 128


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", T=64, H=256, E=16, R=4, k=2, use_fp8=False, routing="uniform",
                   desc="64 tokens, hidden 256, 16 experts on 4 ranks, top-2 uniform, BF16"),
    "decode": Config("decode", T=1024, H=7168, E=256, R=8, k=8, use_fp8=True,
                     routing="softmax_topk",
                     desc="128 tokens per rank x 8 ranks, hidden 7168, 256 experts, "
                          "softmax top-8, FP8 dispatch"),
    "decode_rank": Config("decode_rank", T=128, H=7168, E=256, R=8, k=8, use_fp8=True,
                          routing="softmax_topk",
                          desc="one rank's 128-token decode share, 256 experts on 8 ranks, "
                               "softmax top-8, FP8 dispatch"),
    "prefill": Config("prefill", T=4096, H=7168, E=256, R=32, k=8, use_fp8=True,
                      routing="group_limited", n_groups=8, topk_groups=4,
                      desc="4096 tokens, hidden 7168, 256 experts in 8 groups on 32 ranks, "
                           "group-limited top-4 groups / top-8 experts, FP8 dispatch"),
    "skewed": Config("skewed", T=4096, H=7168, E=256, R=8, k=8, use_fp8=True, routing="zipf",
                     zipf_s=1.2, hot_frac=0.01, hot_scale=100.0,
                     desc="4096 tokens, Zipf(1.2) expert popularity, 1% of rows x100, FP8"),
    "large": Config("large", T=16384, H=7168, E=256, R=32, k=8, use_fp8=False,
                    routing="uniform", backward=True,
                    desc="16384 tokens, 256 experts on 32 ranks, uniform top-8, BF16, "
                         "with backward"),
}


def get_config(name: str, **overrides) -> Config:
    return replace(CONFIGS[name], **overrides) if overrides else CONFIGS[name]


# ---------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------

_STREAMS = ("x", "routing", "weights", "hot", "expert_out", "grad_y", "grad_rows", "perm")


def _rngs(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(_STREAMS, children)}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def _desc_order(scores: np.ndarray) -> np.ndarray:
    """Column order by score descending, ties to the lower index (stable)."""
    return np.argsort(-scores, axis=1, kind="stable")


def _softmax(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.float32)
    m = a.max(axis=1, keepdims=True)
    e = np.exp(a - m, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def make_routing(cfg: Config, rngs) -> tuple:
    """Returns (topk_idx [T,k] int32, topk_w [T,k] float32)."""
    T, E, k = cfg.T, cfg.E, cfg.k
    r = rngs["routing"]
    if T == 0:
        return np.zeros((0, k), np.int32), np.zeros((0, k), np.float32)
    if cfg.routing == "uniform":
        # k distinct experts, uniformly at random, in draw order
        idx = np.argsort(r.random((T, E)), axis=1, kind="stable")[:, :k]
        w = _softmax(rngs["weights"].standard_normal((T, k), dtype=np.float32))
    elif cfg.routing == "softmax_topk":
        # softmax of N(0,1) gate logits over all experts, top-k, renormalized
        p = _softmax(r.standard_normal((T, E), dtype=np.float32))
        idx = _desc_order(p)[:, :k]
        sel = np.take_along_axis(p, idx, axis=1)
        w = (sel / sel.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    elif cfg.routing == "group_limited":
        # sigmoid scores; group score = sum of its top-2 scores; keep the best
        # topk_groups groups; top-k experts inside them; weights normalized
        s = (1.0 / (1.0 + np.exp(-r.standard_normal((T, E), dtype=np.float32)))).astype(np.float32)
        gsz = E // cfg.n_groups
        sg = s.reshape(T, cfg.n_groups, gsz)
        top2 = -np.sort(-sg, axis=2)[:, :, :2]
        gscore = top2.sum(axis=2, dtype=np.float32)
        keep_groups = _desc_order(gscore)[:, :cfg.topk_groups]
        mask = np.zeros((T, cfg.n_groups), bool)
        np.put_along_axis(mask, keep_groups, True, axis=1)
        masked = np.where(np.repeat(mask, gsz, axis=1), s, -np.inf).astype(np.float32)
        idx = _desc_order(masked)[:, :k]
        sel = np.take_along_axis(s, idx, axis=1)
        w = (sel / sel.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    elif cfg.routing == "zipf":
        # Zipf(s) popularity over a seeded random expert permutation; k distinct
        # draws without replacement, as successive sampling (Efraimidis-Spirakis
        # keys log(u)/p, largest first, give the same distribution and order)
        perm = rngs["perm"].permutation(E)
        pr = (np.arange(1, E + 1, dtype=np.float64) ** -cfg.zipf_s)
        pr /= pr.sum()
        p = np.empty(E)
        p[perm] = pr
        u = 1.0 - r.random((T, E))  # (0, 1]
        keys = np.log(u) / p[None, :]
        idx = _desc_order(keys)[:, :k]
        w = _softmax(rngs["weights"].standard_normal((T, k), dtype=np.float32))
    else:
        raise ValueError(cfg.routing)
    return np.ascontiguousarray(idx, dtype=np.int32), np.ascontiguousarray(w, dtype=np.float32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    cfg: Config
    seed: int
    x: np.ndarray          # [T, H] uint16 (bf16 bits)
    topk_idx: np.ndarray   # [T, k] int32
    topk_w: np.ndarray     # [T, k] float32
    hot_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    _rngs: dict = field(default=None, repr=False)

    def expert_out(self, num_rows: int) -> np.ndarray:
        """N(0,1) bf16 rows [num_rows, H] standing in for the experts' outputs."""
        return normal_bf16(self._rngs["expert_out"], (num_rows, self.cfg.H))

    def grad_y(self) -> np.ndarray:
        return normal_bf16(self._rngs["grad_y"], (self.cfg.T, self.cfg.H))

    def grad_rows(self, num_rows: int) -> np.ndarray:
        return normal_bf16(self._rngs["grad_rows"], (num_rows, self.cfg.H))


def make_workload(cfg, seed: int = 0, with_x: bool = True) -> Workload:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rngs = _rngs(seed)
    topk_idx, topk_w = make_routing(cfg, rngs)
    hot = np.zeros(0, np.int64)
    if with_x:
        xf = rngs["x"].standard_normal((cfg.T, cfg.H), dtype=np.float32)
        if cfg.hot_frac > 0 and cfg.T > 0:
            hot = np.sort(rngs["hot"].permutation(cfg.T)[: int(cfg.T * cfg.hot_frac)])
            xf[hot] *= np.float32(cfg.hot_scale)
        x = to_bf16_bits(xf)
        del xf
    else:
        x = np.zeros((0, cfg.H), np.uint16)
    return Workload(cfg=cfg, seed=seed, x=x, topk_idx=topk_idx, topk_w=topk_w,
                    hot_rows=hot, _rngs=rngs)


def device_normal_bf16(shape, seed: int, device="cuda"):
    """Large N(0,1) bf16 tensor drawn on the device (perf-only inputs)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
