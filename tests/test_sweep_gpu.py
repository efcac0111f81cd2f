"""Random shapes through every forward path against the oracle: 40 seeded
configurations (token counts, ranks, experts per rank, top-k, hidden sizes,
BF16 or FP8, empty / bad / repeated slots) each run through the two-call and
fused per-expert paths, the deduplicated paths (two calls and fused) and,
where a source rank has at most 256 tokens, the low-latency path. Every
integer, index and byte output bit-exact; combines bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import to_bf16_bits
from test_dedup_gpu import check_dedup, dedup_cap
from test_ll_gpu import check_ll
from test_parity_gpu import full_check, oracle_cap

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
    epr = int(rng.integers(1, 17))
    E = min(R * epr, 1024 // R * R)
    k = int(rng.integers(1, min(32, E) + 1))
    tpr = int(rng.integers(1, 3000 // R + 2))
    T = R * tpr
    fp8 = bool(rng.integers(0, 2))
    H = int(rng.integers(1, 17)) * 128 if fp8 else int(rng.integers(1, 257)) * 8
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    topk[rng.random((T, k)) < rng.choice([0.0, 0.1, 0.5])] = -1
    if rng.random() < 0.3:
        topk[rng.random((T, k)) < 0.02] = E + 5        # bad ids
    if k > 1 and rng.random() < 0.3:
        rows = rng.random(T) < 0.05
        topk[rows, k - 1] = topk[rows, 0]              # repeats
    w = rng.random((T, k)).astype(np.float32)
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    return dict(T=T, k=k, E=E, R=R, H=H, fp8=fp8, topk=topk, w=w, x=x)


@pytest.mark.parametrize("seed", list(range(40)))
def test_random_shapes_every_path(seed):
    c = random_case(seed)
    T, k, E, R, H, fp8 = c["T"], c["k"], c["E"], c["R"], c["H"], c["fp8"]
    print(f"case {seed}: T={T} k={k} E={E} R={R} H={H} fp8={fp8}", flush=True)
    cap = oracle_cap(c["topk"], E, R)
    for fused in (False, True):
        full_check(c["x"], c["topk"], c["w"], E, R, cap, fp8, fused=fused)
    dcap = dedup_cap(c["topk"], E, R)
    for fused in (False, True):
        check_dedup(c["x"], c["topk"], c["w"], E, R, dcap, fp8, fused=fused)
    if T // R <= 256 and E * T * H <= (1 << 31):
        check_ll(c["x"], c["topk"], c["w"], E, R, fp8)
