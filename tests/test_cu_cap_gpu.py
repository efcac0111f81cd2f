"""The compute-unit cap: kernels on a stream from ep_stream_create_cus run
only on the units its mask enables (checked with the census kernel), the
complementary stream's units are disjoint from them, and the exchange gives
bit-identical results on a capped stream (checked against the oracle)."""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import CONFIGS, make_workload, normal_bf16
from gpu_helpers import compare_handle, compare_layout, compare_rows, dev_bf16, gpu_forward, host, host_u16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback


def census_on(stream=None, blocks=8192):
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        ids = ep.cu_census(blocks)
    torch.cuda.synchronize()
    u = host(ids).astype(np.int64)
    return set(u.tolist()), set((u >> 16).tolist())


def test_census_default_stream_uses_every_xcd():
    units, xcds = census_on()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert xcds == set(range(8))
    assert len(units) >= cus * 3 // 4, len(units)


@pytest.mark.parametrize("num_cus", [16, 64])
def test_capped_stream_runs_on_its_units_only(num_cus):
    with ep.CuStream(num_cus) as cs, ep.CuStream(num_cus, exclude=True) as rest:
        units, xcds = census_on(cs.torch_stream)
        others, oxcds = census_on(rest.torch_stream)
    assert len(units) <= num_cus, (len(units), num_cus)
    assert len(units) >= num_cus // 2
    assert xcds == set(range(8)) == oxcds
    per_xcd = np.bincount(np.array(sorted(units)) >> 16, minlength=8)
    assert per_xcd.max() <= num_cus // 8, per_xcd
    assert not (units & others), "a unit runs work from both the capped and the complementary stream"


@pytest.mark.parametrize("name,fused", [("tiny", False), ("decode_rank", True), ("decode", True),
                                        ("prefill", True), ("prefill", False)])
def test_exchange_on_capped_stream_matches_oracle(name, fused):
    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed=0)
    orc = oracle.default()
    cap = int(orc.layout(wl.topk_idx, cfg.E, cfg.R, 1 << 30).rank_rows.max())
    L, pos, src, rx, rs, rw = orc.forward(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, cfg.use_fp8)
    eo = normal_bf16(np.random.default_rng(3), (cfg.R * cap, cfg.H))
    with ep.CuStream(32) as cs:
        with torch.cuda.stream(cs.torch_stream):
            g = gpu_forward(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, cfg.use_fp8, fused=fused)
            y = g.buf.combine(dev_bf16(eo), g.handle, g.w)
        cs.torch_stream.synchronize()
    assert g.status == L.status == 0
    compare_layout(g, L)
    compare_handle(g, pos, src)
    compare_rows(g, pos, rx, rs, rw, cfg.use_fp8)
    assert np.array_equal(host_u16(y), orc.combine(eo, pos, wl.topk_w))
