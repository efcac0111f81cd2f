"""The seeded input generators: shapes, determinism and routing structure."""
from dataclasses import replace

import numpy as np
import pytest

from combine_get_dispatch_amd.workloads import CONFIGS, make_workload


def test_config_table():
    want = {"tiny": (64, 256, 16, 4, 2, False), "decode": (1024, 7168, 256, 8, 8, True),
            "decode_rank": (128, 7168, 256, 8, 8, True), "prefill": (4096, 7168, 256, 32, 8, True),
            "skewed": (4096, 7168, 256, 8, 8, True), "large": (16384, 7168, 256, 32, 8, False)}
    for n, v in want.items():
        c = CONFIGS[n]
        assert (c.T, c.H, c.E, c.R, c.k, c.use_fp8) == v
        assert c.T % c.R == 0 and c.E % c.R == 0 and c.H % 128 == 0


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "large"])
def test_routing_structure(name):
    cfg = CONFIGS[name]
    if cfg.T > 4096:
        cfg = replace(cfg, T=4096)
    wl = make_workload(cfg, seed=0, with_x=False)
    idx, w = wl.topk_idx, wl.topk_w
    assert idx.shape == (cfg.T, cfg.k) and idx.dtype == np.int32 and w.dtype == np.float32
    assert idx.min() >= 0 and idx.max() < cfg.E
    assert all(len(set(r)) == cfg.k for r in idx.tolist()), "experts must be distinct per token"
    assert np.all(w > 0) and np.allclose(w.sum(1), 1.0, atol=1e-5)
    again = make_workload(cfg, seed=0, with_x=False)
    assert np.array_equal(again.topk_idx, idx) and np.array_equal(again.topk_w, w)
    other = make_workload(cfg, seed=1, with_x=False)
    assert not np.array_equal(other.topk_idx, idx)
    if cfg.routing == "group_limited":
        groups = idx // (cfg.E // cfg.n_groups)
        assert max(len(set(r)) for r in groups.tolist()) <= cfg.topk_groups
    if cfg.routing == "zipf":
        cnt = np.bincount(idx.reshape(-1), minlength=cfg.E)
        assert cnt.max() > 10 * cnt.mean() / 2, "zipf routing should be heavily skewed"
    if cfg.routing in ("softmax_topk", "group_limited"):
        assert np.all(np.diff(w, axis=1) <= 1e-7), "gated slots come in descending score order"


def test_activations_and_hot_rows():
    cfg = replace(CONFIGS["skewed"], T=800, H=256)
    wl = make_workload(cfg, seed=0)
    assert wl.x.shape == (800, 256) and wl.x.dtype == np.uint16
    assert wl.hot_rows.size == 8
    xf = (wl.x.astype(np.uint32) << 16).view(np.float32)
    rms = np.sqrt((xf.astype(np.float64) ** 2).mean(1))
    assert np.all(rms[wl.hot_rows] > 30) and np.median(rms) < 2
    assert np.array_equal(make_workload(cfg, seed=0).x, wl.x)


def test_empty_workload():
    wl = make_workload(replace(CONFIGS["tiny"], T=0), seed=0)
    assert wl.x.shape == (0, 256) and wl.topk_idx.shape == (0, 2)
