"""Parity of the low-latency dispatch (one launch, fixed per-(expert, source)
regions) with the oracle, through the C ABI: positions, source indices,
region counts and status bit-exact; rows, FP8 codes, scales and weights
bit-exact on every used row; the combine on its handle bit-exact; HIP-graph
replays equal to eager launches."""
import gc

import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import CONFIGS, device_normal_bf16, make_workload, to_bf16_bits
from gpu_helpers import compare_bf16, dev, dev_bf16, host, host_u16, used_rows

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback


def gpu_ll(x, topk, w, E, R, fp8):
    T, k = topk.shape
    H = x.shape[1]
    buf = ep.Buffer(T, H, k, E, R, ep.ll_cap_rows(T, E, R))
    topk_d = dev(topk.astype(np.int32))
    w_d = None if w is None else dev(w.astype(np.float32))
    rx, rs, rw, cnt, h = buf.dispatch_low_latency(dev_bf16(x), topk_d, w_d, fp8)
    st = buf.status()
    return buf, rx, rs, rw, cnt, h, st, w_d


def check_ll(x, topk, w, E, R, fp8, combine_seed=9):
    orc = oracle.default()
    T, k = topk.shape
    H = x.shape[1]
    pos_o, src_o, cnt_o, st_o = orc.ll_positions(topk, E, R)
    buf, rx, rs, rw, cnt, h, st, w_d = gpu_ll(x, topk, w, E, R, fp8)
    assert st == st_o, (st, st_o)
    assert np.array_equal(host(cnt), cnt_o), "recv_count"
    pos = host(h.pos)
    assert np.array_equal(pos, pos_o), f"pos differs at {np.argwhere(pos != pos_o)[:5].tolist()}"
    rows = used_rows(pos_o)
    if rows.size == 0:
        return st_o, pos_o
    assert np.array_equal(host(h.src_idx)[rows], src_o[rows]), "src_idx"
    # the oracle's rows, computed on the used rows only (positions remapped)
    remap = np.full(buf.num_rows, -1, np.int64)
    remap[rows] = np.arange(rows.size)
    pos_c = np.where(pos_o >= 0, remap[np.maximum(pos_o, 0)], -1).astype(np.int32)
    rx_o, rs_o, rw_o = orc.dispatch(x, w, pos_c, rows.size, fp8)
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    if fp8:
        assert np.array_equal(rx.index_select(0, idx).cpu().numpy(), rx_o), "fp8 rows"
        assert np.array_equal(rs.index_select(0, idx).cpu().numpy().view(np.uint32), rs_o.view(np.uint32)), "scales"
    else:
        assert np.array_equal(host_u16(rx.index_select(0, idx)), rx_o), "bf16 rows"
    if w is not None:
        assert np.array_equal(rw.index_select(0, idx).cpu().numpy().view(np.uint32), rw_o.view(np.uint32)), "recv_w"
    # combine on the handle: expert outputs on every row, the oracle on the used ones
    eo = device_normal_bf16((buf.num_rows, H), seed=combine_seed)
    y = host_u16(buf.combine(eo, h, w_d))
    y_o = orc.combine(host_u16(eo.index_select(0, idx)), pos_c, w)
    assert compare_bf16(y, y_o, "combine") == 1.0
    return st_o, pos_o


@pytest.mark.parametrize("name", ["tiny", "decode_rank", "decode"])
def test_ll_parity(name):
    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed=0)
    st, pos = check_ll(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cfg.use_fp8)
    assert st == 0 and (pos >= 0).sum() == (wl.topk_idx >= 0).sum()


def rand_case(T, k, E, R, H, fp8, seed=0, mutate=None, weights=True):
    rng = np.random.default_rng(seed)
    topk = (np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32) if T > 0
            else np.zeros((0, k), np.int32))
    if mutate is not None:
        topk = mutate(topk, rng)
    w = rng.random((T, k)).astype(np.float32) if weights else None
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    return check_ll(x, topk, w, E, R, fp8)


LL_EDGE = {
    "empty": dict(T=0, k=2, E=16, R=4, H=256, fp8=False),
    "one_token": dict(T=1, k=1, E=1, R=1, H=8, fp8=False),
    "k32": dict(T=96, k=32, E=64, R=16, H=256, fp8=False),
    "k3_channel_tail": dict(T=300, k=3, E=12, R=4, H=136, fp8=False),
    "R_not_mult4": dict(T=300, k=2, E=12, R=3, H=256, fp8=True),
    "E1024_R64": dict(T=1024, k=8, E=1024, R=64, H=256, fp8=True),
    "tokens_per_rank_256": dict(T=2048, k=8, E=256, R=8, H=1024, fp8=True),
    "tokens_per_rank_65": dict(T=520, k=8, E=64, R=8, H=512, fp8=True),
    "E_equals_R": dict(T=640, k=4, E=8, R=8, H=512, fp8=True),
    "hidden_16k_bf16": dict(T=64, k=4, E=16, R=4, H=16384, fp8=False),
    "no_weights": dict(T=512, k=8, E=64, R=8, H=256, fp8=True, weights=False),
    # waves of 2 and 7 passes (the kernel's 2- and 8-pass row loads; 1 and 4
    # are the decode shapes above)
    "passes_2": dict(T=512, k=8, E=64, R=8, H=7168, fp8=True),
    "passes_7_bf16": dict(T=2048, k=4, E=32, R=8, H=7168, fp8=False),
    "passes_7_fp8": dict(T=2048, k=8, E=64, R=8, H=7168, fp8=True),
}


@pytest.mark.parametrize("name", list(LL_EDGE))
def test_ll_edges(name):
    rand_case(**LL_EDGE[name])


def test_ll_bad_repeated_and_empty_slots():
    def m(t, r):
        t = t.copy()
        t[r.random(t.shape) < 0.2] = -1
        t[3, 1] = 99
        t[4, 0] = -7
        t[5, 2] = t[5, 0] = 1
        t[6, :] = 2
        t[200, :] = 5  # a later source rank
        return t
    st, _ = rand_case(T=640, k=8, E=64, R=8, H=256, fp8=True, mutate=m)
    assert st == ep.EP_ST_BAD_EXPERT | ep.EP_ST_DUP_EXPERT


def test_ll_hot_expert():
    """Every token of every source routed to one expert: full regions."""
    def m(t, r):
        t = t.copy()
        t[:, 0] = 7
        t[:, 1:] = np.where(t[:, 1:] == 7, -1, t[:, 1:])
        return t
    rand_case(T=1024, k=4, E=32, R=4, H=512, fp8=True, mutate=m)


def test_ll_rejects_other_layouts():
    cfg = CONFIGS["tiny"]
    wl = make_workload(cfg, seed=0)
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, 64)  # not E*T/R
    with pytest.raises(ep.EpError) as e:
        buf.dispatch_low_latency(dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w), False)
    assert e.value.code == ep.EP_ERR_ARG
    T, R, E = 4096, 8, 16  # 512 tokens per rank
    big = ep.Buffer(T, 256, 2, E, R, ep.ll_cap_rows(T, E, R))
    x = torch.zeros((T, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ep.EpError) as e:
        big.dispatch_low_latency(x, torch.zeros((T, 2), dtype=torch.int32, device="cuda"), None, False)
    assert e.value.code == ep.EP_ERR_ARG


@pytest.mark.parametrize("name", ["decode_rank", "decode"])
def test_ll_graph_replay_matches_eager(name):
    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed=1)
    T, E, R = cfg.T, cfg.E, cfg.R
    buf = ep.Buffer(T, cfg.H, cfg.k, E, R, ep.ll_cap_rows(T, E, R))
    x, topk, w = dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w)
    out = buf.dispatch_low_latency(x, topk, w, True)
    eo = device_normal_bf16((buf.num_rows, cfg.H), seed=4)
    y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    buf.combine(eo, out[4], w, out=y)
    torch.cuda.synchronize()
    y_eager = y.clone()
    pos_eager = out[4].pos.clone()
    cnt_eager = out[3].clone()
    gc.collect()  # no buffer of an earlier test may be released during the capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            buf.dispatch_low_latency(x, topk, w, True, out=out)
            buf.combine(eo, out[4], w, out=y)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(4):
        y.zero_()
        out[4].pos.fill_(-5)
        out[3].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(out[4].pos, pos_eager) and torch.equal(out[3], cnt_eager)
    assert buf.status() == 0
