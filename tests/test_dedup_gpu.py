"""Parity of the rank-deduplicated exchange (the DeepEP guide's normal
kernels send a token once per destination rank) with the oracle, through the
C ABI: the layout's leader ranks and per-rank token counts, the handle, the
received rows (bf16 copies or e4m3 codes + scales), each row's routing
entries, and the combine of pre-reduced rows. Integer, index and byte outputs
bit-exact; the bf16 combine bit-exact (same fp32 FMA order as the oracle)."""
import gc
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import CONFIGS, device_normal_bf16, make_workload, normal_bf16, to_bf16_bits
from gpu_helpers import LAYOUT_KEYS, compare_bf16, dev, dev_bf16, host, host_u16, used_rows

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback


def dedup_cap(topk, E, R):
    """The most deduplicated rows any rank needs (no capacity drops)."""
    _, rows, _ = oracle.default().layout_dedup(topk, E, R, 1 << 30)
    return int(rows.max()) if rows.size else 0


def gpu_dedup(x, topk, w, E, R, cap, fp8, fused=False):
    """Layout + deduplicated dispatch: two calls, or the fused one."""
    T, k = topk.shape
    H = x.shape[1]
    buf = ep.Buffer(T, H, k, E, R, cap)
    topk_d = dev(topk.astype(np.int32))
    w_d = None if w is None else dev(w.astype(np.float32))
    if fused:
        L, rx, rs, rti, rtw, h = buf.dispatch_dedup_with_layout(dev_bf16(x), topk_d, w_d, fp8)
    else:
        L = buf.get_dispatch_layout(topk_d, buf.new_layout(dedup=True))
        rx, rs, rti, rtw, h = buf.dispatch_dedup(dev_bf16(x), topk_d, w_d, L, fp8)
    st = buf.status()
    return buf, L, rx, rs, rti, rtw, h, st


def check_dedup(x, topk, w, E, R, cap, fp8, combine_seed=7, fused=False):
    """Layout, handle, rows, routing entries and combine, every element."""
    orc = oracle.default()
    T, k = topk.shape
    Lo = orc.layout(topk, E, R, cap)
    rir_o, trows_o, st_o = orc.layout_dedup(topk, E, R, cap)
    pos_o, src_o = orc.positions_dedup(topk, rir_o, E, R, cap)
    n = R * cap
    rx_o, rs_o, rti_o, rtw_o = orc.dispatch_dedup(x, topk, w, pos_o, E, R, n, fp8)

    buf, L, rx, rs, rti, rtw, h, st = gpu_dedup(x, topk, w, E, R, cap, fp8, fused)
    assert st == st_o, (st, st_o)
    for key in LAYOUT_KEYS:  # the per-expert layout is unchanged
        assert np.array_equal(host(getattr(L, key)), getattr(Lo, key)), key
    rir = host(L.rank_in_rank)
    if not np.array_equal(rir, rir_o):
        bad = np.argwhere(rir != rir_o)
        raise AssertionError(f"rank_in_rank differs at {bad[:5].tolist()}")
    assert np.array_equal(host(L.token_rows), trows_o), "token_rows"
    pos = host(h.pos)
    assert np.array_equal(pos, pos_o), f"pos differs at {np.argwhere(pos != pos_o)[:5].tolist()}"
    rows = used_rows(pos_o)
    src = host(h.src_idx)
    assert np.array_equal(src[rows], src_o[rows]), "src_idx differs on kept rows"
    if rows.size:
        idx = torch.from_numpy(rows.astype(np.int64)).cuda()
        if fp8:
            assert np.array_equal(rx.index_select(0, idx).cpu().numpy(), rx_o[rows]), "fp8 rows"
            gs = rs.index_select(0, idx).cpu().numpy()
            assert np.array_equal(gs.view(np.uint32), rs_o[rows].view(np.uint32)), "scales"
        else:
            assert np.array_equal(host_u16(rx.index_select(0, idx)), rx_o[rows]), "bf16 rows"
        assert np.array_equal(host(rti.index_select(0, idx)), rti_o[rows]), "recv_topk_idx"
        if w is not None:
            got = host(rtw.index_select(0, idx))
            assert np.array_equal(got.view(np.uint32), rtw_o[rows].view(np.uint32)), "recv_topk_w"
    # combine of pre-reduced rows (one per destination rank), unit weights
    if T > 0 and n > 0:
        eo = normal_bf16(np.random.default_rng(combine_seed), (n, x.shape[1]))
        eo_d = dev_bf16(eo)
        y_o, acc_o = orc.combine(eo, pos_o, None, return_acc=True)
        assert compare_bf16(host_u16(buf.combine(eo_d, h, None)), y_o, "combine") == 1.0
        acc = host(buf.combine_f32(eo_d, h, None))
        assert np.array_equal(acc.view(np.uint32), acc_o.view(np.uint32)), "fp32 sums"
    return st_o, pos_o, trows_o


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("name", ["tiny", "decode_rank", "decode", "prefill", "skewed"])
def test_dedup_parity(name, fused):
    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed=0)
    cap = dedup_cap(wl.topk_idx, cfg.E, cfg.R)
    st, pos, trows = check_dedup(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, cfg.use_fp8, fused=fused)
    assert st == 0
    # a token lands once per rank it has experts on: fewer rows than slots
    # whenever some token has two experts on one rank
    assert (pos >= 0).sum() == trows.sum() <= (wl.topk_idx >= 0).sum()


def test_dedup_bf16_and_fp8_same_routing():
    cfg = replace(CONFIGS["decode"], T=512, H=1024)
    wl = make_workload(cfg, seed=3)
    cap = dedup_cap(wl.topk_idx, cfg.E, cfg.R)
    for fp8 in (False, True):
        check_dedup(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, fp8)


def rand_case(T, k, E, R, H, fp8, seed=0, mutate=None, cap=None, cap_delta=0, weights=True, fused=False):
    rng = np.random.default_rng(seed)
    topk = (np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32) if T > 0
            else np.zeros((0, k), np.int32))
    if mutate is not None:
        topk = mutate(topk, rng)
    w = rng.random((T, k)).astype(np.float32) if weights else None
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    if cap is None:
        cap = max(dedup_cap(topk, E, R) + cap_delta, 0)
    return check_dedup(x, topk, w, E, R, cap, fp8, fused=fused)


DEDUP_EDGE = {
    "empty": dict(T=0, k=2, E=16, R=4, H=256, fp8=False),
    "one_token": dict(T=1, k=1, E=1, R=1, H=8, fp8=False),
    "R1_all_slots_one_rank": dict(T=300, k=4, E=32, R=1, H=384, fp8=True),
    "E_equals_R_no_dups": dict(T=640, k=4, E=8, R=8, H=512, fp8=True),
    "k32": dict(T=96, k=32, E=64, R=16, H=256, fp8=False),
    "k3_not_mult4": dict(T=300, k=3, E=12, R=4, H=136, fp8=False),
    "R_not_mult4": dict(T=300, k=2, E=12, R=3, H=256, fp8=False),
    "E1024_R64": dict(T=1024, k=8, E=1024, R=64, H=1024, fp8=True),
    "one_full_tile": dict(T=256, k=8, E=256, R=8, H=1024, fp8=True),
    "tiles_ragged": dict(T=5000, k=6, E=200, R=8, H=384, fp8=False),
    "tiles_33": dict(T=8448, k=8, E=256, R=32, H=256, fp8=True),
    "epr_not_pow2": dict(T=1536, k=8, E=192, R=8, H=256, fp8=True),
    "many_tiles": dict(T=65536, k=2, E=32, R=8, H=8, fp8=False),
    "ticket_tiles": dict(T=270336, k=1, E=16, R=8, H=8, fp8=False),
    "no_weights": dict(T=512, k=8, E=64, R=8, H=256, fp8=True, weights=False),
}


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("name", list(DEDUP_EDGE))
def test_dedup_edges(name, fused):
    rand_case(**DEDUP_EDGE[name], fused=fused)


def test_dedup_bad_repeated_and_empty_slots():
    def m(t, r):
        t = t.copy()
        t[r.random(t.shape) < 0.2] = -1  # empty slots
        t[3, 1] = 99            # out of range
        t[4, 0] = -7            # out of range: the rank's leader moves to the next slot
        t[5, 2] = t[5, 0] = 1   # repeat
        t[6, :] = 2             # all repeats: one row
        return t
    for fused in (False, True):
        st, *_ = rand_case(T=640, k=8, E=64, R=8, H=256, fp8=True, mutate=m, fused=fused)
        assert st == ep.EP_ST_BAD_EXPERT | ep.EP_ST_DUP_EXPERT


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("T", [1024, 200])  # several tiles; one tile
def test_dedup_capacity_drops_rows(T, fused):
    st, pos, trows = rand_case(T=T, k=8, E=64, R=8, H=512, fp8=True, cap_delta=-5, fused=fused)
    assert st == ep.EP_ST_CAPACITY and 0 < (pos >= 0).sum() < trows.sum()


def test_dedup_capacity_below_per_expert_rows():
    """A receive capacity that holds every rank's deduplicated rows but not its
    per-expert rows: nothing is dropped and no capacity bit is raised."""
    rng = np.random.default_rng(4)
    T, k, E, R = 512, 8, 32, 4
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    cap = dedup_cap(topk, E, R)
    per_expert = int(oracle.default().layout(topk, E, R, 1 << 30).rank_rows.max())
    assert per_expert > cap
    st, pos, _ = check_dedup(to_bf16_bits(rng.standard_normal((T, 256)).astype(np.float32)), topk,
                             rng.random((T, k)).astype(np.float32), E, R, cap, False)
    assert st == 0 and (pos >= 0).any()


def test_dedup_capacity_zero():
    st, pos, _ = rand_case(T=64, k=2, E=16, R=4, H=256, fp8=False, cap=0)
    assert st == ep.EP_ST_CAPACITY and np.all(pos < 0)


def test_dedup_full_size_sampled():
    """The prefill shape in the launch configuration the bench times: layout
    and handle compared whole, rows and routing entries on sampled tokens."""
    cfg = CONFIGS["prefill"]
    wl = make_workload(cfg, seed=0)
    orc = oracle.default()
    cap = dedup_cap(wl.topk_idx, cfg.E, cfg.R)
    rir_o, trows_o, st_o = orc.layout_dedup(wl.topk_idx, cfg.E, cfg.R, cap)
    pos_o, src_o = orc.positions_dedup(wl.topk_idx, rir_o, cfg.E, cfg.R, cap)
    buf, L, rx, rs, rti, rtw, h, st = gpu_dedup(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, True)
    assert st == st_o == 0
    assert np.array_equal(host(L.rank_in_rank), rir_o) and np.array_equal(host(L.token_rows), trows_o)
    assert np.array_equal(host(h.pos), pos_o)
    rng = np.random.default_rng(0)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 256, replace=False)])).astype(np.int32)
    rx_o, rs_o, rti_o, rtw_o = orc.dispatch_dedup(wl.x, wl.topk_idx, wl.topk_w, pos_o, cfg.E, cfg.R,
                                                  cfg.R * cap, True, tokens=toks)
    rows = used_rows(pos_o[toks])
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    assert np.array_equal(rx.index_select(0, idx).cpu().numpy(), rx_o[rows])
    assert np.array_equal(rs.index_select(0, idx).cpu().numpy().view(np.uint32), rs_o[rows].view(np.uint32))
    assert np.array_equal(host(rti.index_select(0, idx)), rti_o[rows])
    assert np.array_equal(host(rtw.index_select(0, idx)).view(np.uint32), rtw_o[rows].view(np.uint32))
    assert np.array_equal(host(h.src_idx)[rows], src_o[rows])


def test_dedup_layout_rejected_by_fused_call():
    cfg = CONFIGS["tiny"]
    wl = make_workload(cfg, seed=0)
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, 64)
    with pytest.raises(ep.EpError) as e:
        buf.dispatch_with_layout(dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w), False,
                                 layout=buf.new_layout(dedup=True))
    assert e.value.code == ep.EP_ERR_ARG


def test_dedup_and_per_expert_interleaved():
    """Dedup and per-expert layouts alternate on one context (shared look-back
    workspace and epochs)."""
    cfg = replace(CONFIGS["decode"], T=2048, H=512)
    for seed in range(3):
        wl = make_workload(cfg, seed=seed)
        cap = int(oracle.default().layout(wl.topk_idx, cfg.E, cfg.R, 1 << 30).rank_rows.max())
        buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cap)
        topk = dev(wl.topk_idx)
        for _ in range(2):
            Ld = buf.get_dispatch_layout(topk, buf.new_layout(dedup=True))
            Lp = buf.get_dispatch_layout(topk)
            rir_o, trows_o, _ = oracle.default().layout_dedup(wl.topk_idx, cfg.E, cfg.R, cap)
            Lo = oracle.default().layout(wl.topk_idx, cfg.E, cfg.R, cap)
            assert np.array_equal(host(Ld.rank_in_rank), rir_o)
            assert np.array_equal(host(Ld.token_rows), trows_o)
            for key in LAYOUT_KEYS:
                assert np.array_equal(host(getattr(Lp, key)), getattr(Lo, key)), key
        assert buf.status() == 0


@pytest.mark.parametrize("name", ["decode_rank", "decode"])  # one tile (replicas); four tiles
def test_dedup_fused_graph_replay_and_interleaving(name):
    """The fused deduplicated call captured in a HIP graph with a combine,
    replayed with per-expert fused calls and layouts in between on the same
    context (shared flags and epochs): every replay equals the eager result."""
    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed=2)
    cap = int(oracle.default().layout(wl.topk_idx, cfg.E, cfg.R, 1 << 30).rank_rows.max())
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cap)
    x, topk, w = dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w)
    L = buf.new_layout(dedup=True)
    out = buf.dispatch_dedup_with_layout(x, topk, w, True, layout=L)[1:]
    out[2].fill_(-3)  # rows no token uses keep this
    buf.dispatch_dedup_with_layout(x, topk, w, True, layout=L, out=out)
    eo = device_normal_bf16((buf.num_rows, cfg.H), seed=6)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    buf.combine(eo, out[4], None, out=y)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (L.rank_in_rank, L.token_rows, out[4].pos, out[2], y)]
    gc.collect()  # no buffer of an earlier test may be released during the capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            buf.dispatch_dedup_with_layout(x, topk, w, True, layout=L, out=out)
            buf.combine(eo, out[4], None, out=y)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(4):
        for t in (L.rank_in_rank, out[4].pos, out[2], y):
            t.fill_(-3) if t.dtype == torch.int32 else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [L.rank_in_rank, L.token_rows, out[4].pos, out[2], y]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {i}"
        # per-expert work on the same context between replays
        buf.dispatch_with_layout(x, topk, w, True)
        buf.get_dispatch_layout(topk)
    assert buf.status() == 0
