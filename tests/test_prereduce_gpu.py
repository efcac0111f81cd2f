"""Parity of the expert-side pre-reduction of rank-deduplicated rows
(ep_prereduce: each received row's local expert outputs weighted and summed
before combine) with the oracle, through the C ABI; and the whole
deduplicated chain (layout and dispatch, pre-reduction, combine of the
reduced rows with unit weights). The reduced bf16 rows and their fp32 sums
are bit-exact on every used row and unused rows stay untouched; on values
exact in bf16 and fp32 the chain equals the per-expert weighted combine."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import CONFIGS, device_normal_bf16, make_workload, to_bf16_bits
from gpu_helpers import compare_bf16, dev, dev_bf16, host, host_u16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback

SENTINEL = 0x7FBF  # a NaN pattern no bf16 rounding produces (as the oracle's unused-row mark)


def dedup_cap(topk, E, R):
    _, rows, _ = oracle.default().layout_dedup(topk, E, R, 1 << 30)
    return int(rows.max()) if rows.size else 0


def check_prereduce(topk, w, E, R, H, cap, fp8=True, seed=3, chunk_rows=2048):
    """Deduplicated dispatch (fused launch), pre-reduction of random expert
    outputs (bf16 and fp32 sums) and the unit-weight combine of the reduced
    rows, every used row and every token against the oracle; the oracle runs
    on chunks of rows of the same seeded expert outputs."""
    orc = oracle.default()
    T, k = topk.shape
    n = R * cap
    rir_o, trows_o, st_o = orc.layout_dedup(topk, E, R, cap)
    pos_o, _ = orc.positions_dedup(topk, rir_o, E, R, cap)
    # the routing entries do not depend on x: a narrow zero x keeps this cheap
    _, _, rti_o, rtw_o = orc.dispatch_dedup(np.zeros((T, 8), np.uint16), topk, w, pos_o, E, R, n, False)

    rng = np.random.default_rng(seed)
    x = dev_bf16(to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    buf = ep.Buffer(T, H, k, E, R, cap)
    td = dev(topk.astype(np.int32))
    wd = None if w is None else dev(w.astype(np.float32))
    L, rx, rs, rti, rtw, h = buf.dispatch_dedup_with_layout(x, td, wd, fp8)
    assert buf.status() == st_o
    assert np.array_equal(host(h.pos), pos_o)
    if n == 0:
        buf.close()
        return
    eo = device_normal_bf16((n, k, H), seed=seed + 100)
    red = torch.full((n, H), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    red = buf.prereduce(eo, rti, rtw, L.token_rows, out=red)
    acc = torch.full((n, H), float("nan"), dtype=torch.float32, device="cuda")
    acc = buf.prereduce_f32(eo, rti, rtw, L.token_rows, out=acc)
    assert buf.status() == 0  # (the dispatch's bits were read and cleared above)
    red_o_all = np.full((n, H), SENTINEL, np.uint16)
    for lo in range(0, n, chunk_rows):
        hi = min(lo + chunk_rows, n)
        eo_c = host_u16(eo[lo:hi])
        red_o, acc_o = orc.prereduce(eo_c, rti_o[lo:hi], None if w is None else rtw_o[lo:hi], trows_o, R, cap,
                                     row_lo=lo, row_hi=hi, return_acc=True)
        red_o_all[lo:hi] = red_o
        got = host_u16(red[lo:hi])
        if not np.array_equal(got, red_o):  # unused rows: both keep the sentinel
            bad = np.argwhere(got != red_o)
            raise AssertionError(f"reduced rows differ at {(bad[:4] + [lo, 0]).tolist()}")
        got_acc = host(acc[lo:hi])
        used = red_o[:, 0] != SENTINEL
        assert np.array_equal(got_acc[used].view(np.uint32), acc_o[used].view(np.uint32)), f"fp32 sums {lo}.."
        assert np.all(np.isnan(got_acc[~used])), "unused rows of the fp32 sums written"
    # the reduced rows go back to their tokens: combine with unit weights
    if T > 0:
        y_o = orc.combine(red_o_all, pos_o, None)
        assert compare_bf16(host_u16(buf.combine(red, h, None)), y_o, "combine of reduced rows") == 1.0
    buf.close()


@pytest.mark.parametrize("name", ["tiny", "decode_rank", "decode", "prefill", "skewed"])
def test_prereduce_parity(name):
    cfg = CONFIGS[name]
    print(f"pre-reduction parity: {name} T={cfg.T} H={cfg.H}", flush=True)
    wl = make_workload(cfg, seed=0, with_x=False)
    cap = dedup_cap(wl.topk_idx, cfg.E, cfg.R)
    check_prereduce(wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cfg.H, cap, fp8=cfg.use_fp8)


def _routing(T, k, E, seed):
    rng = np.random.default_rng(seed)
    if T == 0:
        return np.zeros((0, k), np.int32), np.zeros((0, k), np.float32), rng
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    return topk, rng.random((T, k)).astype(np.float32), rng


PRE_EDGE = {
    "no_weights": dict(T=256, k=8, E=64, R=8, H=512),
    "capacity_drops": dict(T=512, k=8, E=64, R=8, H=256, cap_delta=-9),
    "zero_capacity_rows_unused": dict(T=0, k=4, E=16, R=4, H=256, cap=6),
    "k32": dict(T=96, k=32, E=64, R=16, H=256),
    "R1": dict(T=128, k=4, E=16, R=1, H=384),
    "E_equals_R": dict(T=320, k=4, E=8, R=8, H=256),
    "bad_repeated_empty_slots": dict(T=300, k=6, E=48, R=6, H=1152, dirty=True),
    "channel_tail": dict(T=200, k=4, E=32, R=4, H=9224, fp8=False),
    "E1024_R64": dict(T=1024, k=8, E=1024, R=64, H=512),
    # the rows per wave the launch picks from k: four rows at k = 16 (all 64
    # lanes hold entries) and k = 3 (12 lanes), two rows at k = 17 (34 lanes)
    "k16_four_rows_full_wave": dict(T=256, k=16, E=64, R=8, H=1024),
    "k3_R3": dict(T=300, k=3, E=12, R=3, H=2048),
    "k17_two_rows": dict(T=96, k=17, E=68, R=4, H=1024),
}


@pytest.mark.parametrize("name", list(PRE_EDGE))
def test_prereduce_edges(name):
    c = dict(PRE_EDGE[name])
    T, k, E, R, H = c["T"], c["k"], c["E"], c["R"], c["H"]
    topk, w, rng = _routing(T, k, E, seed=len(name))
    if c.get("dirty"):
        topk[rng.random(topk.shape) < 0.1] = -1
        topk[rng.random(topk.shape) < 0.05] = E + 5
        dup = rng.random(T) < 0.2
        topk[dup, k - 1] = topk[dup, 0]
    if name == "no_weights":
        w = None
    cap = c.get("cap", max(dedup_cap(topk, E, R) + c.get("cap_delta", 0), 0))
    check_prereduce(topk, w, E, R, H, cap, fp8=c.get("fp8", True))


def test_dedup_chain_equals_per_expert_combine():
    """On values exact in bf16 and fp32 (small integers, power-of-two
    weights) the deduplicated chain (each row's slot outputs taken from the
    per-expert outputs of the same (token, expert), pre-reduced, combined
    with unit weights) gives the per-expert weighted combine bit for bit."""
    orc = oracle.default()
    cfg = replace(CONFIGS["prefill"], T=1024, H=1024)
    wl = make_workload(cfg, seed=5, with_x=False)
    T, k, E, R, H = cfg.T, cfg.k, cfg.E, cfg.R, cfg.H
    rng = np.random.default_rng(6)
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], np.float32), size=(T, k))
    topk = wl.topk_idx
    Lo = orc.layout(topk, E, R, 1 << 30)
    cap_pe = int(Lo.rank_rows.max())
    Lo = orc.layout(topk, E, R, cap_pe)
    pos_pe, _ = orc.positions(topk, Lo, E, R, cap_pe)
    out_pe = dev_bf16(to_bf16_bits(rng.integers(-8, 9, size=(R * cap_pe, H)).astype(np.float32)))
    x = dev_bf16(np.zeros((T, H), np.uint16))
    td, wd = dev(topk), dev(w)
    b_pe = ep.Buffer(T, H, k, E, R, cap_pe)
    _, _, _, _, h_pe = b_pe.dispatch_with_layout(x, td, wd, False)
    y_pe = host_u16(b_pe.combine(out_pe, h_pe, wd))
    cap = dedup_cap(topk, E, R)
    b = ep.Buffer(T, H, k, E, R, cap)
    L, _, _, rti, rtw, h = b.dispatch_dedup_with_layout(x, td, wd, False)
    assert b_pe.status() == 0 and b.status() == 0
    # entry (row, slot) of the expert outputs: the per-expert output row of
    # that (token, expert), gathered with torch (test plumbing)
    pos_dd = host(h.pos)
    src = np.full((R * cap, k), -1, np.int64)
    for t in range(T):
        for j in range(k):
            p = pos_dd[t, j]
            if p < 0:
                continue
            d = p // cap
            for jj in range(k):
                if topk[t, jj] >= 0 and topk[t, jj] // (E // R) == d:
                    src[p, jj] = pos_pe[t, jj]
    gather = torch.from_numpy(np.maximum(src, 0).reshape(-1)).cuda()
    eo = out_pe.index_select(0, gather).view(R * cap, k, H).contiguous()
    red = b.prereduce(eo, rti, rtw, L.token_rows)
    y_dd = host_u16(b.combine(red, h, None))
    assert np.array_equal(y_dd, y_pe), "deduplicated chain differs from the per-expert combine"
    b.close()
    b_pe.close()
