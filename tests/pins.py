"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:
  * values worked out by hand from the definitions (tests/golden/*.json),
  * library routines that implement a special case independently (torch's
    float8_e4m3fn and bfloat16 casts, numpy's stable argsort, fp64 sums),
  * brute force over the definitions on tiny inputs (nearest-code search,
    O(T^2 k) counting of earlier tokens),
  * closed forms and invariants (copies are bit copies, the FP8 error bound,
    positions are a bijection onto the kept rows, identity experts give x
    back, an exact cancellation that depends on the slot order, a product that
    only a fused multiply-add keeps).
The same functions run against copies of the oracle with a planted mistake
(tests/test_oracle_mutants.py) to show that each plausible mistake is caught.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# test-side helpers built only from library routines
# ---------------------------------------------------------------------------

def bf16_bits_of(values) -> np.ndarray:
    """float32 -> bf16 bits using torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_e4m3_decode(codes) -> np.ndarray:
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def torch_e4m3_encode(values) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def nearest_e4m3(values) -> np.ndarray:
    """Brute force: the finite e4m3 code nearest to each value, ties to the
    even code, sign kept. The code table is torch's decoding of codes 0..126
    (all positive finite codes); values are monotone in the code, so a tie is
    always between two adjacent codes."""
    v = np.asarray(values, dtype=np.float32)
    table = torch_e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    out = np.empty(v.shape, np.uint8)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    for s in range(0, flat_v.size, 8192):
        # magnitudes past 1024 have the same nearest code as 1024 (all finite
        # codes are <= 448); clamping keeps the float64 distances exact
        mag = np.minimum(np.abs(flat_v[s:s + 8192].astype(np.float64)), 1024.0)
        d = np.abs(mag[:, None] - table[None, :])
        first = d.argmin(axis=1)
        m = d[np.arange(mag.size), first]
        nxt = np.minimum(first + 1, 126)
        tie = (nxt != first) & (d[np.arange(mag.size), nxt] == m)
        code = np.where(tie & (first % 2 == 1), nxt, first).astype(np.uint8)
        sign = np.signbit(flat_v[s:s + 8192]).astype(np.uint8) << 7
        flat_o[s:s + 8192] = code | sign
    return out


def bitsf(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def pin_e4m3_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan), "NaN codes differ"
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(bitsf(ours[~nan]), bitsf(ref[~nan])), "decoded values differ from torch"
    # values the OCP OFP8 specification states for E4M3
    spec = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 0.875 * 2.0 ** -6,
            0x01: 2.0 ** -9, 0x38: 1.0, 0x00: 0.0}
    for c, val in spec.items():
        assert ours[c] == np.float32(val), (hex(c), ours[c], val)
    assert np.signbit(ours[0x80]) and ours[0x80] == 0.0


def _encode_probe_values(rng):
    allbf = np.arange(65536, dtype=np.uint32)
    allbf = allbf[(allbf & 0x7F80) != 0x7F80]  # finite bf16 patterns
    v_bf = ((allbf << 16).astype(np.uint32)).view(np.float32)
    mags = np.exp2(rng.uniform(-12.0, 9.5, 60000)).astype(np.float32)
    v_rand = np.where(rng.random(60000) < 0.5, -mags, mags).astype(np.float32)
    table = torch_e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)  # exact in fp32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(np.inf))])
    big = np.array([447.9, 448.0, 449.0, 463.9, 464.0, 500.0, 1e6, 3e38], np.float32)
    return np.concatenate([v_bf, v_rand, near, -near, big, -big]).astype(np.float32)


def pin_e4m3_encode(orc):
    rng = np.random.default_rng(1234)
    v = _encode_probe_values(rng)
    ours = orc.e4m3_encode(v)
    ref = nearest_e4m3(v)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. v={v[bad[:4]]} ours={ours[bad[:4]]} ref={ref[bad[:4]]}"
    # library cross-check where torch's cast is defined the same way (|v| <= 448)
    inr = np.abs(v) <= 448.0
    assert np.array_equal(ours[inr], torch_e4m3_encode(v[inr])), "differs from torch float8_e4m3fn cast"


def pin_bf16_round(orc):
    rng = np.random.default_rng(99)
    pats = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    pats = pats[(pats & 0x7F800000) != 0x7F800000]  # finite
    ties = (rng.integers(0, 2 ** 16, 5000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000,
                        0x007FFFFF, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000,
                        0x3F808000, 0x3F818000, 0x7F800000, 0xFF800000], np.uint32)
    v = np.concatenate([pats, ties, special]).view(np.float32)
    ours = orc.bf16_round(v)
    ref = bf16_bits_of(v)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs torch, e.g. {v.view(np.uint32)[bad[:4]]}"


# ---------------------------------------------------------------------------
# layout and positions
# ---------------------------------------------------------------------------

def pin_layout_golden(orc):
    g = golden("layout_by_hand.json")
    topk = np.array(g["topk_idx"], np.int32)
    E, R, H = g["E"], g["R"], g["H"]
    for case in g["cases"]:
        cap = case["cap_rows"]
        L = orc.layout(topk, E, R, cap)
        for key in ("rank_in_expert", "recv_cnt", "expert_off", "rank_rows", "cnt_se",
                    "cnt_sd", "src_expert_off", "is_token_in_rank"):
            assert np.array_equal(getattr(L, key), np.array(g[key])), (key, cap)
        assert L.status == case["status"], (L.status, case["status"])
        pos, src_idx = orc.positions(topk, L, E, R, cap)
        assert np.array_equal(pos, np.array(case["pos"])), ("pos", cap, pos)
        assert np.array_equal(src_idx, np.array(case["src_idx"])), ("src_idx", cap)
        if "combine_y" in case:
            rows = np.repeat(bf16_bits_of(np.arange(1, R * cap + 1, dtype=np.float32))[:, None], H, 1)
            w = np.tile(np.array(case["combine_weights"], np.float32), (topk.shape[0], 1))
            y = f32_of_bf16(orc.combine(rows, pos, w))
            assert np.array_equal(y, np.repeat(np.array(case["combine_y"], np.float32)[:, None], H, 1)), y[:, 0]


def brute_layout(topk, E, R, cap):
    """Direct counting over the definitions, O(T^2 k), for tiny inputs."""
    T, k = topk.shape
    tpr, epr = (T // R if R else 0), E // R
    status = 0
    valid = np.zeros((T, k), bool)
    for t in range(T):
        for j in range(k):
            e = int(topk[t, j])
            if e == -1:
                continue
            if e < -1 or e >= E:
                status |= 1
                continue
            if e in [int(x) for x in topk[t, :j]]:
                status |= 2
                continue
            valid[t, j] = True
    experts_of = [set(int(topk[t, j]) for j in range(k) if valid[t, j]) for t in range(T)]
    rie = np.full((T, k), -1, np.int64)
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                e = int(topk[t, j])
                rie[t, j] = sum(1 for tp in range(t) if e in experts_of[tp])
    src = [t // tpr for t in range(T)]
    cnt_se = np.array([[sum(1 for t in range(T) if src[t] == s and e in experts_of[t])
                        for e in range(E)] for s in range(R)])
    itr = np.array([[int(any(e // epr == d for e in experts_of[t])) for d in range(R)]
                    for t in range(T)], dtype=np.int64).reshape(T, R)
    cnt_sd = np.array([[sum(int(itr[t, d]) for t in range(T) if src[t] == s) for d in range(R)]
                       for s in range(R)])
    recv = np.array([sum(1 for t in range(T) if e in experts_of[t]) for e in range(E)])
    eoff = np.array([sum(int(recv[x]) for x in range((e // epr) * epr, e)) for e in range(E)])
    rrows = np.array([sum(int(recv[e]) for e in range(d * epr, (d + 1) * epr)) for d in range(R)])
    seoff = np.array([[int(eoff[e]) + sum(int(cnt_se[sp, e]) for sp in range(s)) for e in range(E)]
                      for s in range(R)])
    if any(int(r) > cap for r in rrows):
        status |= 4
    return dict(rank_in_expert=rie, cnt_se=cnt_se, is_token_in_rank=itr, cnt_sd=cnt_sd,
                recv_cnt=recv, expert_off=eoff, rank_rows=rrows, src_expert_off=seoff,
                status=status, valid=valid)


def pin_layout_bruteforce(orc):
    rng = np.random.default_rng(7)
    shapes = [(0, 1, 1, 1), (0, 3, 4, 2), (1, 1, 1, 1), (4, 2, 4, 2), (6, 3, 6, 3),
              (16, 2, 16, 4), (12, 4, 8, 4), (20, 3, 5, 5), (24, 5, 12, 6), (8, 8, 8, 8)]
    for it, (T, k, E, R) in enumerate(shapes * 2):
        dirty = it >= len(shapes)  # second round: invalid ids, repeats, -1 slots
        if dirty:
            topk = rng.integers(-3, E + 2, (T, k)).astype(np.int32)
        elif T == 0:
            topk = np.zeros((0, k), np.int32)
        else:
            topk = np.stack([rng.permutation(E)[:k] if k <= E else
                             np.concatenate([rng.permutation(E), -np.ones(k - E, int)])
                             for _ in range(T)]).astype(np.int32).reshape(T, k)
        cap = int(rng.integers(0, max(2, T * k // max(R, 1) + 2)))
        ref = brute_layout(topk, E, R, cap)
        L = orc.layout(topk, E, R, cap)
        for key in ("rank_in_expert", "cnt_se", "is_token_in_rank", "cnt_sd", "recv_cnt",
                    "expert_off", "rank_rows", "src_expert_off"):
            assert np.array_equal(np.asarray(getattr(L, key), np.int64), ref[key]), (key, T, k, E, R)
        assert L.status == ref["status"], ("status", L.status, ref["status"], T, k, E, R)
        # positions: rank*cap + expert_off + rank, dropped at or past cap
        pos, src_idx = orc.positions(topk, L, E, R, cap)
        for t in range(T):
            for j in range(k):
                if not ref["valid"][t, j]:
                    assert pos[t, j] == -1
                    continue
                e = int(topk[t, j])
                local = int(ref["expert_off"][e]) + int(ref["rank_in_expert"][t, j])
                want = -1 if local >= cap else (e // (E // R)) * cap + local
                assert pos[t, j] == want, ("pos", t, j, pos[t, j], want)
                if want >= 0:
                    assert src_idx[want] == t


def pin_layout_argsort(orc):
    """Stable sort re-derivation: the (token, slot) entries in token-major order,
    stably sorted by expert id, are exactly the receive rows in order."""
    rng = np.random.default_rng(11)
    for T, k, E, R in [(2000, 8, 64, 8), (512, 4, 32, 32), (777 * 3, 6, 96, 3)]:
        topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        topk[rng.random((T, k)) < 0.05] = -1  # some empty slots
        cap = T * k
        L = orc.layout(topk, E, R, cap)
        pos, _ = orc.positions(topk, L, E, R, cap)
        flat = topk.reshape(-1)
        keep = np.nonzero(flat >= 0)[0]
        order = np.argsort(flat[keep], kind="stable")  # library stable sort
        sorted_entries = keep[order]
        sorted_exp = flat[sorted_entries]
        first_of_expert = np.searchsorted(sorted_exp, np.arange(E))
        epr = E // R
        first_of_rank = first_of_expert[np.arange(R) * epr]
        idx_in_sorted = np.empty(flat.size, np.int64)
        idx_in_sorted[sorted_entries] = np.arange(keep.size)
        rie = np.full(flat.size, -1, np.int64)
        rie[keep] = idx_in_sorted[keep] - first_of_expert[flat[keep]]
        assert np.array_equal(L.rank_in_expert.reshape(-1), rie), "rank_in_expert != stable argsort rank"
        want_pos = np.full(flat.size, -1, np.int64)
        d = flat[keep] // epr
        want_pos[keep] = d * cap + (idx_in_sorted[keep] - first_of_rank[d])
        assert np.array_equal(pos.reshape(-1), want_pos), "positions != stable argsort rows"


def check_layout_invariants(topk, E, R, cap, L, pos, src_idx):
    T, k = topk.shape
    epr = E // R
    valid = pos >= 0
    assert L.recv_cnt.sum() == (L.rank_in_expert >= 0).sum()
    assert np.array_equal(L.cnt_se.sum(0), L.recv_cnt)
    assert np.array_equal(L.is_token_in_rank.sum(0), L.cnt_sd.sum(0))
    for d in range(R):
        assert L.rank_rows[d] == L.recv_cnt[d * epr:(d + 1) * epr].sum()
    # positions: a bijection onto the kept rows d*cap + [0, min(rank_rows, cap))
    p = pos[valid]
    assert np.unique(p).size == p.size, "two slots share a row"
    want = np.concatenate([d * cap + np.arange(min(int(L.rank_rows[d]), cap)) for d in range(R)] +
                          [np.zeros(0, np.int64)])
    assert np.array_equal(np.sort(p), np.sort(want)), "kept rows are not the rank prefixes"
    tok = np.repeat(np.arange(T), k).reshape(T, k)
    assert np.array_equal(src_idx[p], tok[valid]), "src_idx[pos] != token"
    # every (token, expert) pair of a kept slot lands in that expert's region once
    e = topk[valid]
    local = p - (e // epr) * cap
    assert np.all(local >= L.expert_off[e]) and np.all(local < L.expert_off[e] + L.recv_cnt[e])
    # rows of one expert hold strictly increasing source tokens
    for ee in np.unique(e):
        rows = np.sort(p[e == ee])
        assert np.all(np.diff(src_idx[rows]) > 0), f"expert {ee} rows not in token order"
    # src_expert_off: inside rank d(e)'s region, the rows source rank s sends
    # to expert e start there
    tpr = T // R if T else 1
    for s_, ee, pp in zip(tok[valid] // tpr, e, local):
        lo = L.src_expert_off[s_, ee]
        assert lo <= pp < lo + L.cnt_se[s_, ee]


def pin_layout_invariants(orc):
    from dataclasses import replace
    from combine_get_dispatch_amd.workloads import CONFIGS, make_workload
    for name in ("tiny", "decode", "prefill", "skewed"):
        cfg = CONFIGS[name]
        cfg = replace(cfg, T=min(cfg.T, 1024))
        wl = make_workload(cfg, seed=3, with_x=False)
        E, R = cfg.E, cfg.R
        L0 = orc.layout(wl.topk_idx, E, R, 1 << 30)
        cap = int(L0.rank_rows.max())
        for c in (cap, max(cap - 7, 0)):
            L = orc.layout(wl.topk_idx, E, R, c)
            pos, src_idx = orc.positions(wl.topk_idx, L, E, R, c)
            check_layout_invariants(wl.topk_idx, E, R, c, L, pos, src_idx)
            assert (L.status == 4) == (c < cap)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

def _small_case(orc, rng, T=48, k=3, E=12, R=4, H=384, drop=True):
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if drop:
        topk[rng.random((T, k)) < 0.1] = -1
    w = rng.random((T, k)).astype(np.float32)
    L = orc.layout(topk, E, R, 1 << 30)
    cap = int(L.rank_rows.max())
    L = orc.layout(topk, E, R, cap)
    pos, src_idx = orc.positions(topk, L, E, R, cap)
    return topk, w, L, cap, pos, src_idx


def pin_dispatch_bf16(orc):
    rng = np.random.default_rng(5)
    topk, w, L, cap, pos, _ = _small_case(orc, rng)
    T, k = topk.shape
    x = bf16_bits_of(rng.standard_normal((T, 384)).astype(np.float32))
    recv_x, rs, recv_w = orc.dispatch(x, w, pos, 4 * cap, use_fp8=False)
    assert rs is None
    used = np.zeros(4 * cap, bool)
    for t in range(T):
        for j in range(k):
            p = pos[t, j]
            if p >= 0:
                assert np.array_equal(recv_x[p], x[t]), (t, j)
                assert bitsf(recv_w[p]) == bitsf(w[t, j])
                used[p] = True
    assert not recv_x[~used].any(), "a row no slot maps to was written"


def pin_fp8_golden(orc):
    g = golden("fp8_by_hand.json")
    H = g["H"]
    vals = np.zeros(H, np.float32)
    bits = np.zeros(H, np.uint16)
    codes = np.zeros(H, np.uint8)
    for ch, v, c in g["channels"]:
        if isinstance(v, str):
            bits[ch] = int(v, 16)
        else:
            vals[ch] = v
            bits[ch] = bf16_bits_of(np.array([v], np.float32))[0]
        codes[ch] = c
    assert np.array_equal(f32_of_bf16(bits)[:15], vals[:15])  # all hand values are exact bf16
    q, s = orc.quantize_token(bits)
    assert np.array_equal(q, codes), (np.nonzero(q != codes)[0], q[q != codes])
    assert [hex(int(b)) for b in bitsf(s)] == [h.lower() for h in g["scales_hex"]]
    # the same row through dispatch, one token routed to one expert
    topk = np.zeros((1, 1), np.int32)
    L = orc.layout(topk, 1, 1, 1)
    pos, _ = orc.positions(topk, L, 1, 1, 1)
    rx, rs, _ = orc.dispatch(bits[None, :], np.ones((1, 1), np.float32), pos, 1, use_fp8=True)
    assert np.array_equal(rx[0], codes) and np.array_equal(bitsf(rs[0]), bitsf(s))
    # an all-zero group: all codes zero, scale from the 1e-4 floor
    q0, s0 = orc.quantize_token(np.zeros(128, np.uint16))
    assert not q0.any()
    assert abs(float(s0[0]) - 1e-4 / 448) <= 1e-4 / 448 * 2 ** -22
    qn, _ = orc.quantize_token(np.full(128, 0x8000, np.uint16))  # all -0.0
    assert np.all(qn == 0x80)


def _fp8_rows(rng, T, H):
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[::7] *= 100.0                               # hot rows
    x[1::5, :128] *= np.exp2(rng.uniform(-20, 6, (len(range(1, T, 5)), 128))).astype(np.float32)
    x[2, 128:256] = 0.0                            # an all-zero group
    return bf16_bits_of(x)


def pin_fp8_bound(orc):
    rng = np.random.default_rng(21)
    T, H = 40, 1024
    xb = _fp8_rows(rng, T, H)
    x = f32_of_bf16(xb).astype(np.float64)
    for t in range(T):
        q, s = orc.quantize_token(xb[t])
        deq = torch_e4m3_decode(q).astype(np.float64) * np.repeat(s.astype(np.float64), 128)
        sc = np.repeat(s.astype(np.float64), 128)
        bound = (2.0 ** -4 + 2.0 ** -20) * np.abs(x[t]) + 2.0 ** -10 * sc
        assert np.all(np.abs(x[t] - deq) <= bound), ("fp8 error bound", t)
        for g in range(H // 128):
            grp = x[t, g * 128:(g + 1) * 128]
            amax = np.abs(grp).max()
            if amax >= 1e-4:
                i = np.abs(grp).argmax()
                assert q[g * 128 + i] & 0x7F == 0x7E, ("amax element must encode to 448", t, g)
                assert abs(float(s[g]) * 448.0 - amax) <= amax * 2.0 ** -22


def pin_fp8_torch(orc):
    """Same reading computed with library routines: numpy IEEE fp32 division for
    the scale, torch's float8_e4m3fn cast for the codes."""
    rng = np.random.default_rng(22)
    T, H = 24, 768
    xb = _fp8_rows(rng, T, H)
    x = f32_of_bf16(xb).reshape(T, H // 128, 128)
    amax = np.abs(x).max(axis=2)
    a = np.maximum(amax, np.float32(1e-4)).astype(np.float32)
    inv = (np.float32(448.0) / a).astype(np.float32)
    scale = (a / np.float32(448.0)).astype(np.float32)
    prod = (x * inv[:, :, None]).astype(np.float32)
    ref_q = torch_e4m3_encode(prod).reshape(T, H)
    for t in range(T):
        q, s = orc.quantize_token(xb[t])
        assert np.array_equal(q, ref_q[t]), ("codes differ from torch cast", t)
        assert np.array_equal(bitsf(s), bitsf(scale[t])), ("scales differ", t)


# ---------------------------------------------------------------------------
# combine and backward
# ---------------------------------------------------------------------------

def pin_combine_fp64(orc):
    rng = np.random.default_rng(31)
    topk, w, L, cap, pos, _ = _small_case(orc, rng, T=64, k=8, E=32, R=4, H=256)
    rows = bf16_bits_of(rng.standard_normal((4 * cap, 256)).astype(np.float32))
    y, acc = orc.combine(rows, pos, w, return_acc=True)
    rf = f32_of_bf16(rows).astype(np.float64)
    T, k = pos.shape
    ref = np.zeros((T, 256))
    mag = np.zeros((T, 256))
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                ref[t] += float(w[t, j]) * rf[pos[t, j]]
                mag[t] += abs(float(w[t, j])) * np.abs(rf[pos[t, j]])
    assert np.all(np.abs(acc.astype(np.float64) - ref) <= k * 2.0 ** -24 * mag + 1e-30), "fp32 sum off"
    assert np.array_equal(y, bf16_bits_of(acc)), "output is not the bf16 rounding of the fp32 sum"
    # w = NULL means unit weights
    y1, acc1 = orc.combine(rows, pos, None, return_acc=True)
    ref1 = np.zeros((T, 256))
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                ref1[t] += rf[pos[t, j]]
    assert np.all(np.abs(acc1 - ref1) <= k * 2.0 ** -24 * np.abs(ref1).max() + 1e-30)


def pin_combine_order(orc):
    """Slot order is part of the definition: 2^24 + 1 rounds back to 2^24 in
    fp32, so (2^24, 1, -2^24) sums to 0 in slot order while (-2^24, 1, 2^24)
    sums to 1."""
    rows = np.repeat(bf16_bits_of(np.array([2.0 ** 24, 1.0, -(2.0 ** 24)], np.float32))[:, None], 8, 1)
    pos = np.array([[0, 1, 2], [2, 1, 0]], np.int32)
    w = np.ones((2, 3), np.float32)
    y = f32_of_bf16(orc.combine(rows, pos, w))
    assert np.all(y[0] == 0.0) and np.all(y[1] == 1.0), y[:, 0]


def pin_combine_fma(orc):
    """One fused multiply-add per slot: (1+2^-23)(1+2^-7) needs 31 bits, and
    only a fused operation keeps its 2^-30 term after adding -1."""
    rows = np.repeat(bf16_bits_of(np.array([-1.0, 1.0 + 2.0 ** -7], np.float32))[:, None], 8, 1)
    pos = np.array([[0, 1]], np.int32)
    w = np.array([[1.0, 1.0 + 2.0 ** -23]], np.float32)
    _, acc = orc.combine(rows, pos, w, return_acc=True)
    want = np.float32(2.0 ** -7 + 2.0 ** -23 + 2.0 ** -30)
    assert np.all(acc == want), (acc[0, 0], want)


def pin_combine_identity(orc):
    """Identity experts: dispatch in BF16, feed the received rows straight back,
    combine with weights that sum to one: the result is x itself."""
    from dataclasses import replace
    from combine_get_dispatch_amd.workloads import CONFIGS, make_workload
    cfg = replace(CONFIGS["decode"], T=96, H=512)
    wl = make_workload(cfg, seed=4)
    L = orc.layout(wl.topk_idx, cfg.E, cfg.R, 1 << 30)
    cap = int(L.rank_rows.max())
    L = orc.layout(wl.topk_idx, cfg.E, cfg.R, cap)
    pos, _ = orc.positions(wl.topk_idx, L, cfg.E, cfg.R, cap)
    recv_x, _, _ = orc.dispatch(wl.x, wl.topk_w, pos, cfg.R * cap, use_fp8=False)
    y = orc.combine(recv_x, pos, wl.topk_w)
    assert np.array_equal(y, wl.x), "identity experts did not return x"
    # unit weights: x * k, exact in bf16 for k a power of two
    y8 = orc.combine(recv_x, pos, None)
    assert np.array_equal(f32_of_bf16(y8), f32_of_bf16(wl.x) * np.float32(cfg.k))


def pin_backward(orc):
    rng = np.random.default_rng(41)
    topk, w, L, cap, pos, _ = _small_case(orc, rng, T=32, k=4, E=16, R=4, H=128)
    T, k = pos.shape
    H = 128
    n = 4 * cap
    gy = bf16_bits_of(rng.standard_normal((T, H)).astype(np.float32))
    grows = orc.combine_backward(gy, pos, n)
    ref, _, _ = orc.dispatch(gy, None, pos, n, use_fp8=False)
    assert np.array_equal(grows, ref), "combine_backward is not a bf16 dispatch of grad_y"
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                assert np.array_equal(grows[pos[t, j]], gy[t])
    # adjoint: <dispatch(x), G> == <x, unweighted combine(G)> (fp64, up to the fp32 sums)
    x = bf16_bits_of(rng.standard_normal((T, H)).astype(np.float32))
    G = bf16_bits_of(rng.standard_normal((n, H)).astype(np.float32))
    rx, _, _ = orc.dispatch(x, None, pos, n, use_fp8=False)
    yb, acc = orc.combine(G, pos, None, return_acc=True)
    lhs = float((f32_of_bf16(rx).astype(np.float64) * f32_of_bf16(G)).sum())
    rhs = float((f32_of_bf16(x).astype(np.float64) * acc.astype(np.float64)).sum())
    scale = float((np.abs(f32_of_bf16(x)).astype(np.float64)[:, :] *
                   np.abs(acc).astype(np.float64)).sum())
    assert abs(lhs - rhs) <= k * 2.0 ** -23 * scale, (lhs, rhs)
    gx = orc.dispatch_backward(G, pos, w)
    assert np.array_equal(gx, orc.combine(G, pos, w))


# ---------------------------------------------------------------------------
# rank-deduplicated exchange
# ---------------------------------------------------------------------------

def pin_dedup_golden(orc):
    g = golden("layout_by_hand.json")
    topk = np.array(g["topk_idx"], np.int32)
    E, R, H = g["E"], g["R"], g["H"]
    dd = g["dedup"]
    w = np.tile(np.array([0.5, 0.25], np.float32), (topk.shape[0], 1))
    x = bf16_bits_of(np.arange(topk.shape[0] * H, dtype=np.float32).reshape(-1, H))
    for case in dd["cases"]:
        cap = case["cap_rows"]
        rir, rows, st = orc.layout_dedup(topk, E, R, cap)
        assert np.array_equal(rir, np.array(dd["rank_in_rank"])), rir
        assert np.array_equal(rows, np.array(dd["token_rows"])), rows
        assert st == case["status"], (st, case["status"])
        pos, src_idx = orc.positions_dedup(topk, rir, E, R, cap)
        assert np.array_equal(pos, np.array(case["pos"])), ("pos", cap, pos)
        if "recv_topk_idx" in case:
            rx, _, rti, rtw = orc.dispatch_dedup(x, topk, w, pos, E, R, R * cap, use_fp8=False)
            for row, want in case["recv_topk_idx"].items():
                r = int(row)
                assert np.array_equal(rti[r], np.array(want)), (r, rti[r], want)
                assert np.array_equal(rtw[r], np.where(np.array(want) >= 0, w[src_idx[r]], 0.0)), r
                assert np.array_equal(rx[r], x[src_idx[r]]), r


def brute_dedup(topk, E, R):
    """Leaders and per-rank rows counted directly from the definitions, O(T^2 k)."""
    T, k = topk.shape
    epr = E // R

    def kept(t):  # valid slots of token t, first occurrence only
        seen, out = set(), []
        for j in range(k):
            e = int(topk[t, j])
            if 0 <= e < E and e not in seen:
                out.append((j, e))
            if 0 <= e < E:
                seen.add(e)
        return out

    on = np.zeros((T, R), bool)
    for t in range(T):
        for _, e in kept(t):
            on[t, e // epr] = True
    rir = np.full((T, k), -1, np.int32)
    for t in range(T):
        done = set()
        for j, e in kept(t):
            d = e // epr
            if d in done:
                continue
            done.add(d)
            rir[t, j] = int(on[:t, d].sum())
    return rir, on.sum(0).astype(np.int32), on


def pin_dedup_bruteforce(orc):
    rng = np.random.default_rng(57)
    for T, k, E, R in ((32, 4, 16, 4), (40, 6, 24, 8), (24, 8, 8, 2)):
        topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        topk[rng.random((T, k)) < 0.15] = -1
        topk[rng.random((T, k)) < 0.05] = E + 3                          # bad ids
        dup = rng.random(T) < 0.2
        topk[dup, k - 1] = topk[dup, 0]                                   # repeats
        rir, rows, _ = orc.layout_dedup(topk, E, R, 1 << 30)
        brir, brows, on = brute_dedup(topk, E, R)
        assert np.array_equal(rir, brir), (T, k, E, R)
        assert np.array_equal(rows, brows)
        L = orc.layout(topk, E, R, 1 << 30)
        assert np.array_equal(rows, L.cnt_sd.sum(0)), "token rows != summed cnt_sd"
        assert np.array_equal(on.astype(np.uint8), L.is_token_in_rank)
        assert ((rir >= 0).sum(1) == L.is_token_in_rank.sum(1)).all(), "one leader per (token, rank)"


def pin_dedup_dispatch(orc):
    rng = np.random.default_rng(58)
    T, k, E, R, H = 32, 4, 16, 4, 256
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    topk[rng.random((T, k)) < 0.1] = -1
    w = rng.random((T, k)).astype(np.float32)
    x = bf16_bits_of(rng.standard_normal((T, H)).astype(np.float32))
    rir, rows, _ = orc.layout_dedup(topk, E, R, 1 << 30)
    cap = int(rows.max())
    pos, src_idx = orc.positions_dedup(topk, rir, E, R, cap)
    epr = E // R
    for fp8 in (False, True):
        rx, rs, rti, rtw = orc.dispatch_dedup(x, topk, w, pos, E, R, R * cap, fp8)
        for t in range(T):
            for j in range(k):
                p = pos[t, j]
                if p < 0:
                    continue
                d = p // cap
                assert topk[t, j] // epr == d
                if fp8:
                    q, s = orc.quantize_token(x[t])
                    assert np.array_equal(rx[p], q) and np.array_equal(rs[p], s)
                else:
                    assert np.array_equal(rx[p], x[t])
                for jj in range(k):
                    e = topk[t, jj]
                    here = e >= 0 and e // epr == d
                    assert rti[p, jj] == (e - d * epr if here else -1), (t, j, jj)
                    assert rtw[p, jj] == (w[t, jj] if here else 0.0)


# ---------------------------------------------------------------------------
# expert-side pre-reduction of deduplicated rows
# ---------------------------------------------------------------------------

def f32_nearest(fr):
    """The fp32 value nearest to the rational fr, ties to the even pattern
    (exact: candidates around numpy's double-rounded value compared as
    fractions). Exact zeros come out as +0."""
    from fractions import Fraction
    if fr == 0:
        return np.float32(0.0)
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(np.float32(v).view(np.uint32)) & 1))


def fma32(a, b, c):
    """fp32 fused multiply-add, a * b + c rounded once, by exact arithmetic."""
    from fractions import Fraction
    return f32_nearest(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def pin_prereduce_golden(orc):
    g = golden("layout_by_hand.json")
    dd, pr = g["dedup"], g["prereduce"]
    case = [c for c in dd["cases"] if c["cap_rows"] == pr["cap_rows"]][0]
    R, H, k, cap = g["R"], g["H"], g["k"], pr["cap_rows"]
    n = R * cap
    rti = np.full((n, k), -1, np.int32)
    for p, e in case["recv_topk_idx"].items():
        rti[int(p)] = e
    rtw = np.where(rti >= 0, np.array(pr["slot_weights"], np.float32)[None, :], 0.0).astype(np.float32)
    vals = np.array([[8.0 * (p + 1) + (j + 1) for j in range(k)] for p in range(n)], np.float32)
    eo = np.repeat(bf16_bits_of(vals)[:, :, None], H, 2)
    tr = np.array(pr["token_rows"], np.int32)
    red = orc.prereduce(eo, rti, rtw, tr, R, cap)
    for p, v in pr["reduced"].items():
        assert np.all(f32_of_bf16(red[int(p)]) == v), (p, f32_of_bf16(red[int(p)])[0], v)
    for p in pr["unused_rows"]:
        assert np.all(red[p] == orc.UNUSED_ROW), ("unused row written", p)
    y = f32_of_bf16(orc.combine(red, np.array(case["pos"], np.int32), None))
    assert np.array_equal(y, np.repeat(np.array(pr["combined"], np.float32)[:, None], H, 1)), y[:, 0]
    # a row range computes the same rows
    sub = orc.prereduce(eo[8:], rti[8:], rtw[8:], tr, R, cap, row_lo=8)
    assert np.array_equal(sub, red[8:])


def pin_prereduce_bruteforce(orc):
    """fp32 fused multiply-adds in slot order, by exact arithmetic, on random
    tiny inputs (random slot entries, weights and outputs, rows past
    token_rows and capacity-limited ranks)."""
    rng = np.random.default_rng(71)
    for R, cap, k, H in ((2, 5, 3, 8), (3, 4, 4, 4), (1, 6, 2, 8), (4, 3, 5, 2)):
        n = R * cap
        rti = rng.integers(-1, 3, size=(n, k)).astype(np.int32)
        rtw = rng.standard_normal((n, k)).astype(np.float32)
        eo = bf16_bits_of(rng.standard_normal((n, k, H)).astype(np.float32))
        tr = rng.integers(0, cap + 2, size=R).astype(np.int32)  # some ranks past their capacity
        for weights in (rtw, None):
            red, acc = orc.prereduce(eo, rti, weights, tr, R, cap, return_acc=True)
            for p in range(n):
                d, local = divmod(p, cap)
                if local >= tr[d]:
                    assert np.all(red[p] == orc.UNUSED_ROW) and np.all(np.isnan(acc[p])), ("row", p)
                    continue
                for i in range(H):
                    s = np.float32(0.0)
                    for j in range(k):
                        if rti[p, j] >= 0:
                            wj = np.float32(1.0) if weights is None else weights[p, j]
                            s = fma32(wj, f32_of_bf16(eo[p, j, i]), s)
                    assert acc[p, i].view(np.uint32) == np.float32(s).view(np.uint32), (p, i, acc[p, i], s)
                    assert red[p, i] == bf16_bits_of(np.array([s], np.float32))[0], (p, i)


def pin_prereduce_order_fma(orc):
    """Slot order and one fused multiply-add per slot are part of the
    definition: (2^24, 1, -2^24) sums to 0 in slot order, (-2^24, 1, 2^24) to
    1; (1+2^-23)(1+2^-7) - 1 keeps its 2^-30 term."""
    k, H = 3, 4
    vals = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)], [-(2.0 ** 24), 1.0, 2.0 ** 24],
                     [-1.0, 1.0 + 2.0 ** -7, 0.0]], np.float32)
    eo = np.repeat(bf16_bits_of(vals)[:, :, None], H, 2)
    rti = np.array([[0, 1, 2], [0, 1, 2], [0, 1, -1]], np.int32)
    rtw = np.array([[1, 1, 1], [1, 1, 1], [1.0, 1.0 + 2.0 ** -23, 0]], np.float32)
    red, acc = orc.prereduce(eo, rti, rtw, np.array([3], np.int32), 1, 3, return_acc=True)
    assert np.all(acc[0] == 0.0) and np.all(acc[1] == 1.0), acc[:, 0]
    assert np.all(acc[2] == np.float32(2.0 ** -7 + 2.0 ** -23 + 2.0 ** -30)), acc[2, 0]


def pin_prereduce_fp64(orc):
    """fp64 bound on a larger random case: |sum - sum_j w v| <= k 2^-24 sum_j |w v|."""
    rng = np.random.default_rng(72)
    R, cap, k, H = 4, 40, 8, 256
    n = R * cap
    rti = np.where(rng.random((n, k)) < 0.3, 1, -1).astype(np.int32)
    rtw = rng.random((n, k)).astype(np.float32)
    eo = bf16_bits_of(rng.standard_normal((n, k, H)).astype(np.float32))
    tr = np.full(R, cap, np.int32)
    _, acc = orc.prereduce(eo, rti, rtw, tr, R, cap, return_acc=True)
    wv = np.where(rti[:, :, None] >= 0, rtw[:, :, None].astype(np.float64) * f32_of_bf16(eo).astype(np.float64), 0)
    exact, mag = wv.sum(1), np.abs(wv).sum(1)
    assert np.all(np.abs(acc.astype(np.float64) - exact) <= k * 2.0 ** -24 * mag + 1e-300)


def pin_dedup_prereduce(orc):
    """Per-expert exchange vs deduplicated exchange with the expert side
    pre-reducing (oracle_prereduce: weighting and summing the outputs of a
    row's local experts): on values exact in bf16 and fp32 both give the same
    combined result."""
    rng = np.random.default_rng(59)
    T, k, E, R, H = 48, 4, 16, 4, 128
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    topk[rng.random((T, k)) < 0.1] = -1
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], np.float32), size=(T, k))
    L = orc.layout(topk, E, R, 1 << 30)
    cap = int(L.rank_rows.max())
    L = orc.layout(topk, E, R, cap)
    pos, _ = orc.positions(topk, L, E, R, cap)
    out = bf16_bits_of(rng.integers(-8, 9, size=(R * cap, H)).astype(np.float32))  # per-expert outputs
    y_ref = orc.combine(out, pos, w)
    rir, rows, _ = orc.layout_dedup(topk, E, R, cap)
    pdd, _ = orc.positions_dedup(topk, rir, E, R, cap)
    _, _, rti, rtw = orc.dispatch_dedup(np.zeros((T, H), np.uint16), topk, w, pdd, E, R, R * cap, False)
    # each deduplicated row's slot outputs: the per-expert output of that
    # (token, expert), i.e. what the rank's expert computes for the row
    eo = np.zeros((R * cap, k, H), np.uint16)
    epr = E // R
    for t in range(T):
        for j in range(k):
            p = pdd[t, j]
            if p < 0:
                continue
            for jj in range(k):
                if rti[p, jj] >= 0:
                    assert pos[t, jj] >= 0 and topk[t, jj] == rti[p, jj] + (p // cap) * epr
                    eo[p, jj] = out[pos[t, jj]]
    pre = orc.prereduce(eo, rti, rtw, rows, R, cap)
    y_dd = orc.combine(pre, pdd, None)
    assert np.array_equal(y_dd, y_ref), "dedup + pre-reduction differs from the per-expert combine"


def pin_ll_golden(orc):
    g = golden("layout_by_hand.json")
    topk = np.array(g["topk_idx"], np.int32)
    E, R = g["E"], g["R"]
    ll = g["low_latency"]
    pos, src_idx, cnt, st = orc.ll_positions(topk, E, R)
    assert np.array_equal(pos, np.array(ll["pos"])), pos
    assert np.array_equal(cnt, np.array(ll["recv_count"])), cnt
    assert st == ll["status"]
    for t, row in enumerate(ll["pos"]):
        for p in row:
            if p >= 0:
                assert src_idx[p] == t


def brute_ll(topk, E, R):
    """Low-latency rows counted directly from the definition, O(T^2 k)."""
    T, k = topk.shape
    tpr = T // R

    def kept(t):
        seen, out = set(), []
        for j in range(k):
            e = int(topk[t, j])
            if 0 <= e < E and e not in seen:
                out.append((j, e))
            if 0 <= e < E:
                seen.add(e)
        return out

    pos = np.full((T, k), -1, np.int32)
    for t in range(T):
        s = t // tpr
        for j, e in kept(t):
            before = sum(1 for u in range(s * tpr, t) if any(ee == e for _, ee in kept(u)))
            pos[t, j] = e * R * tpr + s * tpr + before
    return pos


def pin_ll_bruteforce(orc):
    """Brute force, and agreement with the per-expert layout: a region holds
    cnt_se[s][e] rows, and a slot's row inside it is its rank-local row in the
    per-expert layout less where its source's rows start there
    (expert_off + rank_in_expert - src_expert_off)."""
    rng = np.random.default_rng(61)
    for T, k, E, R in ((32, 4, 16, 4), (40, 6, 24, 8), (24, 8, 8, 2), (9, 3, 6, 3)):
        topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        topk[rng.random((T, k)) < 0.15] = -1
        topk[rng.random((T, k)) < 0.05] = E + 2
        dup = rng.random(T) < 0.2
        topk[dup, k - 1] = topk[dup, 0]
        pos, src_idx, cnt, st = orc.ll_positions(topk, E, R)
        assert np.array_equal(pos, brute_ll(topk, E, R)), (T, k, E, R)
        L = orc.layout(topk, E, R, 1 << 30)
        assert st == L.status
        assert np.array_equal(cnt, L.cnt_se.T), "region counts != cnt_se"
        tpr = T // R
        for t in range(T):
            s = t // tpr
            for j in range(k):
                p = pos[t, j]
                assert (p >= 0) == (L.rank_in_expert[t, j] >= 0)
                if p >= 0:
                    e = topk[t, j]
                    assert (p - e * R * tpr - s * tpr ==
                            L.expert_off[e] + L.rank_in_expert[t, j] - L.src_expert_off[s, e])


def pin_ll_invariants(orc):
    """Rows are distinct, inside their (expert, source) region, fill each
    region from its first row in ascending token order, and src_idx inverts
    pos."""
    rng = np.random.default_rng(62)
    T, k, E, R = 256, 8, 64, 8
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    topk[rng.random((T, k)) < 0.1] = -1
    pos, src_idx, cnt, _ = orc.ll_positions(topk, E, R)
    tpr = T // R
    kept = pos[pos >= 0]
    assert kept.size == len(set(kept.tolist())) == (topk >= 0).sum() == cnt.sum()
    for t in range(T):
        for j in range(k):
            p = pos[t, j]
            if p < 0:
                continue
            e, s = topk[t, j], t // tpr
            base = e * R * tpr + s * tpr
            assert base <= p < base + cnt[e, s] and src_idx[p] == t
    used = src_idx.reshape(E, R, tpr)
    for e in range(E):
        for s in range(R):
            toks = used[e, s, :cnt[e, s]]
            assert (toks >= s * tpr).all() and (toks < (s + 1) * tpr).all() and (np.diff(toks) > 0).all()
            assert (used[e, s, cnt[e, s]:] == -1).all()


ALL_PINS = [
    pin_e4m3_decode, pin_e4m3_encode, pin_bf16_round,
    pin_layout_golden, pin_layout_bruteforce, pin_layout_argsort, pin_layout_invariants,
    pin_dispatch_bf16, pin_fp8_golden, pin_fp8_bound, pin_fp8_torch,
    pin_combine_fp64, pin_combine_order, pin_combine_fma, pin_combine_identity, pin_backward,
    pin_dedup_golden, pin_dedup_bruteforce, pin_dedup_dispatch, pin_dedup_prereduce,
    pin_prereduce_golden, pin_prereduce_bruteforce, pin_prereduce_order_fma, pin_prereduce_fp64,
    pin_ll_golden, pin_ll_bruteforce, pin_ll_invariants,
]
