"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the same
seeded inputs. Integer, index and byte outputs (layout, positions, source
indices, FP8 codes, scales, copied rows, weights) must be bit-exact; the bf16
combine must be within 1 bf16 ulp of the oracle (same fp32 FMA order, so 0 is
expected) and its fp32 sums within 1e-6 relative (bit-exact expected)."""
import gc
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import CONFIGS, make_workload, device_normal_bf16
from gpu_helpers import (compare_bf16, compare_handle, compare_layout, compare_rows, dev, dev_bf16,
                         f32_rel_diff, gpu_forward, host, host_u16, used_rows)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback


def oracle_cap(topk, E, R):
    return int(oracle.layout(topk, E, R, 1 << 30).rank_rows.max())


def full_check(x, topk, w, E, R, cap, use_fp8, expert_out_seed=5, check_combine=True, fused=False):
    """Layout + dispatch + combine (+ f32 sums) against the oracle, every element."""
    orc = oracle.default()
    L, pos, src, rx, rs, rw = orc.forward(x, topk, w, E, R, cap, use_fp8)
    g = gpu_forward(x, topk, w, E, R, cap, use_fp8, fused=fused)
    assert g.status == L.status, (g.status, L.status)
    compare_layout(g, L)
    compare_handle(g, pos, src)
    compare_rows(g, pos, rx, rs, rw, use_fp8)
    if check_combine and x.shape[0] > 0:
        rng = np.random.default_rng(expert_out_seed)
        n = R * cap
        eo = oracle_rows = None
        from combine_get_dispatch_amd.workloads import normal_bf16
        eo = normal_bf16(rng, (max(n, 1), x.shape[1]))
        y_o, acc_o = orc.combine(eo, pos, w, return_acc=True)
        eo_d = dev_bf16(eo)
        y = host_u16(g.buf.combine(eo_d, g.handle, g.w))
        frac = compare_bf16(y, y_o, "combine")
        assert frac == 1.0, f"combine not bit-exact ({frac:.6f} exact)"
        acc = host(g.buf.combine_f32(eo_d, g.handle, g.w))
        assert f32_rel_diff(acc, acc_o) <= 1e-6
        assert np.array_equal(acc.view(np.uint32), acc_o.view(np.uint32)), "fp32 sums not bit-exact"
        # unit weights (weights = NULL)
        y1 = host_u16(g.buf.combine(eo_d, g.handle, None))
        assert np.array_equal(y1, orc.combine(eo, pos, None))
    return g, (L, pos, src, rx, rs, rw)


# ---------------------------------------------------------------------------
# the workloads, full element-wise parity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("name", ["tiny", "decode_rank", "decode", "prefill", "skewed"])
def test_forward_parity(name, fused):
    cfg = CONFIGS[name]
    wl = make_workload(cfg, seed=0)
    cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
    full_check(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, cfg.use_fp8, fused=fused)


@pytest.mark.parametrize("seed", list(range(1, 17)))
def test_forward_parity_seeds(seed):
    """Seeds 1..16 on the tiny and the 1024-token decode workloads (the
    fused launch on odd seeds, two calls on even ones)."""
    for name in ("tiny", "decode"):
        cfg = CONFIGS[name]
        wl = make_workload(cfg, seed=seed)
        cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
        full_check(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, cfg.use_fp8, expert_out_seed=seed,
                   fused=bool(seed % 2))


def test_backward_parity_small():
    cfg = replace(CONFIGS["large"], T=1024)
    wl = make_workload(cfg, seed=0)
    cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
    g, (L, pos, src, rx, rs, rw) = full_check(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, False)
    orc = oracle.default()
    n = cfg.R * cap
    gy = wl.grad_y()
    grows_o = orc.combine_backward(gy, pos, n)
    grows = g.buf.combine_backward(dev_bf16(gy), g.handle)
    rows = used_rows(pos)
    assert np.array_equal(host_u16(grows)[rows], grows_o[rows]), "combine_backward rows differ"
    G = wl.grad_rows(n)
    gx_o = orc.dispatch_backward(G, pos, wl.topk_w)
    gx = host_u16(g.buf.dispatch_backward(dev_bf16(G), g.handle, g.w))
    assert compare_bf16(gx, gx_o, "dispatch_backward") == 1.0


# ---------------------------------------------------------------------------
# full-size configs in the launch configuration the bench times: the layout
# and handle are compared entirely, then every row and every token in chunks
# ---------------------------------------------------------------------------

def chunk_rows(pos, toks):
    """The receive rows a chunk of tokens owns (sorted) and the chunk's
    positions renumbered into them (-1 kept)."""
    sub = pos[toks]
    need = used_rows(sub)
    remap = np.full(int(need.max(initial=-1)) + 1, -1, np.int64)
    remap[need] = np.arange(need.size)
    pos_c = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(np.int32)
    return need, pos_c


def chunked_checks(cfg, wl, g, pos, use_fp8, with_backward, chunk=1024):
    """Every token of the workload, a chunk at a time: its dispatch rows
    (codes and scales, or bf16 copies, and weights), its combined bf16 row
    and fp32 sums, and with the backward pair its combine_backward rows and
    dispatch_backward row. A chunk is a complete sub-problem (a row and a
    combined token depend only on their own token's inputs), so the oracle
    runs on the chunk's tokens with its positions renumbered into the rows
    the chunk owns; the chunks together cover every kept row."""
    orc = oracle.default()
    T, H = cfg.T, cfg.H
    n = cfg.R * g.buf.cap_rows
    eo = device_normal_bf16((n, H), seed=11)
    y = g.buf.combine(eo, g.handle, g.w)
    acc = g.buf.combine_f32(eo, g.handle, g.w)
    if with_backward:
        gy = device_normal_bf16((T, H), seed=12)
        grows = g.buf.combine_backward(gy, g.handle)
        G = device_normal_bf16((n, H), seed=13)
        gx = g.buf.dispatch_backward(G, g.handle, g.w)
    assert g.buf.status() == 0
    covered = 0
    for t0 in range(0, T, chunk):
        toks = np.arange(t0, min(t0 + chunk, T))
        tk = torch.from_numpy(toks).cuda()
        need, pos_c = chunk_rows(pos, toks)
        covered += need.size
        idx = torch.from_numpy(need.astype(np.int64)).cuda()
        w_c = wl.topk_w[toks]
        rx_o, rs_o, rw_o = orc.dispatch(wl.x[toks], w_c, pos_c, need.size, use_fp8)
        if use_fp8:
            got = g.recv_x.index_select(0, idx).cpu().numpy()
            assert np.array_equal(got, rx_o), f"fp8 rows of tokens {t0}.. differ"
            gs = g.recv_scales.index_select(0, idx).cpu().numpy()
            assert np.array_equal(gs.view(np.uint32), rs_o.view(np.uint32)), f"scales of tokens {t0}.. differ"
        else:
            assert np.array_equal(host_u16(g.recv_x.index_select(0, idx)), rx_o), f"bf16 rows of tokens {t0}.."
        gw = g.recv_w.index_select(0, idx).cpu().numpy()
        assert np.array_equal(gw.view(np.uint32), rw_o.view(np.uint32)), f"recv_w of tokens {t0}.."
        eo_c = host_u16(eo.index_select(0, idx))
        y_o, acc_o = orc.combine(eo_c, pos_c, w_c, return_acc=True)
        assert compare_bf16(host_u16(y.index_select(0, tk)), y_o, "combine") == 1.0
        acc_c = acc.index_select(0, tk).cpu().numpy()
        assert f32_rel_diff(acc_c, acc_o) <= 1e-6
        assert np.array_equal(acc_c.view(np.uint32), acc_o.view(np.uint32)), f"fp32 sums of tokens {t0}.."
        if with_backward:
            grows_o = orc.combine_backward(host_u16(gy.index_select(0, tk)), pos_c, need.size)
            assert np.array_equal(host_u16(grows.index_select(0, idx)), grows_o), f"combine_backward {t0}.."
            gx_o = orc.dispatch_backward(host_u16(G.index_select(0, idx)), pos_c, w_c)
            assert compare_bf16(host_u16(gx.index_select(0, tk)), gx_o, "dispatch_backward") == 1.0
        print(f"  tokens {t0}..{toks[-1]}: {need.size} rows exact", flush=True)
    assert covered == int((pos >= 0).sum())


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("name", ["prefill", "large"])
def test_full_size(name, fused):
    cfg = CONFIGS[name]
    print(f"full-size parity: {name} T={cfg.T} H={cfg.H} fused={fused}", flush=True)
    wl = make_workload(cfg, seed=0)
    orc = oracle.default()
    L = orc.layout(wl.topk_idx, cfg.E, cfg.R, 1 << 30)
    cap = int(L.rank_rows.max())
    L = orc.layout(wl.topk_idx, cfg.E, cfg.R, cap)
    pos, src = orc.positions(wl.topk_idx, L, cfg.E, cfg.R, cap)
    g = gpu_forward(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, cfg.use_fp8, fused=fused)
    assert g.status == L.status == 0
    compare_layout(g, L)
    compare_handle(g, pos, src)
    chunked_checks(cfg, wl, g, pos, cfg.use_fp8, with_backward=cfg.backward or name == "prefill")
    g.buf.close()
    del g
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def rand_routing(rng, T, k, E):
    if T == 0:
        return np.zeros((0, k), np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def case(T, k, E, R, H, fp8, seed=0, mutate=None, cap=None, cap_delta=0, fused=False):
    rng = np.random.default_rng(seed)
    topk = rand_routing(rng, T, k, E)
    if mutate is not None:
        topk = mutate(topk, rng)
    w = rng.random((T, k)).astype(np.float32)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    from combine_get_dispatch_amd.workloads import to_bf16_bits
    x = to_bf16_bits(xf)
    if cap is None:
        cap = max(oracle_cap(topk, E, R) + cap_delta, 0)
    return full_check(x, topk, w, E, R, cap, fp8, fused=fused)


EDGE = {
    "empty": dict(T=0, k=2, E=16, R=4, H=256, fp8=False),
    "empty_fp8": dict(T=0, k=8, E=256, R=8, H=7168, fp8=True),
    "ragged_tile_bf16_tail": dict(T=300, k=3, E=12, R=4, H=136, fp8=False),
    "ragged_fp8_partial_pass": dict(T=257, k=4, E=32, R=1, H=384, fp8=True),
    "one_token": dict(T=1, k=1, E=1, R=1, H=8, fp8=False),
    "k1_R1_E1_fp8": dict(T=64, k=1, E=1, R=1, H=128, fp8=True),
    "E_equals_R": dict(T=640, k=4, E=8, R=8, H=512, fp8=True),
    "k32": dict(T=96, k=32, E=64, R=16, H=256, fp8=False),
    "E1024_R64": dict(T=1024, k=8, E=1024, R=64, H=1024, fp8=True),
    "R_not_mult4": dict(T=300, k=2, E=12, R=3, H=256, fp8=False),
    "hidden_64k": dict(T=8, k=2, E=4, R=2, H=65536, fp8=True),
    "many_tiles": dict(T=65536, k=2, E=32, R=8, H=8, fp8=False),
    "tiles_exact": dict(T=512, k=8, E=256, R=8, H=1024, fp8=True),
    "ticket_tiles": dict(T=270336, k=1, E=16, R=8, H=8, fp8=False),
    "multi_tile_4_waves": dict(T=4096, k=8, E=1024, R=64, H=256, fp8=True),
    "single_tile_16_waves_ragged": dict(T=1000, k=8, E=256, R=8, H=256, fp8=False),
    # one tile whose layout does not fit beside the slots in a block's LDS
    # (the fused call then uses separate layout blocks and flags)
    "one_tile_E1024_R64": dict(T=192, k=8, E=1024, R=64, H=512, fp8=True),
    # one tile, 32 slots per token: the largest in-block slot table
    "one_tile_k32_E512": dict(T=96, k=32, E=512, R=32, H=384, fp8=True),
    "one_full_tile": dict(T=256, k=8, E=256, R=8, H=7168, fp8=True),
    # several tiles chained by look-back: a source rank per tile and a
    # ragged last tile, wide rows, the most tiles whose source boundaries
    # all fall on tile edges
    "tiles_32": dict(T=8192, k=8, E=256, R=32, H=256, fp8=True),
    "tiles_ragged": dict(T=5000, k=6, E=200, R=8, H=384, fp8=False),
    "tiles_k16": dict(T=2048, k=16, E=128, R=16, H=256, fp8=True),
    "tiles_33": dict(T=8448, k=8, E=256, R=32, H=256, fp8=True),
    # experts per rank not a power of two (division instead of a shift)
    "epr_not_pow2": dict(T=1536, k=8, E=192, R=8, H=256, fp8=True),
    # rows that end inside a wave's 1024-channel pass: the last pass holds
    # 8 channels (BF16) or one 128-channel group (FP8), so the row loads
    # beyond the row's end must read nothing and write nothing
    "bf16_row_ends_in_pass": dict(T=100, k=4, E=32, R=4, H=9224, fp8=False),
    "fp8_row_ends_in_pass": dict(T=3000, k=6, E=48, R=6, H=1152, fp8=True),
    # one tile (the in-block kernel when fused) with waves of 2, 4 and 8
    # passes: every row-load count the in-block kernel is built for
    "one_tile_2_passes_bf16": dict(T=256, k=4, E=32, R=4, H=16384, fp8=False),
    "one_tile_4_passes": dict(T=256, k=4, E=32, R=4, H=32768, fp8=True),
    "one_tile_8_passes": dict(T=256, k=2, E=16, R=4, H=65536, fp8=True),
    "one_tile_8_passes_bf16": dict(T=256, k=2, E=16, R=4, H=65536, fp8=False),
    # combines long enough to run at the residency cap (at least 64 waves
    # per CU of 256): an odd wave count (the last two-wave workgroup holds
    # one wave past the tokens) with a partial last pass, and the FP8 prefill
    # shape just above the threshold
    "capped_combine_odd_waves_tail": dict(T=2349, k=8, E=63, R=3, H=7000, fp8=False),
    "capped_combine_fp8": dict(T=2368, k=8, E=256, R=32, H=7168, fp8=True),
}


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_shapes(name, fused):
    case(**EDGE[name], fused=fused)


def test_all_slots_empty():
    case(T=128, k=4, E=16, R=4, H=256, fp8=True, mutate=lambda t, r: np.full_like(t, -1))


def test_some_slots_empty():
    def m(t, r):
        t = t.copy()
        t[r.random(t.shape) < 0.3] = -1
        return t
    case(T=512, k=8, E=64, R=8, H=1024, fp8=True, mutate=m)


def test_all_to_one_expert():
    def m(t, r):
        t = t.copy()
        t[:, 0] = 5
        t[:, 1:] = -1
        return t
    case(T=2048, k=4, E=16, R=4, H=1024, fp8=True, mutate=m)


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_capacity_and_bad_ids_fused(fused):
    def m(t, r):
        t = t.copy()
        t[3, 1] = 99
        t[5, 2] = t[5, 0]
        return t
    for T in (1024, 200):  # several tiles; one tile
        g, (L, pos, *_ ) = case(T=T, k=8, E=64, R=8, H=512, fp8=True, cap_delta=-9, mutate=m, fused=fused)
        assert L.status == ep.EP_ST_CAPACITY | ep.EP_ST_BAD_EXPERT | ep.EP_ST_DUP_EXPERT


def test_bad_and_repeated_experts():
    def m(t, r):
        t = t.copy()
        t[3, 1] = 99            # out of range
        t[4, 0] = -7            # out of range
        t[5, 2] = t[5, 0]       # repeat
        t[6, :] = t[6, 0]       # all repeats
        return t
    g, (L, *_ ) = case(T=64, k=4, E=16, R=4, H=256, fp8=False, mutate=m)
    assert L.status == ep.EP_ST_BAD_EXPERT | ep.EP_ST_DUP_EXPERT


def test_capacity_overflow_drops_rows():
    g, (L, pos, *_ ) = case(T=1024, k=8, E=64, R=8, H=512, fp8=True, cap_delta=-9)
    assert L.status == ep.EP_ST_CAPACITY and (pos < 0).sum() > 0


def test_capacity_zero():
    g, (L, pos, *_ ) = case(T=64, k=2, E=16, R=4, H=256, fp8=False, cap=0)
    assert L.status == ep.EP_ST_CAPACITY and np.all(pos < 0)


def test_skewed_capacity_limit():
    """The Zipf workload with a receive capacity below the hot rank's need."""
    cfg = replace(CONFIGS["skewed"], T=2048, H=1024)
    wl = make_workload(cfg, seed=0)
    cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
    g, (L, pos, *_ ) = full_check(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap // 2, True)
    assert L.status == ep.EP_ST_CAPACITY


# ---------------------------------------------------------------------------
# FP8 conversion over every finite bf16 pattern
# ---------------------------------------------------------------------------

def test_fp8_all_bf16_patterns():
    """Groups whose first element is the amax A and whose other 127 elements
    run through every finite bf16 value with |v| <= A, for a set of A that
    gives power-of-two and non-power-of-two scales, subnormal outputs, and the
    1e-4 floor."""
    from combine_get_dispatch_amd.workloads import to_bf16_bits
    pats = np.arange(65536, dtype=np.uint32)
    pats = pats[(pats & 0x7F80) != 0x7F80]
    vals = (pats << 16).view(np.float32)
    groups = []
    for A in [448.0, 1.0, 2.0, 3.0, 0.1, 1e-3, 5e-5, 1e4, 1e30, 7.0, -2.5]:
        a_bits = to_bf16_bits(np.array([A], np.float32))[0]
        a = abs(float((np.array([a_bits], np.uint32) << 16).view(np.float32)[0]))
        sel = pats[np.abs(vals) <= a].astype(np.uint16)
        n = (sel.size + 126) // 127
        sel = np.concatenate([sel, np.zeros(n * 127 - sel.size, np.uint16)]).reshape(n, 127)
        groups.append(np.concatenate([np.full((n, 1), a_bits, np.uint16), sel], axis=1))
    g = np.concatenate(groups)
    H = 1024
    pad = (-g.shape[0]) % (H // 128)
    g = np.concatenate([g, np.zeros((pad, 128), np.uint16)])
    x = g.reshape(-1, H)
    T = x.shape[0]
    topk = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    full_check(x, topk, w, 1, 1, T, True, check_combine=False)


# ---------------------------------------------------------------------------
# determinism, repeated calls on one context
# ---------------------------------------------------------------------------

def test_fused_and_separate_calls_interleaved():
    """Fused and two-call forwards alternate on one context (both re-arm the
    shared workspace): every call matches the oracle."""
    cfg = replace(CONFIGS["prefill"], H=1024)
    for seed in range(4):
        wl = make_workload(cfg, seed=seed)
        if seed == 0:
            cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R) + 64
            buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cap)
        L_o, pos_o, src_o, rx_o, rs_o, rw_o = oracle.default().forward(wl.x, wl.topk_idx, wl.topk_w, cfg.E,
                                                                       cfg.R, cap, True)
        x, topk, w = dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w)
        for fused in (True, False):
            if fused:
                L, rx, rs, rw, h = buf.dispatch_with_layout(x, topk, w, True)
            else:
                L = buf.get_dispatch_layout(topk)
                rx, rs, rw, h = buf.dispatch(x, topk, w, L, True)
            assert buf.status() == 0
            assert np.array_equal(host(h.pos), pos_o), (seed, fused)
            assert np.array_equal(host(L.cnt_se), L_o.cnt_se) and np.array_equal(host(L.src_expert_off),
                                                                                 L_o.src_expert_off)
            rows = torch.from_numpy(used_rows(pos_o).astype(np.int64)).cuda()
            assert np.array_equal(rx.index_select(0, rows).cpu().numpy(), rx_o[used_rows(pos_o)]), (seed, fused)


def test_repeated_layouts_on_one_context():
    """The look-back states are re-armed by each call (epochs): ten calls with
    different routing on one context each match the oracle."""
    cfg = replace(CONFIGS["decode"], T=4096, H=256)
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, 4096)
    for seed in range(10):
        wl = make_workload(cfg, seed=seed, with_x=False)
        L_o = oracle.layout(wl.topk_idx, cfg.E, cfg.R, 4096)
        L = buf.get_dispatch_layout(dev(wl.topk_idx))
        assert buf.status() == L_o.status  # 4096 rows per rank is below some ranks' need
        for key in ("rank_in_expert", "recv_cnt", "src_expert_off", "cnt_sd", "is_token_in_rank"):
            assert np.array_equal(host(getattr(L, key)), getattr(L_o, key)), (seed, key)


def test_deterministic_outputs():
    cfg = CONFIGS["skewed"]
    wl = make_workload(cfg, seed=0)
    cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
    outs = []
    for _ in range(2):
        g = gpu_forward(wl.x, wl.topk_idx, wl.topk_w, cfg.E, cfg.R, cap, True)
        eo = device_normal_bf16((cfg.R * cap, cfg.H), seed=3)
        y = g.buf.combine(eo, g.handle, g.w)
        rows = torch.from_numpy(used_rows(host(g.handle.pos)).astype(np.int64)).cuda()
        outs.append([host(g.layout.rank_in_expert), host(g.handle.pos),
                     g.recv_x.index_select(0, rows).cpu().numpy(),
                     g.recv_scales.index_select(0, rows).cpu().numpy(), host_u16(y)])
        del g
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_handle_from_other_config_rejected():
    b1 = ep.Buffer(64, 256, 2, 16, 4, 64)
    b2 = ep.Buffer(128, 256, 2, 16, 4, 64)
    h = b1.new_handle()
    h.num_tokens, h.num_topk = 64, 2
    eo = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ep.EpError) as e:
        b2.combine(eo, h)
    assert e.value.code == ep.EP_ERR_ARG
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")[:, 1:]  # misaligned rows
    topk = torch.zeros((64, 2), dtype=torch.int32, device="cuda")
    L = b1.get_dispatch_layout(topk)
    with pytest.raises(ep.EpError) as e:
        b1.dispatch(x, topk, None, L, False)
    assert e.value.code == ep.EP_ERR_ALIGN
    b1.status()


@pytest.mark.parametrize("cfg_name", ["decode_rank", "decode"])  # one tile; four tiles
@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
def test_graph_replay_matches_eager(fused, cfg_name):
    """The decode step (layout, FP8 dispatch, combine) captured in a HIP graph
    and replayed several times, with eager work and synchronizations between
    replays: every replay equals the eager result (the workspace re-arms
    itself on the device; the path records no memset)."""
    cfg = CONFIGS[cfg_name]
    wl = make_workload(cfg, seed=7)
    cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cap)
    x, topk, w = dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w)
    eo = device_normal_bf16((buf.num_rows, cfg.H), seed=8)
    L = buf.new_layout()
    out = (torch.empty((buf.num_rows, cfg.H), dtype=torch.uint8, device="cuda"),
           torch.empty((buf.num_rows, cfg.H // 128), dtype=torch.float32, device="cuda"),
           torch.empty(buf.num_rows, dtype=torch.float32, device="cuda"), buf.new_handle())
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")

    def step():
        if fused:
            buf.dispatch_with_layout(x, topk, w, True, layout=L, out=out)
        else:
            buf.get_dispatch_layout(topk, L)
            buf.dispatch(x, topk, w, L, True, out=out)
        buf.combine(eo, out[3], w, out=y)

    step()
    torch.cuda.synchronize()
    rows = torch.from_numpy(used_rows(host(out[3].pos)).astype(np.int64)).cuda()
    ref = [host(L.rank_in_expert), host(out[3].pos), out[0].index_select(0, rows).cpu().numpy(),
           out[1].index_select(0, rows).cpu().numpy(), host_u16(y)]
    gc.collect()  # no buffer of an earlier test may be released during the capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t_ in (L.rank_in_expert, out[3].pos, out[0], out[1], y):
            t_.zero_()
        _ = (eo.float() * 2).sum().item()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [host(L.rank_in_expert), host(out[3].pos), out[0].index_select(0, rows).cpu().numpy(),
               out[1].index_select(0, rows).cpu().numpy(), host_u16(y)]
        for a_, b_ in zip(got, ref):
            assert np.array_equal(a_, b_), f"replay {r} differs"
    assert buf.status() == 0


# ---------------------------------------------------------------------------
# two contexts at once: each has its own workspace, epoch and flags
# ---------------------------------------------------------------------------

def test_two_contexts_on_two_streams_concurrently():
    """Fused layout+dispatch and combine of two contexts (4 and 16 layout
    tiles) enqueued alternately on two streams, three times over: every
    output equals the same context's sequential run bit for bit, and the
    sequential handles equal the oracle's."""
    orc = oracle.default()
    shapes = [replace(CONFIGS["decode"], H=1024), replace(CONFIGS["prefill"], H=512)]
    runs = []
    for i, cfg in enumerate(shapes):
        wl = make_workload(cfg, seed=30 + i)
        cap = oracle_cap(wl.topk_idx, cfg.E, cfg.R)
        L = orc.layout(wl.topk_idx, cfg.E, cfg.R, cap)
        pos_o, src_o = orc.positions(wl.topk_idx, L, cfg.E, cfg.R, cap)
        buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cap)
        x, topk, w = dev_bf16(wl.x), dev(wl.topk_idx), dev(wl.topk_w)
        eo = device_normal_bf16((buf.num_rows, cfg.H), seed=40 + i)
        layout, rx, rs, rw, h = buf.dispatch_with_layout(x, topk, w, cfg.use_fp8)
        y = buf.combine(eo, h, w)
        # the reference: the same calls on zeroed outputs (rows no slot maps
        # to are never written, so they keep what the buffer held)
        rx.zero_()
        y.zero_()
        buf.dispatch_with_layout(x, topk, w, cfg.use_fp8, layout=layout, out=(rx, rs, rw, h))
        buf.combine(eo, h, w, out=y)
        torch.cuda.synchronize()
        assert np.array_equal(host(h.pos), pos_o)
        ref = [t.clone() for t in (rx, h.pos, y)]
        runs.append(dict(cfg=cfg, buf=buf, x=x, topk=topk, w=w, eo=eo, layout=layout,
                         out=(rx, rs, rw, h), y=y, ref=ref))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for r in runs:
            r["out"][0].zero_()
            r["y"].zero_()
        torch.cuda.synchronize()
        for r, s_ in zip(runs, streams):
            with torch.cuda.stream(s_):
                r["buf"].dispatch_with_layout(r["x"], r["topk"], r["w"], r["cfg"].use_fp8, layout=r["layout"],
                                              out=r["out"])
        for r, s_ in zip(runs, streams):
            with torch.cuda.stream(s_):
                r["buf"].combine(r["eo"], r["out"][3], r["w"], out=r["y"])
        torch.cuda.synchronize()
        for r in runs:
            got = (r["out"][0], r["out"][3].pos, r["y"])
            for a_, b_ in zip(got, r["ref"]):
                assert torch.equal(a_, b_)
    for r in runs:
        assert r["buf"].status() == 0
