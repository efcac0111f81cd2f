"""The no-allocation entry point, ep_dispatch_with_layout_noalloc (its
workspace is a static device array), against ep_dispatch_with_layout on the
same inputs: layout, handle, received rows, scales and weights bit for bit.
Several calls in a row share the static array, each smaller or larger than
the last (the fused grid with flags, the in-block grid, the two-launch form
beyond sixteen tiles); the status bits go to the caller's word; a workload
whose workspace exceeds the array is refused before any launch."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import CONFIGS, make_workload
from gpu_helpers import LAYOUT_KEYS, dev, dev_bf16, host, used_rows

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback


def outputs(T, k, E, R, H, cap, fp8):
    """Caller-owned layout, handle and receive buffers (torch allocations)."""
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    n = R * cap
    L = ep.Layout(e((R, E), torch.int32), e((R, R), torch.int32), e(E, torch.int32), e(E, torch.int32),
                  e(R, torch.int32), e((R, E), torch.int32), e((T, k), torch.int32), e((T, R), torch.uint8))
    rx = e((n, H), torch.uint8 if fp8 else torch.bfloat16)
    rs = e((n, H // 128), torch.float32) if fp8 else None
    rw = e(n, torch.float32)
    h = ep.Handle(e((T, k), torch.int32), e(n, torch.int32))
    return L, rx, rs, rw, h


def noalloc_call(cfg, x, topk, w, fp8, out, status):
    L, rx, rs, rw, h = out
    ch = h.c()
    ep.ep_dispatch_with_layout_noalloc(cfg, x.data_ptr(), topk.data_ptr(), w.data_ptr(), L.c(), int(fp8),
                                       rx.data_ptr(), None if rs is None else rs.data_ptr(), rw.data_ptr(), ch,
                                       None if status is None else status.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    h.num_tokens, h.num_topk = ch.num_tokens, ch.num_topk


def compare(ref, got, fp8):
    (L0, rx0, rs0, rw0, h0), (L1, rx1, rs1, rw1, h1) = ref, got
    for key in LAYOUT_KEYS:
        assert torch.equal(getattr(L0, key), getattr(L1, key)), key
    assert torch.equal(h0.pos, h1.pos), "pos"
    rows = torch.from_numpy(used_rows(host(h0.pos)).astype(np.int64)).cuda()
    assert torch.equal(h0.src_idx.index_select(0, rows), h1.src_idx.index_select(0, rows)), "src_idx"
    a, b = rx0.index_select(0, rows), rx1.index_select(0, rows)
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "rows"
    if fp8:
        assert torch.equal(rs0.index_select(0, rows).view(torch.int32), rs1.index_select(0, rows).view(torch.int32))
    assert torch.equal(rw0.index_select(0, rows).view(torch.int32), rw1.index_select(0, rows).view(torch.int32))


def one_case(name, T=None, seed=0, bad=False, **over):
    cfg = CONFIGS[name] if T is None else replace(CONFIGS[name], T=T)
    cfg = replace(cfg, **over)
    print(f"no-alloc vs context: {name} T={cfg.T} H={cfg.H} fp8={cfg.use_fp8} bad={bad}", flush=True)
    wl = make_workload(cfg, seed=seed)
    topk_h = wl.topk_idx.copy()
    if bad:
        topk_h[::97, 0] = cfg.E + 3  # ids outside [-1, E): dropped, EP_ST_BAD_EXPERT
    x, topk, w = dev_bf16(wl.x), dev(topk_h), dev(wl.topk_w)
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, 1)
    L0 = buf.get_dispatch_layout(topk)
    cap = int(host(L0.rank_rows).max())
    buf.close()
    buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cap)
    ref = outputs(cfg.T, cfg.k, cfg.E, cfg.R, cfg.H, cap, cfg.use_fp8)
    L, rx, rs, rw, h = ref
    buf.dispatch_with_layout(x, topk, w, cfg.use_fp8, layout=L, out=(rx, rs, rw, h))
    st_ref = buf.status()
    got = outputs(cfg.T, cfg.k, cfg.E, cfg.R, cfg.H, cap, cfg.use_fp8)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    noalloc_call(buf.cfg, x, topk, w, cfg.use_fp8, got, status)
    torch.cuda.synchronize()
    assert int(status.item()) == st_ref, (int(status.item()), st_ref)
    assert (st_ref != 0) == bad
    compare(ref, got, cfg.use_fp8)
    buf.close()


def test_noalloc_matches_context_calls_in_a_row():
    # 4096 tokens (16 tiles, fused grid with flags), then smaller and larger
    # inputs on the same static array: 1024 tokens (4 tiles), 128 tokens (one
    # tile, in-block grid), 8192 BF16 tokens (32 tiles: two launches), bad
    # ids (status into the caller's word), 1024 experts on 64 ranks, the
    # skewed routing, and 4096 tokens again
    one_case("prefill")
    one_case("decode")
    one_case("decode_rank")
    one_case("large", T=8192)
    one_case("decode", seed=3, bad=True)
    one_case("decode", E=1024, R=64)  # more keys per tile: the states indexed differently
    one_case("skewed")
    one_case("prefill", seed=1)


def test_noalloc_refuses_beyond_static_workspace():
    cfg = ep.EpConfig(1 << 22, 8, 256, 32, 7168, 0, 1 << 20)  # about 16K tiles: 37 MB of look-back states
    L = ep.load()
    assert L.ep_dispatch_with_layout_noalloc(cfg, None, None, None, None, 1, None, None, None, None, None,
                                             None) == ep.EP_ERR_SCRATCH
