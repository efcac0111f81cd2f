"""Guard canaries: every output buffer of every call sits between two 4 KB
guard bands filled with a byte pattern, and the receive buffers start out
filled with it too. After each call the bands must be intact, and so must
every receive row (and its scales, weight, source index, routing entries)
that no slot maps to: the kernels write nothing outside the rows the layout
assigns, also when rows are dropped for capacity or ids are bad. The values
written are checked against the oracle by the parity tests; here only where
the writes land is checked."""
import numpy as np
import pytest
import torch

import oracle
from combine_get_dispatch_amd import ep
from combine_get_dispatch_amd.workloads import to_bf16_bits
from gpu_helpers import dev, dev_bf16, host, used_rows

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback

PAD = 4096
FILL = 0xAB


class Guarded:
    """A tensor of `shape`/`dtype` inside a byte buffer whose PAD bytes on
    each side (and the tensor itself, initially) hold FILL."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((PAD + n + PAD,), FILL, dtype=torch.uint8, device="cuda")
        self.n = n
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def check_bands(self, what):
        torch.cuda.synchronize()
        lo = self.raw[:PAD].cpu().numpy()
        hi = self.raw[PAD + self.n:].cpu().numpy()
        assert (lo == FILL).all(), f"{what}: write below the buffer"
        assert (hi == FILL).all(), f"{what}: write above the buffer"

    def untouched_rows(self, rows_used, nrows, what):
        """Rows of a [nrows, ...] buffer not in rows_used still hold FILL."""
        b = self.raw[PAD:PAD + self.n].cpu().numpy().reshape(nrows, -1)
        mask = np.ones(nrows, bool)
        mask[rows_used] = False
        assert (b[mask] == FILL).all(), f"{what}: a row no slot maps to was written"


def routing(T, k, E, seed, bad=False):
    rng = np.random.default_rng(seed)
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    topk[rng.random((T, k)) < 0.1] = -1
    if bad:
        topk[3 % T, 0] = E + 7
        if k > 1:
            topk[5 % T, 1] = topk[5 % T, 0] if topk[5 % T, 0] >= 0 else 0
    return topk, rng.random((T, k)).astype(np.float32), rng


def guarded_layout(T, k, E, R, dedup=False):
    g = {n: Guarded(s, d) for n, s, d in (
        ("cnt_se", (R, E), torch.int32), ("cnt_sd", (R, R), torch.int32), ("recv_cnt", (E,), torch.int32),
        ("expert_off", (E,), torch.int32), ("rank_rows", (R,), torch.int32), ("src_expert_off", (R, E), torch.int32),
        ("rank_in_expert", (T, k), torch.int32), ("is_token_in_rank", (T, R), torch.uint8))}
    if dedup:
        g["rank_in_rank"] = Guarded((T, k), torch.int32)
        g["token_rows"] = Guarded((R,), torch.int32)
    L = ep.Layout(*[g[n].t for n in ("cnt_se", "cnt_sd", "recv_cnt", "expert_off", "rank_rows", "src_expert_off",
                                     "rank_in_expert", "is_token_in_rank")],
                  g["rank_in_rank"].t if dedup else None, g["token_rows"].t if dedup else None)
    return L, g


CASES = [  # T, k, E, R, H, fp8, cap_delta, bad
    (128, 8, 256, 8, 1024, True, 0, False),     # one tile: in-block fused kernel
    (1024, 8, 64, 8, 512, True, -9, True),      # four tiles, capacity drops, bad ids
    (4096, 8, 256, 32, 256, True, 0, False),    # sixteen tiles: fused with flags
    (5120, 6, 60, 4, 136, False, -20, True),    # beyond 16 tiles: two launches; BF16 with a channel tail
    (100, 4, 32, 4, 9224, False, 0, False),     # BF16 rows ending 8 channels into a pass
]


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_k{c[1]}_E{c[2]}_R{c[3]}" for c in CASES])
def test_per_expert_path_writes_only_its_rows(case, fused):
    T, k, E, R, H, fp8, cap_delta, bad = case
    topk, w, rng = routing(T, k, E, 1, bad)
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    orc = oracle.default()
    cap = max(int(orc.layout(topk, E, R, 1 << 30).rank_rows.max()) + cap_delta, 1)
    buf = ep.Buffer(T, H, k, E, R, cap)
    n = R * cap
    L, gl = guarded_layout(T, k, E, R)
    rx = Guarded((n, H), torch.uint8 if fp8 else torch.bfloat16)
    rs = Guarded((n, H // 128), torch.float32) if fp8 else None
    rw = Guarded((n,), torch.float32)
    pos = Guarded((T, k), torch.int32)
    src = Guarded((n,), torch.int32)
    h = ep.Handle(pos.t, src.t)
    out = (rx.t, rs.t if fp8 else None, rw.t, h)
    td, wd, xd = dev(topk), dev(w), dev_bf16(x)
    if fused:
        buf.dispatch_with_layout(xd, td, wd, fp8, layout=L, out=out)
    else:
        buf.get_dispatch_layout(td, L)
        buf.dispatch(xd, td, wd, L, fp8, out=out)
    st = buf.status()
    for name, gg in gl.items():
        gg.check_bands(f"layout.{name}")
    pos_h = host(h.pos)
    rows = used_rows(pos_h)
    for what, gg in (("recv_x", rx), ("recv_scales", rs), ("recv_w", rw), ("src_idx", src)):
        if gg is None:
            continue
        gg.check_bands(what)
        gg.untouched_rows(rows, n, what)
    pos.check_bands("pos")
    if bad:
        assert st & (ep.EP_ST_BAD_EXPERT | ep.EP_ST_DUP_EXPERT)
    if cap_delta < 0:
        assert st & ep.EP_ST_CAPACITY and (pos_h < 0).sum() > (topk < 0).sum()
    # combine, its fp32 form and the backward pair on the same handle
    eo = torch.randn((n, H), device="cuda").to(torch.bfloat16)
    y = Guarded((T, H), torch.bfloat16)
    buf.combine(eo, h, wd, out=y.t)
    y.check_bands("combined_x")
    yf = Guarded((T, H), torch.float32)
    buf.combine_f32(eo, h, wd, out=yf.t)
    yf.check_bands("combined_f32")
    gr = Guarded((n, H), torch.bfloat16)
    buf.combine_backward(xd, h, out=gr.t)
    gr.check_bands("grad_rows")
    gr.untouched_rows(rows, n, "grad_rows")
    gx = Guarded((T, H), torch.bfloat16)
    buf.dispatch_backward(eo, h, wd, out=gx.t)
    gx.check_bands("grad_x")
    assert buf.status() == 0


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("T", [256, 1024, 5120])
def test_dedup_path_writes_only_its_rows(T, fused):
    k, E, R, H, fp8 = 8, 64, 8, 256, True
    topk, w, rng = routing(T, k, E, 2, bad=True)
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    _, trows, _ = oracle.default().layout_dedup(topk, E, R, 1 << 30)
    cap = int(trows.max()) - 3  # some rows dropped
    buf = ep.Buffer(T, H, k, E, R, cap)
    n = R * cap
    L, gl = guarded_layout(T, k, E, R, dedup=True)
    rx, rs = Guarded((n, H), torch.uint8), Guarded((n, H // 128), torch.float32)
    rti, rtw = Guarded((n, k), torch.int32), Guarded((n, k), torch.float32)
    pos, src = Guarded((T, k), torch.int32), Guarded((n,), torch.int32)
    h = ep.Handle(pos.t, src.t)
    out = (rx.t, rs.t, rti.t, rtw.t, h)
    td, wd, xd = dev(topk), dev(w), dev_bf16(x)
    if fused:
        buf.dispatch_dedup_with_layout(xd, td, wd, fp8, layout=L, out=out)
    else:
        buf.get_dispatch_layout(td, L)
        buf.dispatch_dedup(xd, td, wd, L, fp8, out=out)
    st = buf.status()
    assert st & ep.EP_ST_CAPACITY
    for name, gg in gl.items():
        gg.check_bands(f"layout.{name}")
    rows = used_rows(host(h.pos))
    for what, gg in (("recv_x", rx), ("recv_scales", rs), ("recv_topk_idx", rti), ("recv_topk_w", rtw),
                     ("src_idx", src)):
        gg.check_bands(what)
        gg.untouched_rows(rows, n, what)
    pos.check_bands("pos")


@pytest.mark.parametrize("T", [64, 1024])
def test_low_latency_path_writes_only_its_rows(T):
    k, E, R, H = 8, 64, 8, 512
    topk, w, rng = routing(T, k, E, 3, bad=True)
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    buf = ep.Buffer(T, H, k, E, R, ep.ll_cap_rows(T, E, R))
    n = buf.num_rows
    rx, rs, rw = Guarded((n, H), torch.uint8), Guarded((n, H // 128), torch.float32), Guarded((n,), torch.float32)
    cnt = Guarded((E, R), torch.int32)
    pos, src = Guarded((T, k), torch.int32), Guarded((n,), torch.int32)
    h = ep.Handle(pos.t, src.t)
    buf.dispatch_low_latency(dev_bf16(x), dev(topk), dev(w), True, out=(rx.t, rs.t, rw.t, cnt.t, h))
    assert buf.status() & ep.EP_ST_BAD_EXPERT
    rows = used_rows(host(h.pos))
    for what, gg in (("recv_x", rx), ("recv_scales", rs), ("recv_w", rw), ("src_idx", src)):
        gg.check_bands(what)
        gg.untouched_rows(rows, n, what)
    cnt.check_bands("recv_count")
    pos.check_bands("pos")
