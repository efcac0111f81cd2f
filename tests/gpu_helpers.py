"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, bring results back, compare with the
oracle. Nothing here computes any step of the method."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from combine_get_dispatch_amd import ep


def dev_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place (sign-magnitude ordering, +0 == -0)."""
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def f32_rel_diff(a: np.ndarray, b: np.ndarray) -> float:
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    den = np.maximum(np.abs(b), 1e-30)
    return float((np.abs(a - b) / den).max()) if a.size else 0.0


LAYOUT_KEYS = ("cnt_se", "cnt_sd", "recv_cnt", "expert_off", "rank_rows", "src_expert_off",
               "rank_in_expert", "is_token_in_rank")


@dataclass
class GpuForward:
    buf: ep.Buffer
    layout: ep.Layout
    recv_x: torch.Tensor
    recv_scales: Optional[torch.Tensor]
    recv_w: torch.Tensor
    handle: ep.Handle
    status: int
    topk: torch.Tensor
    w: torch.Tensor


def gpu_forward(x_u16, topk_idx, topk_w, E, R, cap_rows, use_fp8, x_dev=None, fused=False) -> GpuForward:
    """Layout + dispatch through the C ABI: two calls, or the fused one."""
    T, k = topk_idx.shape
    H = x_u16.shape[1] if x_dev is None else x_dev.shape[1]
    buf = ep.Buffer(T, H, k, E, R, cap_rows)
    topk = dev(topk_idx.astype(np.int32))
    w = dev(topk_w.astype(np.float32))
    x = x_dev if x_dev is not None else dev_bf16(x_u16)
    if fused:
        L, recv_x, rs, rw, h = buf.dispatch_with_layout(x, topk, w, use_fp8)
    else:
        L = buf.get_dispatch_layout(topk)
        recv_x, rs, rw, h = buf.dispatch(x, topk, w, L, use_fp8)
    st = buf.status()
    return GpuForward(buf, L, recv_x, rs, rw, h, st, topk, w)


def compare_layout(g: GpuForward, o) -> None:
    for key in LAYOUT_KEYS:
        got = host(getattr(g.layout, key))
        want = getattr(o, key)
        assert got.shape == want.shape, key
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            raise AssertionError(f"layout.{key} differs at {bad[:5].tolist()} "
                                 f"(gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]})")


def compare_handle(g: GpuForward, pos_o: np.ndarray, src_o: np.ndarray) -> None:
    pos = host(g.handle.pos)
    assert np.array_equal(pos, pos_o), f"pos differs at {np.argwhere(pos != pos_o)[:5].tolist()}"
    used = src_o >= 0
    src = host(g.handle.src_idx)
    assert np.array_equal(src[used], src_o[used]), "src_idx differs on kept rows"


def used_rows(pos: np.ndarray) -> np.ndarray:
    p = pos.reshape(-1)
    return np.unique(p[p >= 0])


def compare_rows(g: GpuForward, pos_o, recv_x_o, recv_scales_o, recv_w_o, use_fp8) -> None:
    rows = used_rows(pos_o)
    if rows.size == 0:
        return
    idx = torch.from_numpy(rows).cuda()
    if use_fp8:
        got = g.recv_x.index_select(0, idx).cpu().numpy()
        want = recv_x_o[rows]
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            r, c = bad[0]
            raise AssertionError(f"fp8 rows differ at {len(bad)} places, first row {rows[r]} ch {c}: "
                                 f"gpu {got[r, c]:#04x} oracle {want[r, c]:#04x}")
        gs = g.recv_scales.index_select(0, idx).cpu().numpy()
        assert np.array_equal(gs.view(np.uint32), recv_scales_o[rows].view(np.uint32)), "scales differ"
    else:
        got = host_u16(g.recv_x.index_select(0, idx))
        assert np.array_equal(got, recv_x_o[rows]), "bf16 rows differ"
    gw = g.recv_w.index_select(0, idx).cpu().numpy()
    assert np.array_equal(gw.view(np.uint32), recv_w_o[rows].view(np.uint32)), "recv_w differs"


def compare_bf16(got: np.ndarray, want: np.ndarray, what: str, max_ulp: int = 1) -> float:
    """<= max_ulp bf16 ulps everywhere (the arithmetic is the same, so 0 is
    expected); returns the fraction of bit-exact elements."""
    d = bf16_ulp_diff(got, want)
    assert d.max(initial=0) <= max_ulp, f"{what}: {int(d.max())} ulp at {np.argwhere(d == d.max())[:3].tolist()}"
    return float((d == 0).mean()) if d.size else 1.0
