"""CPU oracle for the MoE dispatch/combine hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or runs anything under ``oracle/``.

The arithmetic lives in ``ep_oracle.c`` (plain single-threaded C, built with
gcc); this module only marshals numpy arrays in and out of it. See the header
comment of ``ep_oracle.c`` for what each step computes and which page passage
or reading it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_HDR = os.path.join(_HERE, "ep_oracle.h")
_LIB = os.path.join(_HERE, "libep_oracle.so")

ST_BAD_EXPERT = 1
ST_DUP_EXPERT = 2
ST_CAPACITY = 4

_default = None


def _compile(src: str, out: str) -> None:
    """gcc -O2 with contraction off: every multiply and add stays as written
    (fmaf() is the only fused operation, and it is called explicitly)."""
    tmp = f"{out}.{os.getpid()}.tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = False) -> str:
    """Compile ep_oracle.c into oracle/libep_oracle.so (in-tree) if stale."""
    stale = (not os.path.exists(_LIB)) or any(
        os.path.getmtime(p) > os.path.getmtime(_LIB) for p in (_SRC, _HDR))
    if force or stale:
        _compile(_SRC, _LIB)
    return _LIB


def _bind(lib):
    P = ctypes.c_void_p
    i = ctypes.c_int
    ll = ctypes.c_longlong
    lib.oracle_layout.restype = ctypes.c_uint32
    lib.oracle_layout.argtypes = [i, i, i, i, ll, P, P, P, P, P, P, P, P, P]
    lib.oracle_positions.restype = None
    lib.oracle_positions.argtypes = [i, i, i, i, ll, P, P, P, P, P]
    lib.oracle_dispatch.restype = None
    lib.oracle_dispatch.argtypes = [i, i, i, i, P, P, P, P, i, P, P, P]
    lib.oracle_quantize_token.restype = None
    lib.oracle_quantize_token.argtypes = [i, P, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [i, i, i, P, P, P, P, i, P, P]
    lib.oracle_combine_backward.restype = None
    lib.oracle_combine_backward.argtypes = [i, i, i, P, P, P]
    lib.oracle_layout_dedup.restype = ctypes.c_uint32
    lib.oracle_layout_dedup.argtypes = [i, i, i, i, ll, P, P, P]
    lib.oracle_positions_dedup.restype = None
    lib.oracle_positions_dedup.argtypes = [i, i, i, i, ll, P, P, P, P]
    lib.oracle_ll_positions.restype = ctypes.c_uint32
    lib.oracle_ll_positions.argtypes = [i, i, i, i, P, P, P, P]
    lib.oracle_prereduce.restype = None
    lib.oracle_prereduce.argtypes = [i, ll, i, i, ll, ll, P, P, P, P, P, P]
    lib.oracle_dispatch_dedup.restype = None
    lib.oracle_dispatch_dedup.argtypes = [i, i, i, i, i, i, P, P, P, P, P, i, P, P, P, P]
    for name in ("oracle_e4m3_encode", "oracle_e4m3_decode", "oracle_bf16_round"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [P, P, ll]
    return lib


def _load() -> "Oracle":
    global _default
    if _default is None:
        _default = Oracle(_bind(ctypes.CDLL(build())))
    return _default


def build_variant(source_text: str, workdir: str) -> "Oracle":
    """Compile a modified copy of ep_oracle.c (used by the tests that plant a
    mistake in the oracle and check that the pins catch it)."""
    src = os.path.join(workdir, "ep_oracle_variant.c")
    out = os.path.join(workdir, "libep_oracle_variant.so")
    with open(src, "w") as f:
        f.write(source_text)
    _compile(src, out)
    return Oracle(_bind(ctypes.CDLL(out)))


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def bf16_to_f32(h) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Layout:
    cnt_se: np.ndarray            # [R, E] int32
    cnt_sd: np.ndarray            # [R, R] int32
    recv_cnt: np.ndarray          # [E] int32
    expert_off: np.ndarray        # [E] int32, rank-local
    rank_rows: np.ndarray         # [R] int32
    src_expert_off: np.ndarray    # [R, E] int32
    rank_in_expert: np.ndarray    # [T, k] int32
    is_token_in_rank: np.ndarray  # [T, R] uint8
    status: int


class Oracle:
    """numpy front end of one compiled copy of ep_oracle.c."""

    def __init__(self, lib):
        self.lib = lib

    # -- number formats ----------------------------------------------------
    def e4m3_encode(self, v) -> np.ndarray:
        v = _c(v, np.float32)
        out = np.empty(v.shape, np.uint8)
        self.lib.oracle_e4m3_encode(_ptr(v), _ptr(out), v.size)
        return out

    def e4m3_decode(self, c) -> np.ndarray:
        c = _c(c, np.uint8)
        out = np.empty(c.shape, np.float32)
        self.lib.oracle_e4m3_decode(_ptr(c), _ptr(out), c.size)
        return out

    def bf16_round(self, v) -> np.ndarray:
        """float32 -> bf16 bit patterns (uint16), round to nearest even."""
        v = _c(v, np.float32)
        out = np.empty(v.shape, np.uint16)
        self.lib.oracle_bf16_round(_ptr(v), _ptr(out), v.size)
        return out

    # -- the hot path ------------------------------------------------------
    def layout(self, topk_idx: np.ndarray, E: int, R: int, cap_rows: int) -> Layout:
        topk_idx = _c(topk_idx, np.int32)
        T, k = topk_idx.shape
        assert E % R == 0 and T % R == 0
        L = Layout(
            cnt_se=np.zeros((R, E), np.int32), cnt_sd=np.zeros((R, R), np.int32),
            recv_cnt=np.zeros(E, np.int32), expert_off=np.zeros(E, np.int32),
            rank_rows=np.zeros(R, np.int32), src_expert_off=np.zeros((R, E), np.int32),
            rank_in_expert=np.zeros((T, k), np.int32),
            is_token_in_rank=np.zeros((T, R), np.uint8), status=0)
        L.status = int(self.lib.oracle_layout(
            T, k, E, R, int(cap_rows), _ptr(topk_idx), _ptr(L.cnt_se), _ptr(L.cnt_sd),
            _ptr(L.recv_cnt), _ptr(L.expert_off), _ptr(L.rank_rows),
            _ptr(L.src_expert_off), _ptr(L.rank_in_expert), _ptr(L.is_token_in_rank)))
        return L

    def positions(self, topk_idx: np.ndarray, L: Layout, E: int, R: int, cap_rows: int):
        """Returns (pos [T,k] int32, src_idx [R*cap_rows] int32, -1 where unused)."""
        topk_idx = _c(topk_idx, np.int32)
        T, k = topk_idx.shape
        pos = np.empty((T, k), np.int32)
        src_idx = np.full(R * int(cap_rows), -1, np.int32)
        self.lib.oracle_positions(T, k, E, R, int(cap_rows), _ptr(topk_idx),
                                  _ptr(_c(L.rank_in_expert, np.int32)),
                                  _ptr(_c(L.expert_off, np.int32)), _ptr(pos), _ptr(src_idx))
        return pos, src_idx

    def quantize_token(self, x_row: np.ndarray):
        x_row = _c(x_row, np.uint16)
        H = x_row.shape[0]
        q = np.empty(H, np.uint8)
        s = np.empty(H // 128, np.float32)
        self.lib.oracle_quantize_token(H, _ptr(x_row), _ptr(q), _ptr(s))
        return q, s

    def dispatch(self, x: np.ndarray, topk_w: Optional[np.ndarray], pos: np.ndarray,
                 num_rows: int, use_fp8: bool, tokens: Optional[np.ndarray] = None):
        """Returns (recv_x, recv_scales or None, recv_w); rows no slot maps to stay 0."""
        x = _c(x, np.uint16)
        T, H = x.shape
        pos = _c(pos, np.int32)
        k = pos.shape[1]
        G = H // 128
        recv_x = np.zeros((num_rows, H), np.uint8 if use_fp8 else np.uint16)
        recv_scales = np.zeros((num_rows, G), np.float32) if use_fp8 else None
        recv_w = np.zeros(num_rows, np.float32)
        tw = None if topk_w is None else _c(topk_w, np.float32)
        tk = None if tokens is None else _c(tokens, np.int32)
        self.lib.oracle_dispatch(T, k, H, int(bool(use_fp8)), _ptr(x), _ptr(tw), _ptr(pos),
                                 _ptr(tk), 0 if tk is None else tk.size,
                                 _ptr(recv_x), _ptr(recv_scales), _ptr(recv_w))
        return recv_x, recv_scales, recv_w

    def combine(self, rows: np.ndarray, pos: np.ndarray, w: Optional[np.ndarray],
                tokens: Optional[np.ndarray] = None, return_acc: bool = False):
        """Returns y [T or len(tokens), H] uint16 (and the fp32 sums if asked)."""
        rows = _c(rows, np.uint16)
        pos = _c(pos, np.int32)
        T, k = pos.shape
        H = rows.shape[1]
        tk = None if tokens is None else _c(tokens, np.int32)
        n = T if tk is None else tk.size
        y = np.empty((n, H), np.uint16)
        acc = np.empty((n, H), np.float32) if return_acc else None
        ww = None if w is None else _c(w, np.float32)
        self.lib.oracle_combine(T, k, H, _ptr(rows), _ptr(pos), _ptr(ww), _ptr(tk),
                                0 if tk is None else tk.size, _ptr(y), _ptr(acc))
        return (y, acc) if return_acc else y

    def combine_backward(self, grad_y: np.ndarray, pos: np.ndarray, num_rows: int) -> np.ndarray:
        grad_y = _c(grad_y, np.uint16)
        pos = _c(pos, np.int32)
        T, H = grad_y.shape
        k = pos.shape[1]
        out = np.zeros((num_rows, H), np.uint16)
        self.lib.oracle_combine_backward(T, k, H, _ptr(grad_y), _ptr(pos), _ptr(out))
        return out

    def dispatch_backward(self, grad_rows: np.ndarray, pos: np.ndarray,
                          w: Optional[np.ndarray], tokens: Optional[np.ndarray] = None):
        return self.combine(grad_rows, pos, w, tokens=tokens)

    # -- the rank-deduplicated exchange ------------------------------------
    def layout_dedup(self, topk_idx: np.ndarray, E: int, R: int, cap_rows: int):
        """Returns (rank_in_rank [T,k] int32, token_rows [R] int32, status)."""
        topk_idx = _c(topk_idx, np.int32)
        T, k = topk_idx.shape
        assert E % R == 0 and T % R == 0
        rir = np.empty((T, k), np.int32)
        rows = np.zeros(R, np.int32)
        st = int(self.lib.oracle_layout_dedup(T, k, E, R, int(cap_rows), _ptr(topk_idx), _ptr(rir), _ptr(rows)))
        return rir, rows, st

    def ll_positions(self, topk_idx: np.ndarray, E: int, R: int):
        """Low-latency receive layout. Returns (pos [T,k], src_idx [E*T],
        recv_count [E,R], status); the rows themselves come from dispatch()
        with these positions."""
        topk_idx = _c(topk_idx, np.int32)
        T, k = topk_idx.shape
        assert E % R == 0 and T % R == 0
        pos = np.empty((T, k), np.int32)
        src_idx = np.empty(E * T, np.int32)
        cnt = np.empty((E, R), np.int32)
        st = int(self.lib.oracle_ll_positions(T, k, E, R, _ptr(topk_idx), _ptr(pos), _ptr(src_idx), _ptr(cnt)))
        return pos, src_idx, cnt, st

    def positions_dedup(self, topk_idx: np.ndarray, rank_in_rank: np.ndarray, E: int, R: int, cap_rows: int):
        """Returns (pos [T,k] int32, src_idx [R*cap_rows] int32, -1 where unused)."""
        topk_idx = _c(topk_idx, np.int32)
        T, k = topk_idx.shape
        pos = np.empty((T, k), np.int32)
        src_idx = np.full(R * int(cap_rows), -1, np.int32)
        self.lib.oracle_positions_dedup(T, k, E, R, int(cap_rows), _ptr(topk_idx),
                                        _ptr(_c(rank_in_rank, np.int32)), _ptr(pos), _ptr(src_idx))
        return pos, src_idx

    def dispatch_dedup(self, x: np.ndarray, topk_idx: np.ndarray, topk_w: Optional[np.ndarray],
                       pos: np.ndarray, E: int, R: int, num_rows: int, use_fp8: bool,
                       tokens: Optional[np.ndarray] = None):
        """Returns (recv_x, recv_scales or None, recv_topk_idx, recv_topk_w); rows
        no slot maps to stay 0 (recv_topk_idx -1)."""
        x = _c(x, np.uint16)
        topk_idx = _c(topk_idx, np.int32)
        T, H = x.shape
        k = topk_idx.shape[1]
        G = H // 128
        recv_x = np.zeros((num_rows, H), np.uint8 if use_fp8 else np.uint16)
        recv_scales = np.zeros((num_rows, G), np.float32) if use_fp8 else None
        rti = np.full((num_rows, k), -1, np.int32)
        rtw = np.zeros((num_rows, k), np.float32)
        tw = None if topk_w is None else _c(topk_w, np.float32)
        tk = None if tokens is None else _c(tokens, np.int32)
        self.lib.oracle_dispatch_dedup(T, k, H, E, R, int(bool(use_fp8)), _ptr(x), _ptr(topk_idx), _ptr(tw),
                                       _ptr(_c(pos, np.int32)), _ptr(tk), 0 if tk is None else tk.size,
                                       _ptr(recv_x), _ptr(recv_scales), _ptr(rti), _ptr(rtw))
        return recv_x, recv_scales, rti, rtw

    # sentinel left in the rows the pre-reduction does not use (a NaN pattern
    # that no bf16 rounding produces: quiet NaNs come out as 0x7fc0 | payload)
    UNUSED_ROW = 0x7FBF

    def prereduce(self, expert_out: np.ndarray, recv_topk_idx: np.ndarray, recv_topk_w: Optional[np.ndarray],
                  token_rows: np.ndarray, R: int, cap_rows: int, row_lo: int = 0, row_hi: Optional[int] = None,
                  return_acc: bool = False):
        """Expert-side pre-reduction of deduplicated rows [row_lo, row_hi)
        (default: all R*cap_rows). expert_out: [rows, k, H] bf16 bits for
        those rows; recv_topk_idx / recv_topk_w: [rows, k]. Returns reduced
        [rows, H] (UNUSED_ROW in rows that are not used) and, if asked, the
        fp32 sums (NaN in unused rows)."""
        row_hi = R * cap_rows if row_hi is None else row_hi
        n = row_hi - row_lo
        expert_out = _c(expert_out, np.uint16)
        k, H = expert_out.shape[1], expert_out.shape[2]
        assert expert_out.shape[0] == n
        rti = _c(recv_topk_idx, np.int32)
        assert rti.shape == (n, k)
        rtw = None if recv_topk_w is None else _c(recv_topk_w, np.float32)
        tr = _c(token_rows, np.int32)
        reduced = np.full((n, H), self.UNUSED_ROW, np.uint16)
        acc = np.full((n, H), np.nan, np.float32) if return_acc else None
        self.lib.oracle_prereduce(R, int(cap_rows), k, H, int(row_lo), int(row_hi), _ptr(expert_out), _ptr(rti),
                                  _ptr(rtw), _ptr(tr), _ptr(reduced), _ptr(acc))
        return (reduced, acc) if return_acc else reduced

    def forward(self, x, topk_idx, topk_w, E: int, R: int, cap_rows: int, use_fp8: bool):
        """Layout + positions + dispatch, as one convenience call for tests."""
        L = self.layout(topk_idx, E, R, cap_rows)
        pos, src_idx = self.positions(topk_idx, L, E, R, cap_rows)
        recv_x, recv_scales, recv_w = self.dispatch(x, topk_w, pos, R * cap_rows, use_fp8)
        return L, pos, src_idx, recv_x, recv_scales, recv_w


def default() -> Oracle:
    """The oracle built from oracle/ep_oracle.c."""
    return _load()


def __getattr__(name):
    # module-level shortcuts: oracle.layout(...), oracle.combine(...), ...
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(_load(), name)
    raise AttributeError(name)
