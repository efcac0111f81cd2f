"""ctypes binding of libep.so (include/ep.h), plus a thin torch-tensor wrapper.

The functions ``ep_*`` mirror the C ABI one to one and take raw device
pointers (ints). ``Buffer`` allocates the caller-owned layout / handle /
receive tensors with torch and passes their pointers and torch's current HIP
stream; it does no arithmetic of its own. Every step of the hot path runs in
libep.so's kernels: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libep.so")

EP_OK = 0
EP_ERR_ARG = -1
EP_ERR_ALIGN = -2
EP_ERR_HIP = -3
EP_ERR_NOMEM = -4
EP_ERR_SCRATCH = -5

EP_ST_BAD_EXPERT = 1
EP_ST_DUP_EXPERT = 2
EP_ST_CAPACITY = 4
EP_ST_TIMEOUT = 8
EP_ST_BAD_HANDLE = 16

c_void_p = ctypes.c_void_p


class EpConfig(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_ranks", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cap_rows", ctypes.c_int64)]


LAYOUT_FIELDS = ("cnt_se", "cnt_sd", "recv_cnt", "expert_off", "rank_rows", "src_expert_off",
                 "rank_in_expert", "is_token_in_rank", "rank_in_rank", "token_rows")


class EpLayout(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in LAYOUT_FIELDS]


class EpHandle(ctypes.Structure):
    _fields_ = [("pos", c_void_p), ("src_idx", c_void_p),
                ("num_tokens", ctypes.c_int32), ("num_topk", ctypes.c_int32)]


SIZE_FIELDS = ("cnt_se", "cnt_sd", "recv_cnt", "expert_off", "rank_rows", "src_expert_off",
               "rank_in_expert", "is_token_in_rank", "pos", "src_idx", "x", "recv_x_bf16",
               "recv_x_fp8", "recv_scales", "recv_w", "combined_x", "rank_in_rank", "token_rows",
               "recv_topk_idx", "recv_topk_w", "workspace")


class EpSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in SIZE_FIELDS]


# (name, restype, argtypes) for every symbol include/ep.h declares
SIGNATURES = {
    "ep_version": (ctypes.c_int, []),
    "ep_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "ep_query_sizes": (ctypes.c_int, [ctypes.POINTER(EpConfig), ctypes.POINTER(EpSizes)]),
    "ep_create": (ctypes.c_int, [ctypes.POINTER(EpConfig), ctypes.POINTER(c_void_p)]),
    "ep_destroy": (ctypes.c_int, [c_void_p]),
    "ep_get_dispatch_layout": (ctypes.c_int, [c_void_p, c_void_p, ctypes.POINTER(EpLayout), c_void_p]),
    "ep_dispatch": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, ctypes.POINTER(EpLayout),
                                   ctypes.c_int, c_void_p, c_void_p, c_void_p,
                                   ctypes.POINTER(EpHandle), c_void_p]),
    "ep_dispatch_with_layout": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, ctypes.POINTER(EpLayout),
                                               ctypes.c_int, c_void_p, c_void_p, c_void_p,
                                               ctypes.POINTER(EpHandle), c_void_p]),
    "ep_dispatch_with_layout_noalloc": (ctypes.c_int, [ctypes.POINTER(EpConfig), c_void_p, c_void_p, c_void_p,
                                                       ctypes.POINTER(EpLayout), ctypes.c_int, c_void_p, c_void_p,
                                                       c_void_p, ctypes.POINTER(EpHandle), c_void_p, c_void_p]),
    "ep_dispatch_dedup": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, ctypes.POINTER(EpLayout),
                                         ctypes.c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                         ctypes.POINTER(EpHandle), c_void_p]),
    "ep_dispatch_dedup_with_layout": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p,
                                                     ctypes.POINTER(EpLayout), ctypes.c_int, c_void_p, c_void_p,
                                                     c_void_p, c_void_p, ctypes.POINTER(EpHandle), c_void_p]),
    "ep_dispatch_low_latency": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, ctypes.c_int, c_void_p,
                                               c_void_p, c_void_p, c_void_p, ctypes.POINTER(EpHandle),
                                               c_void_p]),
    "ep_combine": (ctypes.c_int, [c_void_p, c_void_p, ctypes.POINTER(EpHandle), c_void_p, c_void_p,
                                  c_void_p]),
    "ep_combine_f32": (ctypes.c_int, [c_void_p, c_void_p, ctypes.POINTER(EpHandle), c_void_p,
                                      c_void_p, c_void_p]),
    "ep_prereduce": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "ep_prereduce_f32": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "ep_combine_backward": (ctypes.c_int, [c_void_p, c_void_p, ctypes.POINTER(EpHandle), c_void_p,
                                           c_void_p]),
    "ep_dispatch_backward": (ctypes.c_int, [c_void_p, c_void_p, ctypes.POINTER(EpHandle), c_void_p,
                                            c_void_p, c_void_p]),
    "ep_get_status": (ctypes.c_int, [c_void_p, c_void_p, ctypes.POINTER(ctypes.c_uint32)]),
    "ep_copy_bytes": (ctypes.c_int, [c_void_p, c_void_p, ctypes.c_size_t, c_void_p]),
    "ep_cu_mask": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32),
                                  ctypes.c_int]),
    "ep_stream_create_cus": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.POINTER(c_void_p)]),
    "ep_stream_destroy": (ctypes.c_int, [c_void_p]),
    "ep_set_cu_budget": (ctypes.c_int, [c_void_p, ctypes.c_int]),
    "ep_set_spin_limit": (ctypes.c_int, [c_void_p, ctypes.c_uint32]),
    "ep_cu_census": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, c_void_p, c_void_p]),
    "ep_pattern_fill": (ctypes.c_int, [c_void_p, ctypes.c_size_t, c_void_p]),
    "ep_pattern_read": (ctypes.c_int, [c_void_p, ctypes.c_size_t, c_void_p, c_void_p]),
    "ep_pattern_push": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int64, c_void_p]),
    "ep_pattern_gather": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_int, c_void_p]),
}

_lib = None


class EpError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ep_strerror(code)} ({code})")


def load():
    """Load libep.so (built in-tree by combine_get_dispatch_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libep.so not built ({LIB_PATH}); run "
                               "`python -m combine_get_dispatch_amd.build` or __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(code: int, what: str) -> None:
    if code != EP_OK:
        raise EpError(code, what)


# ---------------------------------------------------------------------------
# the C ABI, one function per symbol
# ---------------------------------------------------------------------------

def ep_version() -> int:
    return load().ep_version()


def ep_strerror(code: int) -> str:
    return load().ep_strerror(code).decode()


def ep_query_sizes(cfg: EpConfig) -> EpSizes:
    s = EpSizes()
    _check(load().ep_query_sizes(ctypes.byref(cfg), ctypes.byref(s)), "ep_query_sizes")
    return s


def ep_create(cfg: EpConfig) -> int:
    ctx = c_void_p()
    _check(load().ep_create(ctypes.byref(cfg), ctypes.byref(ctx)), "ep_create")
    return ctx.value


def ep_destroy(ctx: int) -> None:
    _check(load().ep_destroy(ctx), "ep_destroy")


def ep_get_dispatch_layout(ctx: int, topk_idx: int, layout: EpLayout, stream: int) -> None:
    _check(load().ep_get_dispatch_layout(ctx, topk_idx, ctypes.byref(layout), stream),
           "ep_get_dispatch_layout")


def ep_dispatch(ctx: int, x: int, topk_idx: int, topk_weights: Optional[int], layout: EpLayout,
                use_fp8: int, recv_x: int, recv_scales: Optional[int], recv_w: Optional[int],
                handle: EpHandle, stream: int) -> None:
    _check(load().ep_dispatch(ctx, x, topk_idx, topk_weights, ctypes.byref(layout), int(use_fp8),
                              recv_x, recv_scales, recv_w, ctypes.byref(handle), stream), "ep_dispatch")


def ep_dispatch_with_layout(ctx: int, x: int, topk_idx: int, topk_weights: Optional[int], layout: EpLayout,
                            use_fp8: int, recv_x: int, recv_scales: Optional[int], recv_w: Optional[int],
                            handle: EpHandle, stream: int) -> None:
    _check(load().ep_dispatch_with_layout(ctx, x, topk_idx, topk_weights, ctypes.byref(layout), int(use_fp8),
                                          recv_x, recv_scales, recv_w, ctypes.byref(handle), stream),
           "ep_dispatch_with_layout")


def ep_dispatch_with_layout_noalloc(cfg: EpConfig, x: int, topk_idx: int, topk_weights: Optional[int],
                                    layout: EpLayout, use_fp8: int, recv_x: int, recv_scales: Optional[int],
                                    recv_w: Optional[int], handle: EpHandle, status: Optional[int],
                                    stream: int) -> None:
    _check(load().ep_dispatch_with_layout_noalloc(ctypes.byref(cfg), x, topk_idx, topk_weights,
                                                  ctypes.byref(layout), int(use_fp8), recv_x, recv_scales, recv_w,
                                                  ctypes.byref(handle), status, stream),
           "ep_dispatch_with_layout_noalloc")


def ep_dispatch_dedup(ctx: int, x: int, topk_idx: int, topk_weights: Optional[int], layout: EpLayout,
                      use_fp8: int, recv_x: int, recv_scales: Optional[int], recv_topk_idx: Optional[int],
                      recv_topk_w: Optional[int], handle: EpHandle, stream: int) -> None:
    _check(load().ep_dispatch_dedup(ctx, x, topk_idx, topk_weights, ctypes.byref(layout), int(use_fp8),
                                    recv_x, recv_scales, recv_topk_idx, recv_topk_w, ctypes.byref(handle),
                                    stream), "ep_dispatch_dedup")


def ep_dispatch_dedup_with_layout(ctx: int, x: int, topk_idx: int, topk_weights: Optional[int],
                                  layout: EpLayout, use_fp8: int, recv_x: int, recv_scales: Optional[int],
                                  recv_topk_idx: Optional[int], recv_topk_w: Optional[int], handle: EpHandle,
                                  stream: int) -> None:
    _check(load().ep_dispatch_dedup_with_layout(ctx, x, topk_idx, topk_weights, ctypes.byref(layout),
                                                int(use_fp8), recv_x, recv_scales, recv_topk_idx, recv_topk_w,
                                                ctypes.byref(handle), stream), "ep_dispatch_dedup_with_layout")


def ep_dispatch_low_latency(ctx: int, x: int, topk_idx: int, topk_weights: Optional[int], use_fp8: int,
                            recv_x: int, recv_scales: Optional[int], recv_w: Optional[int], recv_count: int,
                            handle: EpHandle, stream: int) -> None:
    _check(load().ep_dispatch_low_latency(ctx, x, topk_idx, topk_weights, int(use_fp8), recv_x, recv_scales,
                                          recv_w, recv_count, ctypes.byref(handle), stream),
           "ep_dispatch_low_latency")


def ll_cap_rows(num_tokens: int, num_experts: int, num_ranks: int) -> int:
    """cap_rows of a context for the low-latency receive layout: every expert
    holds num_tokens rows (one region of num_tokens/num_ranks per source)."""
    return num_experts * num_tokens // num_ranks


def ep_combine(ctx: int, expert_out: int, handle: EpHandle, weights: Optional[int],
               combined_x: int, stream: int) -> None:
    _check(load().ep_combine(ctx, expert_out, ctypes.byref(handle), weights, combined_x, stream),
           "ep_combine")


def ep_combine_f32(ctx: int, expert_out: int, handle: EpHandle, weights: Optional[int],
                   combined_f32: int, stream: int) -> None:
    _check(load().ep_combine_f32(ctx, expert_out, ctypes.byref(handle), weights, combined_f32, stream),
           "ep_combine_f32")


def ep_combine_backward(ctx: int, grad_combined: int, handle: EpHandle, grad_rows: int,
                        stream: int) -> None:
    _check(load().ep_combine_backward(ctx, grad_combined, ctypes.byref(handle), grad_rows, stream),
           "ep_combine_backward")


def ep_dispatch_backward(ctx: int, grad_rows: int, handle: EpHandle, weights: Optional[int],
                         grad_x: int, stream: int) -> None:
    _check(load().ep_dispatch_backward(ctx, grad_rows, ctypes.byref(handle), weights, grad_x, stream),
           "ep_dispatch_backward")


def ep_get_status(ctx: int, stream: int) -> int:
    st = ctypes.c_uint32()
    _check(load().ep_get_status(ctx, stream, ctypes.byref(st)), "ep_get_status")
    return st.value


def ep_copy_bytes(src: int, dst: int, nbytes: int, stream: int) -> None:
    _check(load().ep_copy_bytes(src, dst, nbytes, stream), "ep_copy_bytes")


def ep_pattern_fill(dst: int, nbytes: int, stream: int) -> None:
    _check(load().ep_pattern_fill(dst, nbytes, stream), "ep_pattern_fill")


def ep_pattern_read(src: int, nbytes: int, sink: int, stream: int) -> None:
    _check(load().ep_pattern_read(src, nbytes, sink, stream), "ep_pattern_read")


def ep_pattern_push(x: int, pos: int, rows: int, num_tokens: int, num_topk: int, hidden: int, num_rows: int,
                    stream: int) -> None:
    _check(load().ep_pattern_push(x, pos, rows, num_tokens, num_topk, hidden, num_rows, stream), "ep_pattern_push")


def ep_pattern_gather(rows: int, pos: int, out: int, num_tokens: int, num_topk: int, hidden: int, num_rows: int,
                      capped: bool, stream: int) -> None:
    _check(load().ep_pattern_gather(rows, pos, out, num_tokens, num_topk, hidden, num_rows, int(capped), stream),
           "ep_pattern_gather")


# ---------------------------------------------------------------------------
# torch convenience layer (allocation + pointer marshalling only)
# ---------------------------------------------------------------------------

def ep_cu_mask(cu_count: int, num_cus: int, exclude: bool = False) -> list:
    """The compute-unit mask as a list of 32-bit words (host only)."""
    words = max(cu_count // 32, 1)
    buf = (ctypes.c_uint32 * words)()
    _check(load().ep_cu_mask(cu_count, num_cus, int(bool(exclude)), buf, words), "ep_cu_mask")
    return list(buf)


def ep_stream_create_cus(num_cus: int, exclude: bool = False) -> int:
    out = c_void_p()
    _check(load().ep_stream_create_cus(num_cus, int(bool(exclude)), ctypes.byref(out)), "ep_stream_create_cus")
    return out.value


def ep_set_cu_budget(ctx: int, num_cus: int) -> None:
    _check(load().ep_set_cu_budget(ctx, num_cus), "ep_set_cu_budget")


def ep_set_spin_limit(ctx: int, polls: int) -> None:
    _check(load().ep_set_spin_limit(ctx, polls), "ep_set_spin_limit")


def ep_prereduce(ctx: int, expert_out: int, recv_topk_idx: int, recv_topk_w: Optional[int], token_rows: int,
                 reduced: int, stream: int) -> None:
    _check(load().ep_prereduce(ctx, expert_out, recv_topk_idx, recv_topk_w, token_rows, reduced, stream),
           "ep_prereduce")


def ep_prereduce_f32(ctx: int, expert_out: int, recv_topk_idx: int, recv_topk_w: Optional[int], token_rows: int,
                     reduced: int, stream: int) -> None:
    _check(load().ep_prereduce_f32(ctx, expert_out, recv_topk_idx, recv_topk_w, token_rows, reduced, stream),
           "ep_prereduce_f32")


def ep_stream_destroy(stream: int) -> None:
    _check(load().ep_stream_destroy(stream), "ep_stream_destroy")


def ep_cu_census(blocks: int, naps: int, ids: int, stream: int) -> None:
    _check(load().ep_cu_census(blocks, naps, ids, stream), "ep_cu_census")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Layout:
    cnt_se: "torch.Tensor"
    cnt_sd: "torch.Tensor"
    recv_cnt: "torch.Tensor"
    expert_off: "torch.Tensor"
    rank_rows: "torch.Tensor"
    src_expert_off: "torch.Tensor"
    rank_in_expert: "torch.Tensor"
    is_token_in_rank: "torch.Tensor"
    rank_in_rank: Optional["torch.Tensor"] = None   # [T, k] int32, rank-deduplicated exchange only
    token_rows: Optional["torch.Tensor"] = None     # [R] int32, rank-deduplicated exchange only

    def c(self) -> EpLayout:
        return EpLayout(*[_ptr(getattr(self, n)) for n in LAYOUT_FIELDS])


@dataclass
class Handle:
    pos: "torch.Tensor"       # [T, k] int32
    src_idx: "torch.Tensor"   # [R * cap_rows] int32
    num_tokens: int = 0
    num_topk: int = 0

    def c(self) -> EpHandle:
        return EpHandle(self.pos.data_ptr(), self.src_idx.data_ptr(), self.num_tokens, self.num_topk)


_deferred_contexts = []


def _destroy_deferred() -> None:
    while _deferred_contexts:
        ep_destroy(_deferred_contexts.pop())


class Buffer:
    """One expert-parallel group collapsed onto the current GPU: the analogue
    of the DeepEP guide's buffer (created once for a token count, hidden size
    and top-k), holding the libep context."""

    def __init__(self, num_tokens: int, hidden: int, num_topk: int, num_experts: int,
                 num_ranks: int, cap_rows: int, device=None):
        import torch
        self.torch = torch
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.cfg = EpConfig(num_tokens, num_topk, num_experts, num_ranks, hidden, 0, int(cap_rows))
        self.sizes = ep_query_sizes(self.cfg)
        _destroy_deferred()
        with torch.cuda.device(self.device):
            self.ctx = ep_create(self.cfg)

    # sizes
    @property
    def T(self): return self.cfg.num_tokens

    @property
    def k(self): return self.cfg.num_topk

    @property
    def E(self): return self.cfg.num_experts

    @property
    def R(self): return self.cfg.num_ranks

    @property
    def H(self): return self.cfg.hidden

    @property
    def cap_rows(self): return self.cfg.cap_rows

    @property
    def num_rows(self): return self.R * self.cap_rows

    def close(self):
        """Destroy the context (ep_destroy synchronizes the device, which a
        HIP graph capture forbids: a buffer released while a capture is in
        progress is destroyed by the next close or new buffer instead)."""
        if getattr(self, "ctx", None):
            if self.torch.cuda.is_current_stream_capturing():
                _deferred_contexts.append(self.ctx)
            else:
                _destroy_deferred()
                ep_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _empty(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.device)

    def new_layout(self, dedup: bool = False) -> Layout:
        """Layout buffers; ``dedup`` adds the rank-deduplicated outputs."""
        t = self.torch
        T, k, E, R = self.T, self.k, self.E, self.R
        return Layout(self._empty((R, E), t.int32), self._empty((R, R), t.int32), self._empty(E, t.int32),
                      self._empty(E, t.int32), self._empty(R, t.int32), self._empty((R, E), t.int32),
                      self._empty((T, k), t.int32), self._empty((T, R), t.uint8),
                      self._empty((T, k), t.int32) if dedup else None,
                      self._empty(R, t.int32) if dedup else None)

    def new_handle(self) -> Handle:
        t = self.torch
        return Handle(self._empty((self.T, self.k), t.int32), self._empty(self.num_rows, t.int32))

    def get_dispatch_layout(self, topk_idx, layout: Optional[Layout] = None) -> Layout:
        layout = layout or self.new_layout()
        ep_get_dispatch_layout(self.ctx, topk_idx.data_ptr(), layout.c(), _stream())
        return layout

    def dispatch(self, x, topk_idx, topk_weights, layout: Layout, use_fp8: bool, out=None):
        """Returns (recv_x, recv_scales, recv_w, handle)."""
        t = self.torch
        if out is None:
            recv_x = self._empty((self.num_rows, self.H), t.uint8 if use_fp8 else t.bfloat16)
            recv_scales = self._empty((self.num_rows, self.H // 128), t.float32) if use_fp8 else None
            recv_w = self._empty(self.num_rows, t.float32)
            handle = self.new_handle()
        else:
            recv_x, recv_scales, recv_w, handle = out
        ch = handle.c()
        ep_dispatch(self.ctx, x.data_ptr(), topk_idx.data_ptr(), _ptr(topk_weights), layout.c(),
                    int(bool(use_fp8)), recv_x.data_ptr(), _ptr(recv_scales), _ptr(recv_w), ch, _stream())
        handle.num_tokens, handle.num_topk = ch.num_tokens, ch.num_topk
        return recv_x, recv_scales, recv_w, handle

    def dispatch_with_layout(self, x, topk_idx, topk_weights, use_fp8: bool, layout: Optional[Layout] = None,
                             out=None):
        """Layout and dispatch in one launch. Returns (layout, recv_x,
        recv_scales, recv_w, handle)."""
        t = self.torch
        layout = layout or self.new_layout()
        if out is None:
            recv_x = self._empty((self.num_rows, self.H), t.uint8 if use_fp8 else t.bfloat16)
            recv_scales = self._empty((self.num_rows, self.H // 128), t.float32) if use_fp8 else None
            recv_w = self._empty(self.num_rows, t.float32)
            handle = self.new_handle()
        else:
            recv_x, recv_scales, recv_w, handle = out
        ch = handle.c()
        ep_dispatch_with_layout(self.ctx, x.data_ptr(), topk_idx.data_ptr(), _ptr(topk_weights), layout.c(),
                                int(bool(use_fp8)), recv_x.data_ptr(), _ptr(recv_scales), _ptr(recv_w), ch,
                                _stream())
        handle.num_tokens, handle.num_topk = ch.num_tokens, ch.num_topk
        return layout, recv_x, recv_scales, recv_w, handle

    def dispatch_dedup(self, x, topk_idx, topk_weights, layout: Layout, use_fp8: bool, out=None):
        """Rank-deduplicated dispatch: one row per (token, destination rank).
        ``layout`` must come from ``get_dispatch_layout`` on a layout made with
        ``new_layout(dedup=True)``. Returns (recv_x, recv_scales,
        recv_topk_idx, recv_topk_w, handle)."""
        t = self.torch
        if out is None:
            recv_x = self._empty((self.num_rows, self.H), t.uint8 if use_fp8 else t.bfloat16)
            recv_scales = self._empty((self.num_rows, self.H // 128), t.float32) if use_fp8 else None
            recv_topk_idx = self._empty((self.num_rows, self.k), t.int32)
            recv_topk_w = self._empty((self.num_rows, self.k), t.float32) if topk_weights is not None else None
            handle = self.new_handle()
        else:
            recv_x, recv_scales, recv_topk_idx, recv_topk_w, handle = out
        ch = handle.c()
        ep_dispatch_dedup(self.ctx, x.data_ptr(), topk_idx.data_ptr(), _ptr(topk_weights), layout.c(),
                          int(bool(use_fp8)), recv_x.data_ptr(), _ptr(recv_scales), _ptr(recv_topk_idx),
                          _ptr(recv_topk_w), ch, _stream())
        handle.num_tokens, handle.num_topk = ch.num_tokens, ch.num_topk
        return recv_x, recv_scales, recv_topk_idx, recv_topk_w, handle

    def dispatch_dedup_with_layout(self, x, topk_idx, topk_weights, use_fp8: bool, layout: Optional[Layout] = None,
                                   out=None):
        """Deduplicated layout and dispatch in one launch. Returns (layout,
        recv_x, recv_scales, recv_topk_idx, recv_topk_w, handle)."""
        t = self.torch
        layout = layout or self.new_layout(dedup=True)
        if out is None:
            recv_x = self._empty((self.num_rows, self.H), t.uint8 if use_fp8 else t.bfloat16)
            recv_scales = self._empty((self.num_rows, self.H // 128), t.float32) if use_fp8 else None
            recv_topk_idx = self._empty((self.num_rows, self.k), t.int32)
            recv_topk_w = self._empty((self.num_rows, self.k), t.float32) if topk_weights is not None else None
            handle = self.new_handle()
        else:
            recv_x, recv_scales, recv_topk_idx, recv_topk_w, handle = out
        ch = handle.c()
        ep_dispatch_dedup_with_layout(self.ctx, x.data_ptr(), topk_idx.data_ptr(), _ptr(topk_weights), layout.c(),
                                      int(bool(use_fp8)), recv_x.data_ptr(), _ptr(recv_scales),
                                      _ptr(recv_topk_idx), _ptr(recv_topk_w), ch, _stream())
        handle.num_tokens, handle.num_topk = ch.num_tokens, ch.num_topk
        return layout, recv_x, recv_scales, recv_topk_idx, recv_topk_w, handle

    def dispatch_low_latency(self, x, topk_idx, topk_weights, use_fp8: bool, out=None):
        """Low-latency dispatch (the buffer must have cap_rows =
        ll_cap_rows(T, E, R)). Returns (recv_x, recv_scales, recv_w,
        recv_count [E, R], handle)."""
        t = self.torch
        if out is None:
            recv_x = self._empty((self.num_rows, self.H), t.uint8 if use_fp8 else t.bfloat16)
            recv_scales = self._empty((self.num_rows, self.H // 128), t.float32) if use_fp8 else None
            recv_w = self._empty(self.num_rows, t.float32) if topk_weights is not None else None
            recv_count = self._empty((self.E, self.R), t.int32)
            handle = self.new_handle()
        else:
            recv_x, recv_scales, recv_w, recv_count, handle = out
        ch = handle.c()
        ep_dispatch_low_latency(self.ctx, x.data_ptr(), topk_idx.data_ptr(), _ptr(topk_weights),
                                int(bool(use_fp8)), recv_x.data_ptr(), _ptr(recv_scales), _ptr(recv_w),
                                recv_count.data_ptr(), ch, _stream())
        handle.num_tokens, handle.num_topk = ch.num_tokens, ch.num_topk
        return recv_x, recv_scales, recv_w, recv_count, handle

    def combine(self, expert_out, handle: Handle, weights=None, out=None):
        out = out if out is not None else self._empty((self.T, self.H), self.torch.bfloat16)
        ep_combine(self.ctx, expert_out.data_ptr(), handle.c(), _ptr(weights), out.data_ptr(), _stream())
        return out

    def combine_f32(self, expert_out, handle: Handle, weights=None, out=None):
        out = out if out is not None else self._empty((self.T, self.H), self.torch.float32)
        ep_combine_f32(self.ctx, expert_out.data_ptr(), handle.c(), _ptr(weights), out.data_ptr(), _stream())
        return out

    def prereduce(self, expert_out, recv_topk_idx, recv_topk_w, token_rows, out=None):
        """Expert-side pre-reduction of deduplicated rows: expert_out
        [R*cap_rows, k, H] bf16 (the output of each received row's slot-j
        expert), routing entries and weights from dispatch_dedup, token_rows
        from the deduplicated layout. Returns reduced [R*cap_rows, H] bf16
        (unused rows not written)."""
        out = out if out is not None else self._empty((self.num_rows, self.H), self.torch.bfloat16)
        ep_prereduce(self.ctx, expert_out.data_ptr(), recv_topk_idx.data_ptr(), _ptr(recv_topk_w),
                     token_rows.data_ptr(), out.data_ptr(), _stream())
        return out

    def prereduce_f32(self, expert_out, recv_topk_idx, recv_topk_w, token_rows, out=None):
        out = out if out is not None else self._empty((self.num_rows, self.H), self.torch.float32)
        ep_prereduce_f32(self.ctx, expert_out.data_ptr(), recv_topk_idx.data_ptr(), _ptr(recv_topk_w),
                         token_rows.data_ptr(), out.data_ptr(), _stream())
        return out

    def combine_backward(self, grad_combined, handle: Handle, out=None):
        out = out if out is not None else self._empty((self.num_rows, self.H), self.torch.bfloat16)
        ep_combine_backward(self.ctx, grad_combined.data_ptr(), handle.c(), out.data_ptr(), _stream())
        return out

    def dispatch_backward(self, grad_rows, handle: Handle, weights=None, out=None):
        out = out if out is not None else self._empty((self.T, self.H), self.torch.bfloat16)
        ep_dispatch_backward(self.ctx, grad_rows.data_ptr(), handle.c(), _ptr(weights), out.data_ptr(),
                             _stream())
        return out

    def set_num_cus(self, num_cus: int) -> None:
        """The compute units the stream these calls run on may use (0 = all);
        see CuStream."""
        ep_set_cu_budget(self.ctx, num_cus)

    def set_spin_limit(self, polls: int) -> None:
        """Polls of a bounded wait before it gives up with EP_ST_TIMEOUT (0 = default)."""
        ep_set_spin_limit(self.ctx, polls)

    def status(self) -> int:
        """Synchronize the current stream; return and clear the sticky status bits."""
        return ep_get_status(self.ctx, _stream())


class CuStream:
    """A HIP stream whose kernels run on `num_cus` compute units (or on the
    others, exclude=True), wrapped as a torch external stream; use it with
    ``torch.cuda.stream(s.torch_stream)`` so the ep calls and torch work
    issued inside launch on it. close() destroys the HIP stream."""

    def __init__(self, num_cus: int, exclude: bool = False):
        import torch
        self.num_cus, self.exclude = num_cus, exclude
        self.handle = ep_stream_create_cus(num_cus, exclude)
        self.torch_stream = torch.cuda.ExternalStream(self.handle)

    def close(self):
        if self.handle:
            self.torch_stream.synchronize()
            ep_stream_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def cu_census(blocks: int = 8192, naps: int = 2):
    """The compute units a launch of `blocks` workgroups on the current stream
    ran on (a uint32 tensor of (XCD << 16) | unit bits, one per workgroup)."""
    import torch
    ids = torch.empty(blocks, dtype=torch.int32, device="cuda")
    ep_cu_census(blocks, naps, ids.data_ptr(), _stream())
    return ids


def copy_bytes(src, dst) -> None:
    n = min(src.numel() * src.element_size(), dst.numel() * dst.element_size())
    ep_copy_bytes(src.data_ptr(), dst.data_ptr(), n, _stream())
