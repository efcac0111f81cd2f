"""libep.so loads and exports every symbol include/ep.h declares; host-only
argument validation (no GPU needed, no compute calls)."""
import ctypes
import os
import re

import pytest

from combine_get_dispatch_amd import build as epbuild
from combine_get_dispatch_amd import ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ep.LIB_PATH):
        epbuild.build()  # nothing built yet: build once
    return ep.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ("ep_get_dispatch_layout", "ep_dispatch", "ep_combine", "ep_combine_backward",
              "ep_dispatch_backward", "ep_create", "ep_destroy", "ep_query_sizes", "ep_get_status",
              "ep_strerror"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ep.h but not exported"
    assert set(names) == set(ep.SIGNATURES), "binding and header disagree"


def test_extern_c_symbols_unmangled(lib):
    for n in declared_functions():
        ctypes.cast(getattr(lib, n), ctypes.c_void_p)  # resolves by its plain C name


def test_version_and_strerror(lib):
    assert ep.ep_version() == 2
    assert ep.ep_strerror(0) == "ok"
    assert "argument" in ep.ep_strerror(-1)
    assert "align" in ep.ep_strerror(-2)
    assert ep.ep_strerror(12345) == "unknown error"


def cfg(T=64, k=2, E=16, R=4, H=256, cap=64, reserved=0):
    return ep.EpConfig(T, k, E, R, H, reserved, cap)


@pytest.mark.parametrize("bad", [
    dict(T=63), dict(k=0), dict(k=33), dict(E=15), dict(E=2048, R=4), dict(R=0), dict(R=65, E=130, T=130),
    dict(H=4), dict(H=12), dict(H=65544), dict(cap=-1), dict(reserved=1), dict(T=-4),
    dict(R=64, E=64, T=64, cap=1 << 25),
])
def test_query_sizes_rejects(lib, bad):
    with pytest.raises(ep.EpError) as e:
        ep.ep_query_sizes(cfg(**bad))
    assert e.value.code == ep.EP_ERR_ARG


def test_query_sizes_values(lib):
    s = ep.ep_query_sizes(cfg(T=4096, k=8, E=256, R=32, H=7168, cap=1500))
    rows = 32 * 1500
    assert s.x == 4096 * 7168 * 2
    assert s.recv_x_fp8 == rows * 7168 and s.recv_x_bf16 == rows * 7168 * 2
    assert s.recv_scales == rows * 56 * 4 and s.recv_w == rows * 4 and s.src_idx == rows * 4
    assert s.pos == s.rank_in_expert == 4096 * 8 * 4
    assert s.is_token_in_rank == 4096 * 32
    assert s.cnt_se == s.src_expert_off == 32 * 256 * 4 and s.cnt_sd == 32 * 32 * 4
    assert s.rank_in_rank == 4096 * 8 * 4 and s.token_rows == 32 * 4
    assert s.recv_topk_idx == s.recv_topk_w == rows * 8 * 4
    assert s.workspace >= 16 * 4 + 33 * 288 * 4  # counters + boundary prefixes (+ tile states)
    ep.ep_query_sizes(cfg(T=0))  # empty input is a valid config


def test_null_args_rejected_without_gpu(lib):
    L = lib
    assert L.ep_create(None, None) == ep.EP_ERR_ARG
    out = ctypes.c_void_p()
    assert L.ep_create(ctypes.byref(cfg(T=63)), ctypes.byref(out)) == ep.EP_ERR_ARG and not out.value
    assert L.ep_get_dispatch_layout(None, None, None, None) == ep.EP_ERR_ARG
    assert L.ep_combine(None, None, None, None, None, None) == ep.EP_ERR_ARG
    assert L.ep_dispatch_dedup(None, None, None, None, None, 0, None, None, None, None, None, None) == ep.EP_ERR_ARG
    assert L.ep_destroy(None) == ep.EP_OK
    assert L.ep_copy_bytes(None, None, 0, None) == ep.EP_OK
    assert L.ep_copy_bytes(None, None, 16, None) == ep.EP_ERR_ARG
    # the access-pattern utilities: refusals without a launch
    assert L.ep_pattern_fill(None, 0, None) == ep.EP_OK
    assert L.ep_pattern_fill(None, 1024, None) == ep.EP_ERR_ARG
    assert L.ep_pattern_fill(ctypes.c_void_p(16), 1000, None) == ep.EP_ERR_ARG
    assert L.ep_pattern_fill(ctypes.c_void_p(8), 1024, None) == ep.EP_ERR_ALIGN
    assert L.ep_pattern_read(ctypes.c_void_p(16), 4096, None, None) == ep.EP_ERR_ARG
    assert L.ep_pattern_read(ctypes.c_void_p(16), 1024, ctypes.c_void_p(16), None) == ep.EP_ERR_ARG
    p16 = ctypes.c_void_p(16)
    assert L.ep_pattern_push(p16, p16, p16, 0, 8, 7168, 10, None) == ep.EP_OK
    assert L.ep_pattern_push(p16, p16, p16, 4, 8, 7000, 10, None) == ep.EP_ERR_ARG   # hidden % 1024
    assert L.ep_pattern_push(p16, p16, p16, 4, 8, 9216, 10, None) == ep.EP_ERR_ARG   # > 8192
    assert L.ep_pattern_push(p16, p16, p16, 4, 65, 7168, 10, None) == ep.EP_ERR_ARG  # top-k > 64
    assert L.ep_pattern_push(ctypes.c_void_p(8), p16, p16, 4, 8, 7168, 10, None) == ep.EP_ERR_ALIGN
    assert L.ep_pattern_gather(p16, p16, p16, 4, 9, 7168, 10, 0, None) == ep.EP_ERR_ARG  # top-k > 8
    assert L.ep_pattern_gather(p16, p16, None, 4, 8, 7168, 10, 0, None) == ep.EP_ERR_ARG
    assert L.ep_pattern_gather(p16, p16, ctypes.c_void_p(8), 4, 8, 7168, 10, 1, None) == ep.EP_ERR_ALIGN


def _xcd_counts(mask, cu_count, interleaved):
    per = cu_count // 8
    counts = [0] * 8
    for i in range(cu_count):
        if (mask[i // 32] >> (i % 32)) & 1:
            counts[i % 8 if interleaved else i // per] += 1
    return counts


@pytest.mark.parametrize("num_cus", [8, 32, 64, 128, 200, 248, 256])
def test_cu_mask_same_count_on_every_xcd(lib, num_cus):
    """num_cus/8 units on each XCD under either assignment of mask bits to
    XCDs (bit i on XCD i mod 8, or on XCD i / 32); the complement holds the
    rest, again evenly."""
    C = 256
    m = ep.ep_cu_mask(C, num_cus)
    assert sum(bin(w).count("1") for w in m) == num_cus
    for inter in (False, True):
        assert _xcd_counts(m, C, inter) == [num_cus // 8] * 8
    if num_cus < C:
        c = ep.ep_cu_mask(C, num_cus, exclude=True)
        assert all((a & b) == 0 for a, b in zip(m, c)) and all((a | b) == 0xFFFFFFFF for a, b in zip(m, c))
        for inter in (False, True):
            assert _xcd_counts(c, C, inter) == [(C - num_cus) // 8] * 8


@pytest.mark.parametrize("bad", [dict(num_cus=0), dict(num_cus=12), dict(num_cus=264), dict(num_cus=-8),
                                 dict(num_cus=256, exclude=True), dict(cu_count=250, num_cus=8)])
def test_cu_mask_rejects(lib, bad):
    args = dict(cu_count=256, exclude=False)
    args.update(bad)
    with pytest.raises(ep.EpError) as e:
        ep.ep_cu_mask(args["cu_count"], args["num_cus"], args["exclude"])
    assert e.value.code == ep.EP_ERR_ARG
    assert lib.ep_stream_create_cus(8, 0, None) == ep.EP_ERR_ARG
    assert lib.ep_cu_census(-1, 0, None, None) == ep.EP_ERR_ARG
    assert lib.ep_stream_destroy(None) == ep.EP_OK


def test_low_latency_rejects_other_receive_sizes(lib):
    assert lib.ep_dispatch_low_latency(None, None, None, None, 0, None, None, None, None, None, None) == ep.EP_ERR_ARG
    assert ep.ll_cap_rows(1024, 256, 8) == 32768  # every expert holds T rows: R*cap_rows = E*T


def test_new_entry_points_reject_null_without_gpu(lib):
    L = lib
    assert L.ep_dispatch_dedup_with_layout(None, None, None, None, None, 0, None, None, None, None, None,
                                           None) == ep.EP_ERR_ARG
    assert L.ep_set_cu_budget(None, 8) == ep.EP_ERR_ARG
    assert L.ep_set_spin_limit(None, 1) == ep.EP_ERR_ARG
    assert L.ep_prereduce(None, None, None, None, None, None, None) == ep.EP_ERR_ARG
    assert L.ep_prereduce_f32(None, None, None, None, None, None, None) == ep.EP_ERR_ARG
    # the no-allocation call refuses a workload beyond its static workspace
    # before touching the GPU
    big = ep.EpConfig(1 << 22, 8, 256, 32, 7168, 0, 1 << 20)
    assert L.ep_dispatch_with_layout_noalloc(big, None, None, None, None, 1, None, None, None, None, None,
                                             None) == ep.EP_ERR_SCRATCH
    assert L.ep_dispatch_with_layout_noalloc(None, None, None, None, None, 1, None, None, None, None, None,
                                             None) == ep.EP_ERR_ARG
    assert L.ep_cu_census(0, 0, None, None) == ep.EP_OK  # nothing to launch
    assert L.ep_cu_census(16, 65, None, None) == ep.EP_ERR_ARG
