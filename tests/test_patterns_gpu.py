"""The access-pattern measurement calls (ep_pattern_*) write exactly what
their declarations state and nothing outside the buffers given: each result
is checked against a numpy computation of the same bytes on small inputs
(these calls carry none of the method's arithmetic, so no oracle is
involved). Guard bands around every output catch a stray write."""
import numpy as np
import pytest
import torch

from combine_get_dispatch_amd import ep
from gpu_helpers import dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ep.load()  # the HIP library must be the path that runs; no fallback

GUARD = 4096  # bytes of a known pattern on each side of an output
PAT = 0xA5


def _stream():
    return torch.cuda.current_stream().cuda_stream


def guarded(nbytes):
    """A device byte buffer with GUARD pattern bytes on both sides; returns
    (whole buffer, view of the nbytes in the middle)."""
    buf = torch.full((nbytes + 2 * GUARD,), PAT, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + nbytes]


def guards_intact(buf):
    h = buf.cpu().numpy()
    return bool(np.all(h[:GUARD] == PAT) and np.all(h[-GUARD:] == PAT))


def test_fill_writes_wave_index_per_kb():
    nkb = 777
    buf, mid = guarded(nkb * 1024)
    ep.ep_pattern_fill(mid.data_ptr(), nkb * 1024, _stream())
    torch.cuda.synchronize()
    got = mid.cpu().numpy().view(np.uint32).reshape(nkb, 256)
    assert np.array_equal(got, np.repeat(np.arange(nkb, dtype=np.uint32)[:, None], 256, axis=1))
    assert guards_intact(buf)


def test_read_writes_nothing_on_zero_data():
    src = torch.zeros(64 * 4096, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    ep.ep_pattern_read(src.data_ptr(), src.numel(), sink.data_ptr(), _stream())
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


def _positions(rng, T, k, num_rows):
    """Distinct rows for most slots, -1 for some, some at or past num_rows
    (which the calls must skip)."""
    pos = rng.permutation(num_rows)[:T * k].astype(np.int32).reshape(T, k)
    pos[rng.random((T, k)) < 0.15] = -1
    pos[rng.random((T, k)) < 0.05] = num_rows + 3
    return pos


@pytest.mark.parametrize("H", [1024, 7168, 8192])
def test_push_stores_high_bytes_at_each_position(H):
    rng = np.random.default_rng(H)
    T, k, num_rows = 37, 8, 400
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    pos = _positions(rng, T, k, num_rows)
    buf, rows = guarded(num_rows * H)
    xd, pd = dev(x.view(np.int16)), dev(pos)
    ep.ep_pattern_push(xd.data_ptr(), pd.data_ptr(), rows.data_ptr(), T, k, H, num_rows, _stream())
    torch.cuda.synchronize()
    want = np.full((num_rows, H), PAT, np.uint8)
    for t in range(T):
        for j in range(k):
            p = pos[t, j]
            if 0 <= p < num_rows:
                want[p] = (x[t] >> 8).astype(np.uint8)
    assert np.array_equal(rows.cpu().numpy().reshape(num_rows, H), want)
    assert guards_intact(buf)


@pytest.mark.parametrize("capped", [False, True])
@pytest.mark.parametrize("k", [1, 8])
def test_gather_stores_xor_of_each_tokens_rows(capped, k):
    rng = np.random.default_rng(10 * k + capped)
    T, H, num_rows = 53, 3072, 500
    rows = rng.integers(0, 1 << 16, size=(num_rows, H), dtype=np.uint16)
    pos = _positions(rng, T, k, num_rows)
    buf, out = guarded(T * H * 2)
    rd, pd = dev(rows.view(np.int16)), dev(pos)
    ep.ep_pattern_gather(rd.data_ptr(), pd.data_ptr(), out.data_ptr(), T, k, H, num_rows, capped, _stream())
    torch.cuda.synchronize()
    want = np.zeros((T, H), np.uint16)
    for t in range(T):
        for j in range(k):
            p = pos[t, j]
            if 0 <= p < num_rows:
                want[t] ^= rows[p]
    assert np.array_equal(out.cpu().numpy().view(np.uint16).reshape(T, H), want)
    assert guards_intact(buf)
