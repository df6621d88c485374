"""The oracle's host encoders over every fp32 bit pattern (NaNs excluded).

* bf16: oracle.formats.f32_to_bf16_bits (a choice between the two
  neighbouring bf16 values by exact float64 distance) against the integer
  form of round-to-nearest-even on the fp32 bits (add 0x7FFF plus the lowest
  kept bit, drop 16 bits).
* e4m3fn / e5m2: oracle.formats encoders (code-table search) against
  PyTorch's float8 casts below the largest finite value, and saturation to
  the largest code at and beyond it.

2^32 patterns in 1024 slices of 2^22, spread over the host's cores."""
import multiprocessing as mp
import os

import numpy as np
import pytest

pytestmark = pytest.mark.slow

SLICE_BITS = 22


def _check_slice(c):
    import torch

    from oracle import formats
    u = np.arange(1 << SLICE_BITS, dtype=np.uint32) + np.uint32(c << SLICE_BITS)
    mag = u & np.uint32(0x7FFFFFFF)
    u = u[mag <= np.uint32(0x7F800000)]                   # NaNs excluded
    x = u.view(np.float32)
    bad = []
    # bf16: integer round-to-nearest-even of the bits (infinities stay)
    want = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    inf = (u & np.uint32(0x7FFFFFFF)) == np.uint32(0x7F800000)
    want = np.where(inf, (u >> np.uint32(16)).astype(np.uint16), want)
    got = formats.f32_to_bf16_bits(x)
    if not np.array_equal(got, want):
        bad.append(("bf16", int(u[np.flatnonzero(got != want)[0]])))
    xd = x.astype(np.float64)
    for name, enc, tdt, fmax, top in (("e4m3", formats.e4m3_encode, torch.float8_e4m3fn, 448.0, 0x7E),
                                      ("e5m2", formats.e5m2_encode, torch.float8_e5m2, 57344.0, 0x7B)):
        got = enc(xd)
        small = np.abs(xd) < fmax
        ref = torch.from_numpy(x[small]).to(tdt).view(torch.uint8).numpy()
        if not np.array_equal(got[small], ref):
            bad.append((name, int(u[small][np.flatnonzero(got[small] != ref)[0]])))
        sat = ~small
        want_sat = np.where(np.signbit(xd[sat]), top | 0x80, top).astype(np.uint8)
        if not np.array_equal(got[sat], want_sat):
            bad.append((name + " saturation", int(u[sat][np.flatnonzero(got[sat] != want_sat)[0]])))
    return c, bad


def test_encoders_over_all_fp32_patterns():
    n = 1 << (32 - SLICE_BITS)
    procs = max(1, min(8, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    old = os.environ.get("PYTHONPATH", "")
    os.environ["PYTHONPATH"] = root + (os.pathsep + old if old else "")
    try:
        with ctx.Pool(procs) as pool:
            results = pool.map(_check_slice, range(n), chunksize=4)
    finally:
        os.environ["PYTHONPATH"] = old
    failures = [(c, b) for c, b in results if b]
    assert len(results) == n
    assert not failures, failures[:4]
