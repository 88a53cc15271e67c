"""GPU test of ra_count_nonfinite_noalloc, the entry point that allocates
nothing: through the C ABI it must return exactly what ra_count_nonfinite
returns, on two calls in a row (the second on a smaller input, after the first
left its count in the shared scratch), and what numpy counts on host copies.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from ring_attention_ra_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield
    torch.cuda.synchronize()


def _planted(n, dtype, n_bad, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, generator=g).to(dtype)
    idx = torch.randperm(n, generator=g)[:n_bad]
    vals = torch.tensor([float("nan"), float("inf"), -float("inf")])[torch.arange(n_bad) % 3]
    x[idx] = vals.to(dtype)
    return x


def _count_c(fn, x, stream):
    n = ctypes.c_int64(-1)
    st = fn(ctypes.c_void_p(x.data_ptr()), x.numel(), _lib.dtype_code(x.dtype), ctypes.byref(n),
            ctypes.c_void_p(stream.cuda_stream))
    assert st == _lib.RA_OK, _lib.ra_last_error()
    return n.value


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_allocating_entry_point_twice(dtype):
    lib = _lib.lib()
    stream = torch.cuda.current_stream()
    first = _planted(1 << 22, dtype, 1000, 1)
    second = _planted(4097, dtype, 7, 2)  # smaller, fewer non-finite values
    for x in (first, second):
        ref_np = int((~np.isfinite(x.float().numpy())).sum())
        xd = x.cuda()
        got = _count_c(lib.ra_count_nonfinite_noalloc, xd, stream)
        ref = _count_c(lib.ra_count_nonfinite, xd, stream)
        assert got == ref == ref_np, (got, ref, ref_np)
    # a clean input after a dirty one reads 0: the scratch is cleared per call
    clean = torch.randn(1000, dtype=torch.float32).to(dtype).cuda()
    assert _count_c(lib.ra_count_nonfinite_noalloc, clean, stream) == 0
    assert _lib.ra_count_nonfinite_noalloc(clean) == 0


def test_noalloc_validation():
    lib = _lib.lib()
    n = ctypes.c_int64(5)
    assert lib.ra_count_nonfinite_noalloc(None, 0, 0, ctypes.byref(n), None) == 0 and n.value == 0
    assert lib.ra_count_nonfinite_noalloc(None, 4, 0, ctypes.byref(n), None) == 1
    assert lib.ra_count_nonfinite_noalloc(1, 4, 0, None, None) == 1
    assert lib.ra_count_nonfinite_noalloc(1, 4, 5, ctypes.byref(n), None) == 1
