"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/ra.h declares, and rejects invalid arguments before
launching anything. Also the binding's host logic (ring order, slopes)."""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from ring_attention_ra_amd import _lib, configs, ring

L = _lib.lib()


def _dims(b=1, hq=2, hkv=2, d=128, lq=128, lkv=128, dt=_lib.RA_BF16):
    return _lib.RaDims(b, hq, hkv, d, lq, lkv, dt)


def _fwd(dims, ptr=1, scale=0.1, slopes=None):
    return L.ra_step_fwd(None if dims is None else ctypes.byref(dims), ptr, ptr, ptr, ptr, ptr, 1, scale,
                         slopes, ptr, ptr, ptr, None)


def test_exports_every_declared_symbol():
    names = _lib.header_symbols()
    assert set(names) >= {"ra_layout_permute", "ra_step_fwd", "ra_finalize", "ra_step_bwd", "ra_positions",
                          "ra_state_init", "ra_bwd_delta", "ra_last_error", "ra_abi_version"}
    for n in names:
        assert hasattr(L, n), n
    assert L.ra_abi_version() == 1


@pytest.mark.parametrize("dims,status,needle", [
    (None, 1, "dims is NULL"),
    (_dims(hq=3, hkv=2), 1, "multiple of heads_kv"),
    (_dims(hkv=0), 1, "multiple of heads_kv"),
    (_dims(d=96), 2, "head_dim"),
    (_dims(d=129, dt=_lib.RA_FP32), 2, "head_dim"),
    (_dims(d=0), 1, "head_dim"),
    (_dims(lq=-1), 1, "negative"),
    (_dims(dt=7), 1, "dtype"),
])
def test_step_fwd_validation(dims, status, needle):
    assert _fwd(dims) == status
    assert needle in _lib.ra_last_error()


def test_step_fwd_null_pointer_and_scale():
    assert _fwd(_dims(), ptr=None) == 1 and "NULL" in _lib.ra_last_error()
    assert _fwd(_dims(), scale=float("nan")) == 1 and "scale" in _lib.ra_last_error()
    assert _fwd(_dims(), scale=float("inf")) == 1


def test_empty_work_is_ok_without_launch():
    assert _fwd(_dims(lkv=0), ptr=None) == 0
    assert _fwd(_dims(lq=0), ptr=None) == 0
    assert _fwd(_dims(b=0), ptr=None) == 0
    assert L.ra_finalize(ctypes.byref(_dims()), None, None, None, None, None, None) == 0
    assert L.ra_layout_permute(None, None, None, 0, 16, 8, 0, 4, 0, -1, 0, None) == 0


@pytest.mark.parametrize("args,needle", [
    ((16, 0, -1, 0), "n_ranks"),
    ((18, 4, -1, 0), "multiple"),
    ((16, 4, 4, 0), "rank"),
    ((16, 4, -2, 0), "rank"),
    ((16, 4, 0, 5), "layout"),
    ((2 ** 31, 4, 0, 0), "int32"),
])
def test_positions_validation(args, needle):
    s, n, r, lay = args
    assert L.ra_positions(s, n, r, lay, 1, None) == 1
    assert needle in _lib.ra_last_error()
    assert L.ra_positions(16, 4, 0, 0, None, None) == 1


def test_permute_validation():
    buf = ctypes.create_string_buffer(4096)
    base = ctypes.addressof(buf)
    # overlapping src/dst
    assert L.ra_layout_permute(base, base + 16, None, 1, 16, 8, 0, 4, 0, -1, 0, None) == 1
    assert "overlap" in _lib.ra_last_error()
    assert L.ra_layout_permute(base, base + 2048, None, 1, 16, 8, 0, 4, 0, -1, 2, None) == 1
    assert L.ra_layout_permute(base, base + 2048, None, 1, 16, 0, 0, 4, 0, -1, 0, None) == 1
    assert L.ra_layout_permute(base, base + 2048, None, 1, 16, 8, 3, 4, 0, -1, 0, None) == 1
    assert L.ra_layout_permute(None, base, None, 1, 16, 8, 0, 4, 0, -1, 0, None) == 1


def test_rope_validation():
    buf = ctypes.create_string_buffer(4096)
    base = ctypes.addressof(buf)
    ok = (base, base, base + 2048, 2, 4, 64, 0, 10000.0, None)
    bad = [
        ((base, base, base + 2048, 2, 4, 63, 0, 10000.0, None), "even"),      # odd head_dim
        ((base, base, base + 2048, 2, 4, 258, 0, 10000.0, None), "even"),     # too wide
        ((base, base, base + 2048, 2, 4, 64, 7, 10000.0, None), "dtype"),
        ((base, base, base + 2048, 2, 4, 64, 0, 0.0, None), "base"),
        ((base, base, base + 2048, 2, 4, 64, 0, float("inf"), None), "base"),
        ((base, base, None, 2, 4, 64, 0, 10000.0, None), "NULL"),
        ((base, base + 2, base + 2048, 2, 4, 64, 0, 10000.0, None), "overlap"),
        ((base, base, base + 2048, -1, 4, 64, 0, 10000.0, None), "negative"),
    ]
    for args, needle in bad:
        assert L.ra_rope(*args) == 1
        assert needle in _lib.ra_last_error()
    # no work: nothing is validated beyond the shape and nothing is launched
    assert L.ra_rope(None, None, None, 0, 4, 64, 0, 10000.0, None) == 0
    assert L.ra_rope(None, None, None, 2, 0, 64, 0, 10000.0, None) == 0
    assert ok  # the valid form launches, which needs a GPU: covered by the GPU tests


def test_bwd_validation():
    d = _dims(d=64)
    args = [ctypes.byref(d)] + [None] * 5 + [1, 0.1, None] + [None] * 6 + [None]
    assert L.ra_step_bwd(*args) == 2 and "head_dim 128" in _lib.ra_last_error()
    d = _dims(dt=_lib.RA_FP32, d=129)
    assert L.ra_step_bwd(ctypes.byref(d), *args[1:]) == 2 and "head_dim" in _lib.ra_last_error()
    d = _dims(dt=_lib.RA_FP32, d=64)
    assert L.ra_step_bwd(ctypes.byref(d), *args[1:]) == 1 and "NULL" in _lib.ra_last_error()
    d = _dims()
    args = [ctypes.byref(d)] + [1] * 5 + [1, 0.1, None] + [1] * 5 + [None, None]
    assert L.ra_step_bwd(*args) == 1


def test_binding_checks_tensors():
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        _lib._ptr(t, "t")  # host tensor
    with pytest.raises(ValueError):
        _lib.dtype_code(torch.float16)


def test_ring_schedule_and_slopes_agree_with_oracle():
    for n in (1, 4, 8, 64):
        for r in range(n):
            assert ring.ring_schedule(n, r) == oracle.ring_schedule(n, r)
    for h in (1, 8, 16, 64):
        got = ring.alibi_slopes(h, device="cpu").numpy()
        np.testing.assert_array_equal(got, oracle.alibi_slopes(h).astype(np.float32))


def test_workloads_match_their_names():
    assert len(configs.WORKLOADS) == 6
    assert [w.index for w in configs.WORKLOADS] == list(range(1, 7))
    for w in configs.WORKLOADS:
        assert w.seq_len % w.n_ranks == 0 and 0 <= w.rank < w.n_ranks
        assert w.heads_q % w.heads_kv == 0
    assert configs.HEADLINE.seq_len == 131072 and configs.HEADLINE.layout == "zigzag"
    assert math.isclose(configs.get(4).std ** 2, 0.5)
    w4, w6 = configs.get(4), configs.get(6)
    assert (w6.heads_q, w6.heads_kv, w6.seq_len, w6.layout, w6.alibi, w6.backward) == \
        (w4.heads_q, w4.heads_kv, w4.seq_len, w4.layout, True, True)


# ---------------------------------------------------------------------------
# size limits: every size the kernels cannot address is refused before any
# launch. Every call passes NULL tensors: a refused size returns
# RA_ERR_UNSUPPORTED, an accepted one fails the NULL check that follows the
# limit checks, so nothing is ever launched.
# ---------------------------------------------------------------------------

def _bwd(dims, ptr=None):
    return L.ra_step_bwd(ctypes.byref(dims), ptr, ptr, ptr, ptr, ptr, 1, 0.1, None, ptr, ptr, ptr, ptr, ptr, ptr,
                         None)


@pytest.mark.parametrize("d,limit", [(128, 4194304), (64, 8388608)])
def test_step_fwd_bf16_slab_limit(d, limit):
    # one head's fp32 o_acc slab (len_q * head_dim * 4 bytes) must stay below 2^31
    assert limit * d * 4 == 2 ** 31
    assert _fwd(_dims(d=d, lq=limit), ptr=None) == 2 and "slab" in _lib.ra_last_error()
    assert _fwd(_dims(d=d, lq=limit - 1), ptr=None) == 1 and "NULL" in _lib.ra_last_error()
    # the key length is addressed with 64-bit pointers in the forward step
    assert _fwd(_dims(d=d, lkv=limit), ptr=None) == 1


def test_step_bwd_slab_limits():
    limit = 2 ** 31 // (128 * 2)  # q / d_o and k / v slabs of one head, bf16
    assert _bwd(_dims(lq=limit)) == 2 and "q / d_o" in _lib.ra_last_error()
    assert _bwd(_dims(lkv=limit)) == 2 and "k / v" in _lib.ra_last_error()
    assert _bwd(_dims(lq=limit - 1, lkv=limit - 1), ptr=None) == 1 and "NULL" in _lib.ra_last_error()


def test_grid_limits():
    # batch x heads x row tiles must fit the int32 grid
    assert _fwd(_dims(b=2 ** 16, hq=2 ** 8, hkv=1, lq=256 * 128), ptr=None) == 2 and "grid" in _lib.ra_last_error()
    assert _fwd(_dims(b=2 ** 16, hq=2 ** 8, hkv=1, lq=32 * 256, dt=_lib.RA_FP32, d=64), ptr=None) == 2
    assert _bwd(_dims(b=2 ** 16, hq=2 ** 8, hkv=1, lq=128 * 128)) == 2 and "grid" in _lib.ra_last_error()
    assert _fwd(_dims(b=2 ** 16, hq=2 ** 7, hkv=1, lq=128), ptr=None) == 1


def test_limits_do_not_apply_to_empty_work():
    assert _fwd(_dims(lq=2 ** 30, b=0), ptr=None) == 0
    assert _bwd(_dims(lq=2 ** 30, lkv=0), ptr=None) == 0


def test_count_nonfinite_validation():
    n = ctypes.c_int64(7)
    assert L.ra_count_nonfinite(1, 4, 0, None, None) == 1 and "count" in _lib.ra_last_error()
    assert L.ra_count_nonfinite(1, -1, 0, ctypes.byref(n), None) == 1
    assert L.ra_count_nonfinite(1, 4, 9, ctypes.byref(n), None) == 1 and "dtype" in _lib.ra_last_error()
    assert L.ra_count_nonfinite(None, 4, 0, ctypes.byref(n), None) == 1 and "NULL" in _lib.ra_last_error()
    assert L.ra_count_nonfinite(None, 0, 0, ctypes.byref(n), None) == 0 and n.value == 0


def test_bind_records_one_call_and_defers_it():
    # A bound call marshals now and calls the library only when invoked; the
    # invalid call below (NULL output) is rejected by the library's host-side
    # checks, before any launch.
    call = _lib.bind(lambda: _lib._invoke("ra_positions", 16, 4, 0, 0, None, None))
    assert callable(call)
    with pytest.raises(_lib.RaError) as err:
        call()
    assert err.value.status == _lib.RA_ERR_INVALID_ARGUMENT
    with pytest.raises(ValueError):
        _lib.bind(lambda: None)  # records no call

    def two_calls():
        _lib._invoke("ra_positions", 16, 4, 0, 0, None, None)
        _lib._invoke("ra_positions", 16, 4, 0, 0, None, None)

    with pytest.raises(ValueError):
        _lib.bind(two_calls)
    with pytest.raises(ValueError):
        _lib.bind(_lib.ra_positions, 16, 4, 0, "zigzag", torch.zeros(4, dtype=torch.int32))  # host tensor
    # recording ended: a direct call reaches the library again
    with pytest.raises(_lib.RaError):
        _lib._invoke("ra_positions", 16, 4, 0, 0, None, None)
