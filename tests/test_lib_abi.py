"""Host-only checks of the C ABI: the library loads, exports every entry point
include/mla.h declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_34_amd as mla
from mla_latent_kv_34_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        from mla_latent_kv_34_amd import build
        build.build()
    return mla.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(mla.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(["MLA_OK", "MLA_ERR_INVALID_ARG", "MLA_ERR_UNSUPPORTED",
                                 "MLA_ERR_WORKSPACE", "MLA_ERR_HIP"]):
        assert lib.mla_status_string(code).decode() == name


def _dims(**kw):
    base = dict(n_heads=128, d_nope=128, d_rope=64, d_latent=512, page_size=64, dtype=0,
                sm_scale=0.0, reserved=0.0, rope_base=10000.0)
    base.update(kw)
    return _lib._Dims(**base)


def test_invalid_arguments_rejected_on_host(lib):
    d = _dims()
    cache = _lib._Cache(None, 1, 1, None)
    st = lib.mla_cache_append(ctypes.byref(d), ctypes.byref(cache), 1, None, 1, None, None, None)
    assert st == mla.MLA_ERR_INVALID_ARG
    assert b"NULL" in lib.mla_last_error()
    bad = _dims(d_rope=63)
    st = lib.mla_cache_append(ctypes.byref(bad), ctypes.byref(cache), 1, None, 1, None, None, None)
    assert st == mla.MLA_ERR_INVALID_ARG and b"d_rope" in lib.mla_last_error()
    big = _dims(d_latent=4096, n_heads=16)
    st = lib.mla_decode(ctypes.byref(big), ctypes.byref(cache), 1, None, None, None, None, None, None,
                        None, 0, 0, None, None)
    assert st == mla.MLA_ERR_UNSUPPORTED
    assert lib.mla_decode_workspace_size(None, 1, 0) == 0
    assert lib.mla_prefill_workspace_size(ctypes.byref(_dims()), 0, 10) == 0


def test_misaligned_pointer_rejected(lib):
    d = _dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, dtype=1)
    cache = _lib._Cache(0x1008, 2, 2, 0x2000)   # never dereferenced: validation fails first
    st = lib.mla_cache_append(ctypes.byref(d), ctypes.byref(cache), 1, 0x3000, 1, 0x4000, 0x5000, None)
    assert st == mla.MLA_ERR_INVALID_ARG and b"aligned" in lib.mla_last_error()


def test_workspace_size_generic_family_needs_no_device(lib):
    d = _dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, dtype=1)
    assert lib.mla_decode_workspace_size(ctypes.byref(d), 3, 0) == 0
    # generic prefill: fp32 K^C and V^C for every prompt token and head
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 2, 10) == 2 * 10 * 2 * 4 * 16 * 4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(mla.LibraryMissing):
        _lib.load()


def test_decode_hidden_rejections_on_host(lib):
    """mla_decode_hidden validates before anything is launched: the generic
    family is unsupported, K sizes must be positive multiples of 64, and the
    workspace size query returns 0 for sizes it does not implement."""
    cache = _lib._Cache(0x1000, 1, 1, 0x2000)   # never dereferenced
    args = lambda d, dm, dq: (ctypes.byref(d), ctypes.byref(cache), 1, 0x3000, dm, dq,  # noqa: E731
                              0x4000, 0x5000, 0x6000, 0x7000, 0x8000, 0x9000, 0xa000, 0xb000, 0xc000,
                              0xd000, 1 << 30, 0, None, None)
    tiny = _dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, dtype=1)
    assert lib.mla_decode_hidden(*args(tiny, 128, 0)) == mla.MLA_ERR_INVALID_ARG   # generic: any K >= 1
    assert b"d_q" in lib.mla_last_error()
    v2 = _dims()
    assert lib.mla_decode_hidden(*args(v2, 5000, 1536)) == mla.MLA_ERR_INVALID_ARG
    assert b"d_model" in lib.mla_last_error()
    assert lib.mla_decode_hidden(*args(v2, 5120, 0)) == mla.MLA_ERR_INVALID_ARG
    assert b"d_q" in lib.mla_last_error()
    assert lib.mla_decode_hidden_workspace_size(ctypes.byref(tiny), 4, 0, 128, 48) > 0
    assert lib.mla_decode_hidden_workspace_size(ctypes.byref(tiny), 4, 0, 128, 0) == 0
    assert lib.mla_decode_hidden_workspace_size(ctypes.byref(v2), 4, 0, 5000, 1536) == 0


def test_prefill_chunk_rejections_on_host(lib):
    """mla_prefill_chunk validates before anything is launched: start_pos is
    required, max_context must cover the chunk and fit the page table, and the
    workspace must cover max_context positions per sequence."""
    d = _dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, dtype=1)
    cache = _lib._Cache(0x1000, 4, 2, 0x2000)   # 2 pages of 64 positions per sequence
    def call(start, T, ctx, ws_bytes=1 << 30):
        return lib.mla_prefill_chunk(ctypes.byref(d), ctypes.byref(cache), 1, start, T, ctx, 0, 0x4000, 0x5000,
                                     0x6000, 0x7000, 0x8000, 0x9000, 0xa000, 0xb000, ws_bytes, None, None)
    assert call(None, 8, 64) == mla.MLA_ERR_INVALID_ARG and b"start_pos" in lib.mla_last_error()
    assert call(0x3000, 8, 7) == mla.MLA_ERR_INVALID_ARG and b"max_context" in lib.mla_last_error()
    assert call(0x3000, 8, 129) == mla.MLA_ERR_INVALID_ARG and b"page_table" in lib.mla_last_error()
    assert call(0x3002, 8, 64) == mla.MLA_ERR_INVALID_ARG and b"aligned" in lib.mla_last_error()
    size = lambda dd, B, T, ctx, mode=0: lib.mla_prefill_chunk_workspace_size(  # noqa: E731
        ctypes.byref(dd), B, T, ctx, mode)
    need = size(d, 1, 8, 100)
    assert need == 100 * 2 * 4 * 16 * 4                  # fp32 K^C and V^C for 100 positions
    assert size(d, 1, 8, 100, mla.CHUNK_EXPAND) == need
    assert call(0x3000, 8, 100, need - 1) == mla.MLA_ERR_WORKSPACE
    assert size(d, 1, 8, 7) == 0
    assert size(d, 1, 8, 100, mla.CHUNK_ABSORB) == 0     # the absorbed form: V2 sizes only
    assert size(d, 1, 8, 100, 3) == 0                    # not a mode
    # a whole prompt is the chunk at start 0 with max_context = its length
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 3, 50) == size(d, 3, 50, 50)
    v2 = _dims()
    assert lib.mla_prefill_workspace_size(ctypes.byref(v2), 2, 4096) == size(v2, 2, 4096, 4096)
    assert size(v2, 2, 512, 4096) > size(v2, 2, 512, 512)
    assert size(v2, 2, 512, 4096, mla.CHUNK_ABSORB) == 0  # above 256 tokens


def test_layer_and_merge_rejections_on_host(lib):
    """The layer, merged-weight and merge entry points validate on the host:
    the merged forms exist for the V2 sizes only, K sizes must be positive
    (multiples of 64 for the V2 sizes), and a NULL weight is named in the error."""
    cache = _lib._Cache(0x1000, 1, 1, 0x2000)   # never dereferenced
    tiny = _dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, dtype=1)
    v2 = _dims()
    P = [0x4000 + 0x1000 * i for i in range(12)]

    # pointer arguments in order: h, W^DKV, W^KR, W^DQ, W^UQ, W^QR, W^UK, then
    # W^UV, W^O (mla_decode_layer) or W^OV (mla_decode_layer_merged), then u, workspace
    def layer(fn, n_ptr, d, dm, dq, nulled=None):
        ptrs = list(P[:n_ptr])
        if nulled is not None:
            ptrs[nulled] = None
        return fn(ctypes.byref(d), ctypes.byref(cache), 1, 0x3000, dm, dq, *ptrs, 1 << 30, 0, None, None)

    for fn, n_ptr, name in ((lib.mla_decode_layer, 11, b"w_o"), (lib.mla_decode_layer_merged, 10, b"w_ov")):
        assert len(fn.argtypes) == 6 + n_ptr + 4
        if fn is lib.mla_decode_layer_merged:
            assert layer(fn, n_ptr, tiny, 128, 64) == mla.MLA_ERR_UNSUPPORTED   # merged: V2 only
        else:
            assert layer(fn, n_ptr, tiny, 128, 0) == mla.MLA_ERR_INVALID_ARG
        assert layer(fn, n_ptr, v2, 5000, 1536) == mla.MLA_ERR_INVALID_ARG
        assert b"d_model" in lib.mla_last_error()
        assert layer(fn, n_ptr, v2, 5120, 1536, nulled=n_ptr - 3) == mla.MLA_ERR_INVALID_ARG
        assert name + b" is NULL" in lib.mla_last_error(), lib.mla_last_error()
    assert len(lib.mla_decode_hidden_merged.argtypes) == 6 + 9 + 4
    hm = lambda d, dm, dq: lib.mla_decode_hidden_merged(  # noqa: E731
        ctypes.byref(d), ctypes.byref(cache), 1, 0x3000, dm, dq, *P[:9], 1 << 30, 0, None, None)
    assert hm(tiny, 128, 64) == mla.MLA_ERR_UNSUPPORTED
    assert hm(v2, 5120, 100) == mla.MLA_ERR_INVALID_ARG and b"d_q" in lib.mla_last_error()
    assert lib.mla_merge_query_weights(ctypes.byref(tiny), 64, P[0], P[1], P[2], None) == mla.MLA_ERR_UNSUPPORTED
    assert lib.mla_merge_query_weights(ctypes.byref(v2), 1536, P[0], None, P[2], None) == mla.MLA_ERR_INVALID_ARG
    assert b"w_uk" in lib.mla_last_error()
    assert lib.mla_merge_output_weights(ctypes.byref(v2), 5000, P[0], P[1], P[2], None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_merge_output_weights(ctypes.byref(v2), 5120, P[0], P[1], None, None) == mla.MLA_ERR_INVALID_ARG
    assert b"w_ov" in lib.mla_last_error()


def test_noalloc_step_rejections_on_host(lib):
    """mla_decode_step_noalloc exists for the V2 sizes only and checks its
    pointers before looking at any device."""
    cache = _lib._Cache(0x1000, 1, 1, 0x2000)
    P = [0x4000 + 0x1000 * i for i in range(8)]
    tiny = _dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, dtype=1)
    v2 = _dims()
    call = lambda d, ptrs: lib.mla_decode_step_noalloc(  # noqa: E731
        ctypes.byref(d), ctypes.byref(cache), 2, 0x3000, *ptrs, 0, None, None)
    assert call(tiny, P[:7]) == mla.MLA_ERR_UNSUPPORTED
    bad = list(P[:7])
    bad[4] = None                                        # w_uk
    assert call(v2, bad) == mla.MLA_ERR_INVALID_ARG and b"w_uk" in lib.mla_last_error()
