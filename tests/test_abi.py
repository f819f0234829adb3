"""The C ABI without a GPU: the built library loads, exports every entry point that
include/ctxattn.h declares, and rejects bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

from context_attention_lse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ctxattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libctxattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_error_string():
    lib = _lib.load()
    assert lib.ca_version().decode() == "0.1.0"
    assert isinstance(lib.ca_last_error(), bytes)


def _fake(n=0x1000):
    return ctypes.c_void_p(n)   # never dereferenced: validation fails first


def test_rejections_without_gpu():
    lib = _lib.load()
    st = _lib.ca_strides(0, 128, 0)
    # unknown dtype
    assert lib.ring_attn_step(_fake(), st, _fake(), _fake(), st, 9, 1, 1, 4, 4, 128, 0.0, 0, _fake(), _fake(), None, 0, None) == _lib.CA_ERR_DTYPE
    # bf16 head_dim other than 64 and 128
    assert lib.ring_attn_step(_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 96, 0.0, 0, _fake(), _fake(), None, 0, None) == _lib.CA_ERR_UNSUPPORTED
    assert b"64 or 128" in lib.ca_last_error()
    # sink lists need bf16 with head_dim 128 (the MFMA kernel)
    assert lib.ring_attn_const_max_step_sinks(_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 64, 0.0,
                                              _fake(), _fake(), 0, None, 0, None, _fake(), _fake(), 8, 0, None, 0,
                                              None) == _lib.CA_ERR_UNSUPPORTED
    # unknown mask
    assert lib.ring_attn_step(_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, 7, _fake(), _fake(), None, 0, None) == _lib.CA_ERR_UNSUPPORTED
    # NULL inputs
    assert lib.ring_attn_step(None, st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, 0, _fake(), _fake(), None, 0, None) == _lib.CA_ERR_NULL
    # misaligned q
    assert lib.ring_attn_step(_fake(0x1002), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, 0, _fake(), _fake(), None, 0, None) == _lib.CA_ERR_SHAPE
    # empty query shard is a no-op success
    assert lib.ring_attn_step(None, st, None, None, st, _lib.CA_BF16, 1, 1, 0, 0, 128, 0.0, 0, None, None, None, 0, None) == _lib.CA_OK
    # const-max: middle phase without an accumulator
    assert lib.ring_attn_const_max_step(_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, _fake(), None, 0, None, 0, None, None, 0, None) == _lib.CA_ERR_NULL
    # merge: n = 0, unsupported D, overlapping output
    assert lib.lse_merge(0, _fake(), _fake(), 4, 128, _fake(0x9000), 1, None, None) == _lib.CA_ERR_SHAPE
    assert lib.lse_merge(2, _fake(), _fake(), 4, 96, _fake(0x9000), 1, None, None) == _lib.CA_ERR_UNSUPPORTED
    assert lib.lse_merge(2, _fake(0x1000), _fake(), 4, 128, _fake(0x1400), 1, None, None) == _lib.CA_ERR_SHAPE
    # decode: head_dim other than 64 and 128, GQA group above 16, wrong block size, small workspace
    args = (_fake(), _fake(), _fake(), _fake(), _fake())
    assert lib.dcp_decode_partial(*args, 2, 64, 8, 96, 16, 8, 100, 0.0, _fake(), _fake(), _fake(), 1 << 30, None) == _lib.CA_ERR_UNSUPPORTED
    assert b"64 or 128" in lib.ca_last_error()
    assert lib.dcp_decode_partial(*args, 2, 64, 2, 128, 16, 8, 100, 0.0, _fake(), _fake(), _fake(), 1 << 30, None) == _lib.CA_ERR_UNSUPPORTED
    assert lib.dcp_decode_partial(*args, 2, 64, 8, 128, 32, 8, 100, 0.0, _fake(), _fake(), _fake(), 1 << 30, None) == _lib.CA_ERR_UNSUPPORTED
    assert lib.dcp_decode_partial(*args, 2, 64, 8, 128, 16, 8, 100, 0.0, _fake(), _fake(), _fake(), 16, None) == _lib.CA_ERR_WORKSPACE
    # a block table with entries over an empty pool: no block could stand in for missing ids
    assert lib.dcp_decode_partial(*args, 2, 64, 8, 128, 16, 8, 0, 0.0, _fake(), _fake(), _fake(), 1 << 30, None) == _lib.CA_ERR_SHAPE
    assert b"no block" in lib.ca_last_error()
    assert lib.dcp_decode_partial_active(_fake(), None, None, None, _fake(), _fake(), _fake(), 0, 2, 16, 2, 64, 8, 128,
                                         16, 8, 0, 0.0, _fake(), _fake(), _fake(), 1 << 30, None) == _lib.CA_ERR_SHAPE
    # the no-allocation decode: sizes over its fixed scratch are refused before any device call
    assert lib.dcp_decode_partial_noalloc(*args, 64, 64, 8, 128, 16, 8192, 100, 0.0, _fake(), _fake(), None) == _lib.CA_ERR_WORKSPACE
    assert b"scratch" in lib.ca_last_error()
    n = ctypes.c_size_t(0)
    assert lib.dcp_decode_workspace_size(32, 64, 128, 16, 4096, ctypes.byref(n)) == _lib.CA_OK
    assert n.value == 32 * 64 * 43 * 129 * 4   # 43 splits of 1536 tokens (an odd count)
    # chunk copy: misaligned pointer, size not a multiple of 16, empty copy
    assert lib.kv_chunk_copy(_fake(0x1008), _fake(), _fake(), _fake(), 4096, None) == _lib.CA_ERR_SHAPE
    assert lib.kv_chunk_copy(_fake(), _fake(0x2000), _fake(0x3000), _fake(0x4000), 4100, None) == _lib.CA_ERR_SHAPE
    assert lib.kv_chunk_copy(None, None, None, None, 0, None) == _lib.CA_OK
    # step workspace: fp32 never splits; bf16 needs one; too small a workspace is rejected
    n = ctypes.c_size_t(1)
    assert lib.ring_attn_workspace_size(_lib.CA_FP32, 1, 2, 300, 300, 64, 0, ctypes.byref(n)) == _lib.CA_OK
    assert n.value == 0
    assert lib.ring_attn_workspace_size(_lib.CA_BF16, 1, 2, 300, 300, 128, 2, ctypes.byref(n)) == _lib.CA_OK
    assert n.value > 0
    assert lib.ring_attn_workspace_size(_lib.CA_BF16, 1, 2, 300, 300, 128, 9, ctypes.byref(n)) == _lib.CA_ERR_UNSUPPORTED
    # bf16 with head_dim 64 runs on the vector kernel, which never splits
    n = ctypes.c_size_t(1)
    assert lib.ring_attn_workspace_size(_lib.CA_BF16, 1, 2, 300, 300, 64, 0, ctypes.byref(n)) == _lib.CA_OK
    assert n.value == 0
    assert lib.ring_attn_step(_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, 0, _fake(), _fake(),
                              _fake(0x10000), 16, None) == _lib.CA_ERR_WORKSPACE
    assert lib.ring_attn_step(_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, 0, _fake(), _fake(),
                              _fake(0x10010), 1 << 30, None) == _lib.CA_ERR_SHAPE   # misaligned workspace


def test_step_pair_rejections_without_gpu():
    lib = _lib.load()
    st = _lib.ca_strides(0, 128, 0)
    hops = (None,) * 8
    # first chunk not a multiple of 32 keys; fp32 (the pair runs on the MFMA kernel only); bf16 D = 64
    assert lib.ring_attn_step_pair(_fake(), st, _fake(), _fake(), _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 100,
                                   64, 128, 0.0, 0, _fake(), _fake(), None, 0, *hops, 0, None) == _lib.CA_ERR_UNSUPPORTED
    assert b"multiple of 32" in lib.ca_last_error()
    assert lib.ring_attn_step_pair(_fake(), st, _fake(), _fake(), _fake(), _fake(), st, _lib.CA_FP32, 1, 1, 4, 64,
                                   64, 128, 0.0, 0, _fake(), _fake(), None, 0, *hops, 0, None) == _lib.CA_ERR_UNSUPPORTED
    assert lib.ring_attn_step_pair(_fake(), st, _fake(), _fake(), _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 64,
                                   64, 64, 0.0, 0, _fake(), _fake(), None, 0, *hops, 0, None) == _lib.CA_ERR_UNSUPPORTED
    # a hop of a size that is not a multiple of 16
    assert lib.ring_attn_step_pair(_fake(), st, _fake(), _fake(), _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 64,
                                   64, 128, 0.0, 0, _fake(), _fake(), None, 0, _fake(0x2000), _fake(0x3000),
                                   _fake(0x4000), _fake(0x5000), None, None, None, None, 100, None) == _lib.CA_ERR_SHAPE


def test_hop_and_workspace_rejections_without_gpu():
    lib = _lib.load()
    st = _lib.ca_strides(0, 128, 0)
    step = (_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, 0, _fake(), _fake(), None, 0)
    for name in ("ring_attn_step_hop", "ring_attn_step_fold_hop"):
        fn = getattr(lib, name)
        # hop size not a multiple of 16, a misaligned hop pointer, a missing hop buffer
        assert fn(*step, _fake(0x2000), _fake(0x3000), _fake(0x4000), _fake(0x5000), 100, None) == _lib.CA_ERR_SHAPE
        assert fn(*step, _fake(0x2008), _fake(0x3000), _fake(0x4000), _fake(0x5000), 4096, None) == _lib.CA_ERR_SHAPE
        assert fn(*step, None, _fake(0x3000), _fake(0x4000), _fake(0x5000), 4096, None) == _lib.CA_ERR_NULL
        assert b"hop" in lib.ca_last_error()
        # no hop and no rows: nothing to do
        assert fn(None, st, None, None, st, _lib.CA_BF16, 1, 1, 0, 0, 128, 0.0, 0, None, None, None, 0,
                  None, None, None, None, 0, None) == _lib.CA_OK
    cm = (_fake(), st, _fake(), _fake(), st, _lib.CA_BF16, 1, 1, 4, 4, 128, 0.0, _fake(), _fake(), 0, None, 0, None,
          None, 0)
    assert lib.ring_attn_const_max_step_hop(*cm, _fake(0x2000), _fake(0x3000), _fake(0x4000), _fake(0x5000), 24,
                                            None) == _lib.CA_ERR_SHAPE
    # segmented prefill: the workspace holds the gathered prior K and V only
    n = ctypes.c_size_t(0)
    assert lib.segmented_attention_workspace_size(32, 8, 8192, 128, 32768, ctypes.byref(n)) == _lib.CA_OK
    assert n.value == 2 * 32768 * 8 * 128 * 2
    assert lib.segmented_attention_workspace_size(32, 8, 8192, 128, 0, ctypes.byref(n)) == _lib.CA_OK
    assert n.value == 0
