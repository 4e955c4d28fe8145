"""The C ABI: the library loads on a CPU host, exports every declared entry
point, and rejects bad host-visible arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

from long_context_sparse_approx_amd import ssa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssa.LIB_PATH):
        pytest.skip("libssa.so not built")
    return ssa.lib()


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(ssa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(ssa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def good(**kw):
    base = dict(batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128, max_blocks_per_seq=64,
                num_blocks=128, max_seq_len=1000, pair_count=32)
    base.update(kw)
    return ssa.make_params(**base)


def test_workspace_size_for_valid_params(lib):
    p = good()
    n = ssa.workspace_bytes(p)
    assert n > 0 and n % 256 == 0
    assert ssa.num_chunks(p) == 1
    assert ssa.num_chunks(good(max_seq_len=1024, max_blocks_per_seq=64)) == 1
    assert ssa.num_chunks(good(max_seq_len=4097, max_blocks_per_seq=4097 // 16 + 1)) == 2
    # more chunks -> more workspace
    assert ssa.workspace_bytes(good(max_seq_len=20000, max_blocks_per_seq=1250)) > n


@pytest.mark.parametrize("bad", [
    dict(head_dim=96), dict(num_q_heads=30), dict(num_q_heads=8 * 17), dict(pair_count=12),
    dict(pair_count=0), dict(pair_begin=2), dict(pair_begin=-4), dict(pair_begin=40),
    dict(max_seq_len=1025), dict(max_seq_len=0), dict(block_size=32), dict(num_splits=-1),
    dict(out_dtype=7), dict(softmax_scale=-1.0), dict(softmax_scale=float("nan")),
    dict(batch=0), dict(num_kv_heads=0), dict(num_blocks=0), dict(num_queries=0),
    dict(query_group=0), dict(num_queries=257), dict(batch=4000, num_queries=4),
    dict(num_blocks=1 << 24, num_kv_heads=8),
])
def test_invalid_params_rejected(lib, bad):
    p = good(**bad)
    assert lib.ssa_workspace_bytes(ctypes.byref(p)) == 0
    assert lib.ssa_num_chunks(ctypes.byref(p)) == 0
    fake = ctypes.c_void_p(4096)
    rc = lib.ssa_decode(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                        fake, fake, ctypes.c_size_t(1 << 40), None)
    assert rc == ssa.SSA_ERR_INVALID


def test_null_and_misaligned_pointers_rejected(lib):
    p = good()
    fake = ctypes.c_void_p(4096)
    big = ctypes.c_size_t(1 << 40)
    # q, k, v, block_table, seq_lens, topk, top_p, sample_budget, seed, out
    args = [fake] * 10
    for i in range(10):
        if i == 6:  # top_p is optional
            continue
        a = list(args)
        a[i] = None
        rc = lib.ssa_decode(ctypes.byref(p), *a, fake, big, None)
        assert rc == ssa.SSA_ERR_INVALID, i
    mis = ctypes.c_void_p(4096 + 2)
    rc = lib.ssa_decode(ctypes.byref(p), mis, *args[1:], fake, big, None)
    assert rc == ssa.SSA_ERR_INVALID
    rc = lib.ssa_decode(ctypes.byref(p), *args, None, big, None)  # no workspace
    assert rc == ssa.SSA_ERR_INVALID


def test_small_workspace_rejected(lib):
    p = good()
    fake = ctypes.c_void_p(4096)
    n = ssa.workspace_bytes(p)
    rc = lib.ssa_decode(ctypes.byref(p), *([fake] * 10), fake, ctypes.c_size_t(n - 256), None)
    assert rc == ssa.SSA_ERR_WORKSPACE
    rc = lib.ssa_score(ctypes.byref(p), fake, fake, fake, fake, fake, fake, ctypes.c_size_t(16), None)
    assert rc == ssa.SSA_ERR_WORKSPACE
    rc = lib.ssa_select(ctypes.byref(p), *([fake] * 11), fake, ctypes.c_size_t(16), None)
    assert rc == ssa.SSA_ERR_WORKSPACE
    rc = lib.ssa_attend(ctypes.byref(p), *([fake] * 9), fake, ctypes.c_size_t(16), None)
    assert rc == ssa.SSA_ERR_WORKSPACE


def test_debug_hooks_validate(lib):
    assert lib.ssa_debug_philox(0, 0, 0, 0, 0, -1, ctypes.c_void_p(4096), None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_debug_philox(0, 0, 0, 0, 2**31 - 4, 8, ctypes.c_void_p(4096), None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_debug_philox(0, 0, 0, -1, 0, 4, ctypes.c_void_p(4096), None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_debug_philox(0, 0, 0, 0, 0, 0, ctypes.c_void_p(4096), None) == ssa.SSA_OK
    assert lib.ssa_debug_sexp(None, ctypes.c_void_p(4096), 4, None) == ssa.SSA_ERR_INVALID


def test_error_strings(lib):
    for code in (0, -1, -2, -3, 99):
        assert isinstance(ssa.error_string(code), str) and ssa.error_string(code)
