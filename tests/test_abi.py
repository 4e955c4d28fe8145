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
    rc = lib.ssa_select(ctypes.byref(p), *([fake] * 15), fake, ctypes.c_size_t(16), None)
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


def test_key_layouts_checked(lib):
    """Whole-key entry points refuse split params and the split ones whole
    params; split keys need an aligned rest array unless the scored pairs
    cover the head; append checks its layout, sizes and pointers."""
    fake = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    big = ctypes.c_size_t(1 << 40)
    assert lib.ssa_workspace_bytes(ctypes.byref(good(key_layout=2))) == 0
    ps = good(key_layout=ssa.SSA_KEYS_SPLIT)
    pw = good()
    assert ssa.workspace_bytes(ps) == ssa.workspace_bytes(pw)
    ten = [fake] * 10
    assert lib.ssa_decode(ctypes.byref(ps), *ten, fake, big, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_attend(ctypes.byref(ps), *([fake] * 9), fake, big, None) == ssa.SSA_ERR_INVALID

    def split(p, k_rest, k_dom=fake):
        return lib.ssa_decode_split(ctypes.byref(p), fake, k_dom, k_rest, *([fake] * 8), fake,
                                    ctypes.c_size_t(16), None, None)

    def attend_split(p, k_rest):
        return lib.ssa_attend_split(ctypes.byref(p), fake, fake, k_rest, *([fake] * 7), fake,
                                    ctypes.c_size_t(16), None)

    assert split(pw, fake) == ssa.SSA_ERR_INVALID
    assert split(ps, None) == ssa.SSA_ERR_INVALID
    assert split(ps, mis) == ssa.SSA_ERR_INVALID
    assert split(ps, fake, k_dom=mis) == ssa.SSA_ERR_INVALID
    assert attend_split(pw, fake) == ssa.SSA_ERR_INVALID
    assert attend_split(ps, None) == ssa.SSA_ERR_INVALID
    # past the layout checks the (too small) workspace is what fails
    assert split(ps, fake) == ssa.SSA_ERR_WORKSPACE
    assert attend_split(ps, fake) == ssa.SSA_ERR_WORKSPACE
    whole_head = good(key_layout=ssa.SSA_KEYS_SPLIT, pair_begin=0, pair_count=64)
    assert split(whole_head, None) == ssa.SSA_ERR_WORKSPACE

    def append(p, n, k_rest, k_cache=fake):
        return lib.ssa_append_kv(ctypes.byref(p), n, fake, fake, fake, fake, k_cache, k_rest,
                                 fake, None)

    assert append(pw, 1, fake) == ssa.SSA_ERR_INVALID        # whole keys take no rest array
    assert append(ps, 1, None) == ssa.SSA_ERR_INVALID        # split keys need one
    assert append(pw, -1, None) == ssa.SSA_ERR_INVALID
    assert append(pw, 1, None, k_cache=mis) == ssa.SSA_ERR_INVALID
    assert append(good(num_kv_heads=128, num_q_heads=128), 1, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_append_kv(ctypes.byref(pw), 1, None, fake, fake, fake, fake, None, fake,
                             None) == ssa.SSA_ERR_INVALID
    assert append(pw, 0, None) == ssa.SSA_OK                  # nothing to write
    assert append(ps, 0, fake) == ssa.SSA_OK
    assert lib.ssa_host_device_address(None, ctypes.byref(ctypes.c_void_p())) == ssa.SSA_ERR_INVALID
    assert lib.ssa_host_device_address(fake, None) == ssa.SSA_ERR_INVALID


@pytest.mark.parametrize("bad", [
    dict(max_seq_len=20000, max_blocks_per_seq=1250),           # stratum bound above 16384
    dict(max_seq_len=20000, max_blocks_per_seq=1250, max_topk=16385),
    dict(num_queries=8, query_group=8),                         # 8 members x 4 heads > 16 rows
    dict(max_topk=-1),
])
def test_early_stop_limits_rejected(lib, bad):
    """Early stopping is refused before any launch when the stratum could
    exceed its kernels' capacity or the unit has too many query rows."""
    p = good(early_stop=0.05, **bad)
    assert lib.ssa_workspace_bytes(ctypes.byref(p)) == 0
    fake = ctypes.c_void_p(4096)
    rc = lib.ssa_decode(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                        fake, fake, ctypes.c_size_t(1 << 40), None)
    assert rc == ssa.SSA_ERR_INVALID


def test_early_stop_within_limits_accepted(lib):
    for kw in (dict(), dict(max_seq_len=20000, max_blocks_per_seq=1250, max_topk=16384),
               dict(num_queries=8, query_group=4)):
        assert lib.ssa_workspace_bytes(ctypes.byref(good(early_stop=0.05, **kw))) > 0
    # without early stopping the bound is free
    assert lib.ssa_workspace_bytes(ctypes.byref(good(max_seq_len=20000,
                                                     max_blocks_per_seq=1250))) > 0


def test_early_stop_selection_needs_query_and_keys(lib):
    p = good(early_stop=0.05)
    n = ssa.workspace_bytes(p)
    fake = ctypes.c_void_p(4096)
    for q, k, bt in ((None, fake, fake), (fake, None, fake), (fake, fake, None)):
        rc = lib.ssa_select(ctypes.byref(p), fake, fake, fake, None, fake, fake, None, q, k,
                            None, bt, fake, fake, fake, fake, fake, ctypes.c_size_t(n), None)
        assert rc == ssa.SSA_ERR_INVALID


def test_measurement_aids_reject_bad_arguments_on_the_host(lib):
    # validation comes before any HIP call, so these run without a GPU
    fake = ctypes.c_void_p(1 << 20)
    assert lib.ssa_measure_stream(None, 16, fake, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_stream(fake, 24, fake, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_stream(fake, 0, fake, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_stream(ctypes.c_void_p((1 << 20) + 4), 16, fake, None) == \
        ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_gather(fake, 256, 0, fake, 4, fake, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_gather(fake, 256, 16, None, 4, fake, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_gather(fake, 256, 16, fake, -1, fake, None) == ssa.SSA_ERR_INVALID
    assert lib.ssa_measure_gather(fake, 256, 16, fake, 0, fake, None) == ssa.SSA_OK


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defines = dict(re.findall(r"#define (SSA_\w+) \(?(-?\d+)\)?", text))
    assert int(defines["SSA_MEASURE_SINK_WORDS"]) == ssa.MEASURE_SINK_WORDS
    assert int(defines["SSA_STOP_MAX_STRATUM"]) == ssa.STOP_MAX_STRATUM
    assert int(defines["SSA_STOP_MAX_ROWS"]) == ssa.STOP_MAX_ROWS
    assert int(defines["SSA_ERR_INVALID"]) == ssa.SSA_ERR_INVALID
    assert int(defines["SSA_OK"]) == ssa.SSA_OK
