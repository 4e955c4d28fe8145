"""ctypes binding of libssa.so (include/ssa.h).  Argument marshalling only.

torch supplies device memory and the current stream; every step of the decode
path runs in the library's HIP kernels.  There is no fallback: if the library
is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssa.so")

SSA_OK = 0
SSA_ERR_INVALID = -1
SSA_ERR_WORKSPACE = -2
SSA_ERR_HIP = -3
SSA_ERR_STATIC_LIMIT = -4
STATIC_WORKSPACE_BYTES = 128 << 20
SSA_F32 = 0
SSA_BF16 = 1
SSA_KEYS_WHOLE = 0
SSA_KEYS_SPLIT = 1
STOP_MAX_STRATUM = 16384
STOP_MAX_ROWS = 16
MEASURE_SINK_WORDS = 4096
BLOCK_TOKENS = 16
CHUNK_TOKENS = 4096
STAGES = ("init", "index", "filter", "resolve", "sample", "attend", "merge")
EXPORTS = ("ssa_workspace_bytes", "ssa_num_chunks", "ssa_decode", "ssa_decode_static",
           "ssa_decode_timed",
           "ssa_decode_split", "ssa_score", "ssa_select", "ssa_attend", "ssa_attend_split",
           "ssa_append_kv", "ssa_host_device_address", "ssa_debug_philox", "ssa_debug_sexp",
           "ssa_debug_tail_exp",
           "ssa_measure_stream", "ssa_measure_gather", "ssa_error_string")


class SsaParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("pair_begin", ctypes.c_int32), ("pair_count", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("num_queries", ctypes.c_int32),
                ("query_group", ctypes.c_int32), ("early_stop", ctypes.c_float),
                ("key_layout", ctypes.c_int32), ("max_topk", ctypes.c_int32),
                ("refine", ctypes.c_int32)]


class SsaError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {error_string(code)} ({code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(SsaParams)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        L.ssa_workspace_bytes.argtypes = [_PP]
        L.ssa_workspace_bytes.restype = ctypes.c_size_t
        L.ssa_num_chunks.argtypes = [_PP]
        L.ssa_num_chunks.restype = ctypes.c_int32
        common = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.ssa_decode.argtypes = common
        L.ssa_decode.restype = ctypes.c_int
        L.ssa_decode_static.argtypes = common[:11] + [_P]
        L.ssa_decode_static.restype = ctypes.c_int
        L.ssa_decode_timed.argtypes = common + [_P]
        L.ssa_decode_timed.restype = ctypes.c_int
        L.ssa_decode_split.argtypes = ([_PP, _P, _P, _P] + common[3:] + [_P])
        L.ssa_decode_split.restype = ctypes.c_int
        L.ssa_score.argtypes = [_PP, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.ssa_score.restype = ctypes.c_int
        L.ssa_select.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _P, ctypes.c_size_t, _P]
        L.ssa_select.restype = ctypes.c_int
        L.ssa_attend.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.ssa_attend.restype = ctypes.c_int
        L.ssa_attend_split.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]
        L.ssa_attend_split.restype = ctypes.c_int
        L.ssa_append_kv.argtypes = [_PP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P]
        L.ssa_append_kv.restype = ctypes.c_int
        L.ssa_host_device_address.argtypes = [_P, ctypes.POINTER(ctypes.c_void_p)]
        L.ssa_host_device_address.restype = ctypes.c_int
        L.ssa_debug_philox.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]
        L.ssa_debug_philox.restype = ctypes.c_int
        L.ssa_debug_sexp.argtypes = [_P, _P, ctypes.c_int32, _P]
        L.ssa_debug_sexp.restype = ctypes.c_int
        L.ssa_debug_tail_exp.argtypes = [_P, _P, ctypes.c_int32, _P]
        L.ssa_debug_tail_exp.restype = ctypes.c_int
        L.ssa_measure_stream.argtypes = [_P, ctypes.c_size_t, _P, _P]
        L.ssa_measure_stream.restype = ctypes.c_int
        L.ssa_measure_gather.argtypes = [_P, ctypes.c_size_t, ctypes.c_int64, _P, ctypes.c_int64,
                                         _P, _P]
        L.ssa_measure_gather.restype = ctypes.c_int
        L.ssa_error_string.argtypes = [ctypes.c_int]
        L.ssa_error_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def error_string(code: int) -> str:
    return lib().ssa_error_string(code).decode()


def _check(code: int, what: str):
    if code != SSA_OK:
        raise SsaError(code, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def host_device_address(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor (torch's pin_memory), through
    the library; raises for memory the device cannot address."""
    assert not t.is_cuda and t.is_pinned(), "a pinned host tensor"
    out = ctypes.c_void_p()
    _check(lib().ssa_host_device_address(ctypes.c_void_p(t.data_ptr()), ctypes.byref(out)),
           "ssa_host_device_address")
    return int(out.value)


def _kv_ptr(t):
    """A cache argument: a device tensor, or a pinned host tensor (offloaded
    cache), passed by the address kernels use."""
    if t is None:
        return None
    if t.is_cuda:
        return ctypes.c_void_p(t.data_ptr())
    return ctypes.c_void_p(host_device_address(t))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_params(*, batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
                max_seq_len, pair_begin=None, pair_count=32, num_splits=0, out_dtype=SSA_F32,
                softmax_scale=0.0, block_size=BLOCK_TOKENS, num_queries=1,
                query_group=1, early_stop=0.0, key_layout=SSA_KEYS_WHOLE,
                max_topk=0, refine=0) -> SsaParams:
    if pair_begin is None:
        pair_begin = head_dim // 2 - pair_count
    return SsaParams(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_seq_len, pair_begin, pair_count, num_splits, out_dtype,
                     float(softmax_scale), int(num_queries), int(query_group),
                     float(early_stop), int(key_layout), int(max_topk), int(refine))


def params_for(q, k_cache, block_table, max_seq_len, **kw) -> SsaParams:
    """Params from tensor shapes: q [B, Hq, d] or [B, T, Hq, d] (T query
    positions per sequence), k_cache [nblk, Hkv, 16, d]."""
    if q.dim() == 3:
        B, Hq, d = q.shape
        T = 1
    else:
        B, T, Hq, d = q.shape
    kw.setdefault("num_queries", T)
    return make_params(batch=B, num_q_heads=Hq, num_kv_heads=k_cache.shape[1], head_dim=d,
                       max_blocks_per_seq=block_table.shape[1], num_blocks=k_cache.shape[0],
                       max_seq_len=int(max_seq_len), **kw)


def num_groups(p: SsaParams) -> int:
    g = min(p.query_group, p.num_queries)
    return -(-p.num_queries // g)


def selection_rows(p: SsaParams) -> int:
    """Selection units per sequence: groups x kv heads, or with refine one
    per query position and kv head (every member has its own selection)."""
    return (p.num_queries if p.refine > 0 else num_groups(p)) * p.num_kv_heads


def workspace_bytes(p: SsaParams) -> int:
    n = lib().ssa_workspace_bytes(ctypes.byref(p))
    if n == 0:
        raise SsaError(SSA_ERR_INVALID, "ssa_workspace_bytes")
    return int(n)


def num_chunks(p: SsaParams) -> int:
    return int(lib().ssa_num_chunks(ctypes.byref(p)))


def alloc_workspace(p: SsaParams, device) -> torch.Tensor:
    return torch.empty(workspace_bytes(p), dtype=torch.uint8, device=device)


def _ws(p, workspace, device):
    if workspace is None:
        workspace = alloc_workspace(p, device)
    return workspace


def _check_top_p(top_p, B):
    if top_p is not None:
        assert top_p.dtype == torch.float32 and top_p.numel() == B, "top_p: [B] float32"


def decode(p: SsaParams, q, k_cache, v_cache, block_table, seq_lens, topk, sample_budget, seed,
           out=None, workspace=None, stream=None, events=None, top_p=None):
    """One decode step; returns out [B, Hq, d] (f32 or bf16 per params).
    ``top_p`` ([B] float32 on the device, optional) caps the deterministic
    stratum at the top-p prefix."""
    _check_top_p(top_p, p.batch)
    if out is None:
        dt = torch.float32 if p.out_dtype == SSA_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    workspace = _ws(p, workspace, q.device)
    args = (ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(topk), _ptr(top_p), _ptr(sample_budget), _ptr(seed), _ptr(out),
            _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    if events is None:
        _check(lib().ssa_decode(*args), "ssa_decode")
    else:
        _check(lib().ssa_decode_timed(*args, ctypes.c_void_p(events)), "ssa_decode_timed")
    return out


def decode_static(p: SsaParams, q, k_cache, v_cache, block_table, seq_lens, topk,
                  sample_budget, seed, out=None, stream=None, top_p=None):
    """decode() with the library's own static device workspace (no
    workspace argument; the library allocates nothing).  Raises SsaError
    with SSA_ERR_STATIC_LIMIT when the step needs more than
    STATIC_WORKSPACE_BYTES."""
    _check_top_p(top_p, p.batch)
    if out is None:
        dt = torch.float32 if p.out_dtype == SSA_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    _check(lib().ssa_decode_static(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(topk), _ptr(top_p), _ptr(sample_budget), _ptr(seed), _ptr(out),
        _stream(stream)), "ssa_decode_static")
    return out


def decode_split(p: SsaParams, q, k_dom, k_rest, v_cache, block_table, seq_lens, topk,
                 sample_budget, seed, out=None, workspace=None, stream=None, events=None,
                 top_p=None):
    """One decode step over split keys (p.key_layout == SSA_KEYS_SPLIT):
    k_dom [nblk, Hkv, 16, 2*pair_count] on the device; k_rest
    [nblk, Hkv, 16, d - 2*pair_count] and v_cache on the device or in pinned
    host memory."""
    _check_top_p(top_p, p.batch)
    if out is None:
        dt = torch.float32 if p.out_dtype == SSA_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    workspace = _ws(p, workspace, q.device)
    _check(lib().ssa_decode_split(
        ctypes.byref(p), _ptr(q), _ptr(k_dom), _kv_ptr(k_rest), _kv_ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(topk), _ptr(top_p), _ptr(sample_budget),
        _ptr(seed), _ptr(out), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
        _stream(stream), None if events is None else ctypes.c_void_p(events)),
        "ssa_decode_split")
    return out


def append_kv(p: SsaParams, k_new, v_new, block_table, seq_lens, k_cache, k_rest, v_cache,
              stream=None):
    """Write k_new, v_new [B, T, Hkv, d] at positions seq_lens[b] - T + t of
    the cache (whole keys: k_rest None; split keys: k_cache gets the scored
    dims, k_rest the others)."""
    assert k_new.shape == v_new.shape and k_new.dim() == 4 and k_new.shape[0] == p.batch
    _check(lib().ssa_append_kv(ctypes.byref(p), int(k_new.shape[1]), _ptr(k_new), _ptr(v_new),
                               _ptr(block_table), _ptr(seq_lens), _kv_ptr(k_cache),
                               _kv_ptr(k_rest), _kv_ptr(v_cache), _stream(stream)),
           "ssa_append_kv")


def score(p: SsaParams, q, k_cache, block_table, seq_lens, scores=None, workspace=None,
          stream=None):
    """Approximate scores [B, NG*Hkv, max_seq_len] f32, one row per selection
    unit (group-major; entries past the unit's span untouched)."""
    if scores is None:
        scores = torch.zeros((p.batch, num_groups(p) * p.num_kv_heads, p.max_seq_len),
                             dtype=torch.float32, device=q.device)
    workspace = _ws(p, workspace, q.device)
    _check(lib().ssa_score(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(block_table),
                           _ptr(seq_lens), _ptr(scores), _ptr(workspace),
                           ctypes.c_size_t(workspace.numel()), _stream(stream)), "ssa_score")
    return scores


def select(p: SsaParams, scores, seq_lens, topk, sample_budget, seed, w_in=None, workspace=None,
           stream=None, top_p=None, q=None, k_cache=None, k_rest=None, block_table=None):
    """Selection from a score array: (sel_idx, sel_logw, sel_count, norm_out),
    each [B, NG*Hkv, ...] (one row per selection unit).  With early stopping
    (p.early_stop > 0) the query, keys (k_rest for split keys) and block
    table are needed too: the stratum is weighed by exact attention.  With
    refine (p.refine > 0) they are needed as well (each member scores the
    group's candidates), the selections are the members' ([B, T*Hkv, ...])
    and w_in, norm_out are per member."""
    _check_top_p(top_p, p.batch)
    dev = scores.device
    nc = num_chunks(p)
    UH = selection_rows(p)
    U = p.batch * UH
    sel_idx = torch.empty((p.batch, UH, nc * CHUNK_TOKENS), dtype=torch.int32, device=dev)
    sel_logw = torch.empty((p.batch, UH, nc * CHUNK_TOKENS), dtype=torch.float32, device=dev)
    sel_count = torch.empty((p.batch, UH, nc, 2), dtype=torch.int32, device=dev)
    norm = torch.empty((p.batch, UH, 2), dtype=torch.float32, device=dev)
    workspace = _ws(p, workspace, dev)
    assert w_in is None or w_in.numel() == U
    _check(lib().ssa_select(ctypes.byref(p), _ptr(scores), _ptr(seq_lens), _ptr(topk),
                            _ptr(top_p), _ptr(sample_budget), _ptr(seed), _ptr(w_in), _ptr(q),
                            _kv_ptr(k_cache), _kv_ptr(k_rest), _ptr(block_table), _ptr(sel_idx),
                            _ptr(sel_logw), _ptr(sel_count), _ptr(norm), _ptr(workspace),
                            ctypes.c_size_t(workspace.numel()), _stream(stream)), "ssa_select")
    return sel_idx, sel_logw, sel_count, norm


def attend(p: SsaParams, q, k_cache, v_cache, block_table, seq_lens, sel_idx, sel_logw, sel_count,
           out=None, workspace=None, stream=None):
    """Attention over a given selection; returns out [B, Hq, d]."""
    if out is None:
        dt = torch.float32 if p.out_dtype == SSA_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    workspace = _ws(p, workspace, q.device)
    _check(lib().ssa_attend(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                            _ptr(block_table), _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_logw),
                            _ptr(sel_count), _ptr(out), _ptr(workspace),
                            ctypes.c_size_t(workspace.numel()), _stream(stream)), "ssa_attend")
    return out


def attend_split(p: SsaParams, q, k_dom, k_rest, v_cache, block_table, seq_lens, sel_idx,
                 sel_logw, sel_count, out=None, workspace=None, stream=None):
    """attend() over split keys."""
    if out is None:
        dt = torch.float32 if p.out_dtype == SSA_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=dt, device=q.device)
    workspace = _ws(p, workspace, q.device)
    _check(lib().ssa_attend_split(ctypes.byref(p), _ptr(q), _ptr(k_dom), _kv_ptr(k_rest),
                                  _kv_ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                  _ptr(sel_idx), _ptr(sel_logw), _ptr(sel_count), _ptr(out),
                                  _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                  _stream(stream)), "ssa_attend_split")
    return out


def debug_philox(seed: int, b: int, h: int, j0: int, n: int, device="cuda", group: int = 0):
    words = torch.empty(n, dtype=torch.int32, device=device)
    _check(lib().ssa_debug_philox(ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), b, h, group, j0, n,
                                  _ptr(words), _stream(None)), "ssa_debug_philox")
    return words


def debug_sexp(x: torch.Tensor):
    y = torch.empty_like(x)
    _check(lib().ssa_debug_sexp(_ptr(x), _ptr(y), x.numel(), _stream(None)), "ssa_debug_sexp")
    return y


def debug_tail_exp(x: torch.Tensor):
    y = torch.empty_like(x)
    _check(lib().ssa_debug_tail_exp(_ptr(x), _ptr(y), x.numel(), _stream(None)),
           "ssa_debug_tail_exp")
    return y


def measure_stream(src: torch.Tensor, nbytes: int, sink: torch.Tensor, stream=None):
    """Contiguous read of the first nbytes of src (measurement aid); XOR of its
    32-bit words folded into sink (MEASURE_SINK_WORDS int32, cleared by the
    caller; the XOR of sink's words is the XOR of the data)."""
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the source tensor")
    if sink.numel() < MEASURE_SINK_WORDS or sink.element_size() != 4:
        raise ValueError("sink must hold MEASURE_SINK_WORDS 32-bit words")
    _check(lib().ssa_measure_stream(_ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "ssa_measure_stream")


def measure_gather(src: torch.Tensor, row_bytes: int, rows: torch.Tensor, sink: torch.Tensor,
                   stream=None):
    """Gather of the rows (int32 ids) of src viewed as rows of row_bytes
    (measurement aid); XOR of their 32-bit words folded into sink as in
    measure_stream."""
    if sink.numel() < MEASURE_SINK_WORDS or sink.element_size() != 4:
        raise ValueError("sink must hold MEASURE_SINK_WORDS 32-bit words")
    num_rows = src.numel() * src.element_size() // row_bytes
    _check(lib().ssa_measure_gather(_ptr(src), row_bytes, num_rows, _ptr(rows), rows.numel(),
                                    _ptr(sink), _stream(stream)), "ssa_measure_gather")


def decode_workload(wl, **kw):
    """Convenience: params + decode for a synth.Workload."""
    p = params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len, pair_begin=wl.pair_begin,
                   pair_count=wl.pair_count, **kw)
    return p, decode(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.topk,
                     wl.sample_budget, wl.seed)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
