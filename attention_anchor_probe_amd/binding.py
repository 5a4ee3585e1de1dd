"""ctypes binding of libacache.so (the C ABI in include/acache.h).

Argument marshalling only: each function checks tensor placement, dtype and
contiguity, turns tensors into device pointers and calls the C entry point of
the same name on the given stream (torch's current HIP stream by default);
workspaces it allocates itself are allocated on that stream.  Every step of
the path runs in the library's HIP kernels; nothing here computes.  If the
library is missing the first call fails: there is no fallback.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libacache.so")

ACACHE_F32, ACACHE_BF16 = 0, 1
_DT = {torch.float32: ACACHE_F32, torch.bfloat16: ACACHE_BF16}

STATUS = {0: "OK", -1: "EINVAL", -2: "EDTYPE", -3: "ESHAPE", -4: "ERANGE", -5: "EREGION", -6: "EDUP",
          -7: "EWORKSPACE", -8: "EDEVICE", -9: "EALIGN"}


class AcacheError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({_lib().acache_status_string(status).decode()})")


class KVPool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("n_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class MapArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("affix_l", ctypes.c_int32), ("L", ctypes.c_int32), ("K", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("seq_len", ctypes.c_void_p), ("shared_slots", ctypes.c_void_p), ("private_pages", ctypes.c_void_p),
                ("private_page_offsets", ctypes.c_void_p), ("kv_offsets", ctypes.c_void_p),
                ("rc_offsets", ctypes.c_void_p), ("read_slot", ctypes.c_void_p), ("recompute_pos", ctypes.c_void_p),
                ("recompute_slot", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIG = {
    "acache_version": ([], ctypes.c_int),
    "acache_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "acache_anchor_count": ([_I, ctypes.c_double, ctypes.POINTER(_I)], ctypes.c_int),
    "acache_probe_workspace_bytes": ([_I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "acache_probe_scores": ([ctypes.POINTER(KVPool), _P, _I, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, ctypes.c_float,
                             _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "acache_probe_attention": ([ctypes.POINTER(KVPool), _P, _I, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P],
                               ctypes.c_int),
    "acache_probe_column_mass_workspace_bytes": ([_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
                                                 ctypes.c_int),
    "acache_probe_column_mass": ([ctypes.POINTER(KVPool), _P, _I, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I,
                                  ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "acache_topk_anchors": ([_P, _I, _I, _I, _I, _P, ctypes.POINTER(MapArgs), _P], ctypes.c_int),
    "acache_build_maps": ([_P, ctypes.POINTER(MapArgs), _P], ctypes.c_int),
    "acache_scatter_private": ([ctypes.POINTER(KVPool), _P, _P, _P, _I, _I, _I, _P], ctypes.c_int),
    "acache_block_slots": ([_P, _P, _P, _I, _I, _P, _P], ctypes.c_int),
    "acache_mapped_attention_workspace_bytes": ([_I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "acache_mapped_attention": ([ctypes.POINTER(KVPool), _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float,
                                 _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "acache_mapped_attention_shared_workspace_bytes": ([ctypes.POINTER(KVPool), _I, _I, _I, _I, _I, _I, _I,
                                                        ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "acache_mapped_attention_shared": ([ctypes.POINTER(KVPool), _P, _P, _I, _I, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                        _I, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "acache_mapped_attention_shared_noalloc": ([ctypes.POINTER(KVPool), _P, _P, _I, _I, _P, _P, _I, _P, _I, _I, _I,
                                                _I, _I, _I, ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "acache_store_attend_workspace_bytes": ([ctypes.POINTER(KVPool), _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
                                            ctypes.c_int),
    "acache_store_attend": ([ctypes.POINTER(KVPool), _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I,
                             _I, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "acache_hkvd_scores": ([ctypes.POINTER(KVPool), _P, _I, _P, _P, _I, _I, _I, _P, _P], ctypes.c_int),
    "acache_lse_merge": ([_I, ctypes.c_int64, _I, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "acache_kv_footprint": ([_I, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_uint64),
                             ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "acache_validate_slots": ([_P, _I, _P, _P, _I, _I, _I, ctypes.POINTER(_I)], ctypes.c_int),
    "acache_check_slots_workspace_bytes": ([_I, _I, _I, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "acache_check_slots": ([_P, _I, _P, _I, _P, _I, _I, _I, ctypes.POINTER(_I), _P, ctypes.c_size_t, _P],
                           ctypes.c_int),
    "acache_scatter_private_checked": ([ctypes.POINTER(KVPool), _P, _P, _P, _I, _P, _I, _P, _I, _I,
                                        ctypes.POINTER(_I), _P, ctypes.c_size_t, _P], ctypes.c_int),
}
EXPORTS = tuple(_SIG)

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIG.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def _check(fn, st):
    if st != 0:
        raise AcacheError(fn, st)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dev(t, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return _ptr(t)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _scratch(nbytes, device, stream):
    """A workspace for one call, allocated on the stream the call runs on: the
    caching allocator then hands its memory out again only to work ordered
    after the call's kernels on that stream."""
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream), device=device)
    with torch.cuda.stream(s):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def make_pool(k, v, page_size=None):
    """KVPool over tensors k, v of shape [n_layers][n_pages][n_kv_heads][page_size][head_dim]."""
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 5:
        raise ValueError("k and v must be [n_layers][n_pages][n_kv_heads][page_size][head_dim] of one dtype")
    if k.dtype not in _DT:
        raise ValueError(f"unsupported dtype {k.dtype}")
    N, npg, hkv, ps, d = k.shape
    if page_size is not None and page_size != ps:
        raise ValueError("page_size disagrees with the pool shape")
    return KVPool(_dev(k), _dev(v), _DT[k.dtype], N, npg, ps, hkv, d)


def acache_version():
    return _lib().acache_version()


def acache_anchor_count(L, rate):
    k = _I()
    _check("acache_anchor_count", _lib().acache_anchor_count(int(L), float(rate), ctypes.byref(k)))
    return k.value


def acache_probe_workspace_bytes(n_rows, B, L, n_q_heads, n_layers, lse_given):
    out = ctypes.c_size_t()
    _check("acache_probe_workspace_bytes",
           _lib().acache_probe_workspace_bytes(n_rows, B, L, n_q_heads, n_layers, int(bool(lse_given)),
                                               ctypes.byref(out)))
    return out.value


def acache_probe_scores(pool_k, pool_v, q, masked_rows, masked_offsets, shared_slots, scores, *, max_masked,
                        o_aff=None, lse_aff=None, layer_begin=0, scale=None, workspace=None, stream=None):
    """Probe (Eq. 4-5).  q: [n_layers][n_rows][Hq][d]; scores [B][L] fp32 is accumulated.
    The number of layers processed is q.shape[0], starting at pool layer `layer_begin`."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_rows, hq, d = q.shape
    B, L = scores.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = acache_probe_workspace_bytes(n_rows, B, L, hq, n_layers, lse_aff is not None)
    if workspace is None:
        workspace = _scratch(max(need, 1), q.device, stream)
    st = _lib().acache_probe_scores(
        ctypes.byref(pool), _dev(q, pool_k.dtype), n_rows, _dev(masked_rows, torch.int32),
        _dev(masked_offsets, torch.int32), masked_rows.numel(), int(max_masked), _dev(shared_slots, torch.int32), L, B,
        hq, layer_begin, n_layers, float(scale), _dev(scores, torch.float32), _dev(o_aff, pool_k.dtype),
        _dev(lse_aff, torch.float32), _dev(workspace), workspace.numel(), _stream(stream))
    _check("acache_probe_scores", st)


def acache_probe_attention(pool_k, pool_v, q, shared_slots, lse_aff, *, o_aff=None, layer_begin=0, scale=None,
                           stream=None):
    """Probe forward only: O_aff (nullable) and LSE_aff of every row over the affix."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_rows, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib().acache_probe_attention(ctypes.byref(pool), _dev(q, pool_k.dtype), n_rows,
                                       _dev(shared_slots, torch.int32), shared_slots.numel(), hq, layer_begin,
                                       n_layers, float(scale), _dev(o_aff, pool_k.dtype),
                                       _dev(lse_aff, torch.float32), _stream(stream))
    _check("acache_probe_attention", st)


def acache_probe_column_mass_workspace_bytes(n_rows, B, L, n_q_heads, n_layers):
    out = ctypes.c_size_t()
    _check("acache_probe_column_mass_workspace_bytes",
           _lib().acache_probe_column_mass_workspace_bytes(n_rows, B, L, n_q_heads, n_layers, ctypes.byref(out)))
    return out.value


def acache_probe_column_mass(pool_k, pool_v, q, masked_rows, masked_offsets, shared_slots, lse_aff, scores, *,
                             max_masked, layer_begin=0, scale=None, workspace=None, stream=None):
    """Column mass of the masked rows added to scores [B][L] (Eq. 5); lse_aff from acache_probe_attention."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_rows, hq, d = q.shape
    B, L = scores.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = acache_probe_column_mass_workspace_bytes(n_rows, B, L, hq, n_layers)
    if workspace is None:
        workspace = _scratch(max(need, 1), q.device, stream)
    st = _lib().acache_probe_column_mass(
        ctypes.byref(pool), _dev(q, pool_k.dtype), n_rows, _dev(masked_rows, torch.int32),
        _dev(masked_offsets, torch.int32), masked_rows.numel(), int(max_masked), _dev(shared_slots, torch.int32), L,
        B, hq, layer_begin, n_layers, float(scale), _dev(lse_aff, torch.float32), _dev(scores, torch.float32),
        _dev(workspace), workspace.numel(), _stream(stream))
    _check("acache_probe_column_mass", st)


def map_args(B, affix_l, L, K, page_size, max_seq_len, seq_len, shared_slots, private_pages, private_page_offsets,
             kv_offsets, rc_offsets, read_slot, recompute_pos=None, recompute_slot=None):
    i32 = torch.int32
    return MapArgs(B, affix_l, L, K, page_size, max_seq_len, _dev(seq_len, i32), _dev(shared_slots, i32),
                   _dev(private_pages, i32), _dev(private_page_offsets, i32), _dev(kv_offsets, i32),
                   _dev(rc_offsets, i32), _dev(read_slot, i32), _dev(recompute_pos, i32), _dev(recompute_slot, i32))


def acache_topk_anchors(scores, K, affix_l, anchors, maps=None, stream=None):
    """Top-K (Eq. 6) of scores [B][L] into anchors [B][K] (ascending positions);
    `maps` (a MapArgs) also builds the two maps."""
    B, L = scores.shape
    st = _lib().acache_topk_anchors(_dev(scores, torch.float32), B, L, int(K), int(affix_l),
                                    _dev(anchors, torch.int32), ctypes.byref(maps) if maps is not None else None,
                                    _stream(stream))
    _check("acache_topk_anchors", st)


def acache_build_maps(anchors, maps, stream=None):
    _check("acache_build_maps", _lib().acache_build_maps(_dev(anchors, torch.int32), ctypes.byref(maps),
                                                         _stream(stream)))


def acache_scatter_private(pool_k, pool_v, k_src, v_src, dst_slots, layer_begin=0, stream=None):
    """pool[layer_begin+n][dst_slots[i]] = src[n][i] for all KV heads.  src: [n_layers][n_rows][Hkv][d]."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_rows = k_src.shape[0], k_src.shape[1]
    st = _lib().acache_scatter_private(ctypes.byref(pool), _dev(k_src, pool_k.dtype), _dev(v_src, pool_k.dtype),
                                       _dev(dst_slots, torch.int32), n_rows, layer_begin, n_layers, _stream(stream))
    _check("acache_scatter_private", st)


ACACHE_CHECK_READ, ACACHE_CHECK_WRITE = 0, 1


def _check_ws(n_pages, page_size, mode, device, stream):
    ws_bytes = ctypes.c_size_t()
    _check("acache_check_slots_workspace_bytes",
           _lib().acache_check_slots_workspace_bytes(int(n_pages), int(page_size), int(mode), ctypes.byref(ws_bytes)))
    return _scratch(ws_bytes.value, device, stream)


def acache_check_slots(slots, n_pages, page_size, mode, offsets=None, page_owner=None, workspace=None,
                       stream=None):
    """Checked mode's device pre-pass over a slot table.  Returns (status,
    bad_index): status 0 (OK), or the first failing class ERANGE (-4),
    EREGION (-5), EDUP (-6) with its smallest failing entry.  Other errors
    raise AcacheError."""
    B = offsets.numel() - 1 if offsets is not None else 0
    if workspace is None:
        workspace = _check_ws(n_pages, page_size, mode, slots.device, stream)
    bad = _I(-2)
    st = _lib().acache_check_slots(_dev(slots, torch.int32), slots.numel(), _dev(offsets, torch.int32), B,
                                   _dev(page_owner, torch.int32), int(n_pages), int(page_size), int(mode),
                                   ctypes.byref(bad), _dev(workspace), workspace.numel(), _stream(stream))
    if st not in (0, -4, -5, -6):
        _check("acache_check_slots", st)
    return st, bad.value


def acache_scatter_private_checked(pool_k, pool_v, k_src, v_src, dst_slots, row_offsets, page_owner, layer_begin=0,
                                   workspace=None, stream=None):
    """acache_scatter_private after the write-mode pre-pass: raises AcacheError
    (status ERANGE / EREGION / EDUP, bad_index set) with the pool untouched
    when a destination is out of range, outside its request's private pages
    or repeated."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_rows = k_src.shape[0], k_src.shape[1]
    B = row_offsets.numel() - 1
    if workspace is None:
        workspace = _check_ws(pool.n_pages, pool.page_size, ACACHE_CHECK_WRITE, pool_k.device, stream)
    bad = _I(-2)
    st = _lib().acache_scatter_private_checked(
        ctypes.byref(pool), _dev(k_src, pool_k.dtype), _dev(v_src, pool_k.dtype), _dev(dst_slots, torch.int32),
        n_rows, _dev(row_offsets, torch.int32), B, _dev(page_owner, torch.int32), layer_begin, n_layers,
        ctypes.byref(bad), _dev(workspace), workspace.numel(), _stream(stream))
    if st != 0:
        err = AcacheError("acache_scatter_private_checked", st)
        err.bad_index = bad.value
        raise err


def acache_block_slots(read_slot, kv_offsets, block_start, block_len, dst_slots, stream=None):
    B = block_start.numel()
    st = _lib().acache_block_slots(_dev(read_slot, torch.int32), _dev(kv_offsets, torch.int32),
                                   _dev(block_start, torch.int32), B, int(block_len), _dev(dst_slots, torch.int32),
                                   _stream(stream))
    _check("acache_block_slots", st)


def acache_mapped_attention(pool_k, pool_v, q, q_offsets, read_slot, kv_offsets, out, *, max_q_per_req,
                            max_kv_per_req, lse=None, layer_begin=0, scale=None, workspace=None, stream=None):
    """Read-slot attention.  q/out: [n_layers][n_q][Hq][d]."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_q, hq, d = q.shape
    B = q_offsets.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = ctypes.c_size_t()
    _check("acache_mapped_attention_workspace_bytes",
           _lib().acache_mapped_attention_workspace_bytes(B, n_q, hq, n_layers, ctypes.byref(ws_bytes)))
    if workspace is None and ws_bytes.value > 0:
        workspace = _scratch(ws_bytes.value, q.device, stream)
    st = _lib().acache_mapped_attention(
        ctypes.byref(pool), _dev(q, pool_k.dtype), _dev(q_offsets, torch.int32), n_q, int(max_q_per_req),
        _dev(read_slot, torch.int32), _dev(kv_offsets, torch.int32), int(max_kv_per_req), B, hq, layer_begin,
        n_layers, float(scale), _dev(out, pool_k.dtype), _dev(lse, torch.float32),
        _dev(workspace) if workspace is not None else None, workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check("acache_mapped_attention", st)


def acache_mapped_attention_shared_workspace_bytes(pool_k, pool_v, *, B, n_q, max_q_per_req, n_q_heads, n_layers,
                                                   max_kv_per_req, L):
    pool = make_pool(pool_k, pool_v)
    ws_bytes = ctypes.c_size_t()
    _check("acache_mapped_attention_shared_workspace_bytes",
           _lib().acache_mapped_attention_shared_workspace_bytes(
               ctypes.byref(pool), int(B), int(n_q), int(max_q_per_req), int(n_q_heads), int(n_layers),
               int(max_kv_per_req), int(L), ctypes.byref(ws_bytes)))
    return ws_bytes.value


def acache_mapped_attention_shared(pool_k, pool_v, q, q_offsets, read_slot, kv_offsets, shared_slots, out, *,
                                   affix_l, max_q_per_req, max_kv_per_req, lse=None, layer_begin=0, scale=None,
                                   workspace=None, stream=None):
    """Read-slot attention of a batch sharing one affix (same result as
    acache_mapped_attention).  q/out: [n_layers][n_q][Hq][d]; shared_slots [L]."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_q, hq, d = q.shape
    B = q_offsets.numel() - 1
    L = shared_slots.numel()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        nb = acache_mapped_attention_shared_workspace_bytes(
            pool_k, pool_v, B=B, n_q=n_q, max_q_per_req=max_q_per_req, n_q_heads=hq, n_layers=n_layers,
            max_kv_per_req=max_kv_per_req, L=L)
        if nb > 0:
            workspace = _scratch(nb, q.device, stream)
    st = _lib().acache_mapped_attention_shared(
        ctypes.byref(pool), _dev(q, pool_k.dtype), _dev(q_offsets, torch.int32), n_q, int(max_q_per_req),
        _dev(read_slot, torch.int32), _dev(kv_offsets, torch.int32), int(max_kv_per_req),
        _dev(shared_slots, torch.int32), int(affix_l), L, B, hq, layer_begin, n_layers, float(scale),
        _dev(out, pool_k.dtype), _dev(lse, torch.float32),
        _dev(workspace) if workspace is not None else None, workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check("acache_mapped_attention_shared", st)


def acache_mapped_attention_shared_noalloc(pool_k, pool_v, q, q_offsets, read_slot, kv_offsets, shared_slots, out,
                                           *, affix_l, max_q_per_req, max_kv_per_req, lse=None, layer_begin=0,
                                           scale=None, stream=None):
    """acache_mapped_attention_shared without a workspace: the library keeps
    the plan in its fixed per-GPU scratch array (calls on one GPU must not
    overlap; a plan beyond the array's size raises EWORKSPACE)."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_q, hq, d = q.shape
    B = q_offsets.numel() - 1
    L = shared_slots.numel()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib().acache_mapped_attention_shared_noalloc(
        ctypes.byref(pool), _dev(q, pool_k.dtype), _dev(q_offsets, torch.int32), n_q, int(max_q_per_req),
        _dev(read_slot, torch.int32), _dev(kv_offsets, torch.int32), int(max_kv_per_req),
        _dev(shared_slots, torch.int32), int(affix_l), L, B, hq, layer_begin, n_layers, float(scale),
        _dev(out, pool_k.dtype), _dev(lse, torch.float32), _stream(stream))
    _check("acache_mapped_attention_shared_noalloc", st)


def acache_store_attend_workspace_bytes(pool_k, pool_v, *, B, max_q_per_req, max_kv_per_req):
    pool = make_pool(pool_k, pool_v)
    ws_bytes = ctypes.c_size_t()
    _check("acache_store_attend_workspace_bytes",
           _lib().acache_store_attend_workspace_bytes(ctypes.byref(pool), int(B), int(max_q_per_req),
                                                      int(max_kv_per_req), ctypes.byref(ws_bytes)))
    return ws_bytes.value


def acache_store_attend(pool_k, pool_v, k_src, v_src, src_pos, src_slot, src_offsets, q, q_offsets, read_slot,
                        kv_offsets, out, *, max_q_per_req, max_kv_per_req, lse=None, layer_begin=0, scale=None,
                        workspace=None, stream=None):
    """Store the source rows to their private slots and attend through the
    read-slot map (same result as acache_scatter_private followed by
    acache_mapped_attention).  k_src/v_src: [n_layers][n_src][Hkv][d];
    src_pos/src_slot [n_src]; src_offsets [B+1]; q/out: [n_layers][n_q][Hq][d]."""
    pool = make_pool(pool_k, pool_v)
    n_layers, n_q, hq, d = q.shape
    B = q_offsets.numel() - 1
    n_src = src_slot.numel()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        nb = acache_store_attend_workspace_bytes(pool_k, pool_v, B=B, max_q_per_req=max_q_per_req,
                                                 max_kv_per_req=max_kv_per_req)
        if nb > 0:
            workspace = _scratch(nb, q.device, stream)
    st = _lib().acache_store_attend(
        ctypes.byref(pool), _dev(k_src, pool_k.dtype), _dev(v_src, pool_k.dtype), _dev(src_pos, torch.int32),
        _dev(src_slot, torch.int32), _dev(src_offsets, torch.int32), n_src, _dev(q, pool_k.dtype),
        _dev(q_offsets, torch.int32), n_q, int(max_q_per_req), _dev(read_slot, torch.int32),
        _dev(kv_offsets, torch.int32), int(max_kv_per_req), B, hq, layer_begin, n_layers, float(scale),
        _dev(out, pool_k.dtype), _dev(lse, torch.float32),
        _dev(workspace) if workspace is not None else None, workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check("acache_store_attend", st)


def acache_hkvd_scores(pool_k, pool_v, shared_slots, k_full, v_full, scores, layer_begin=0, stream=None):
    """HKVD deviation scores.  k_full/v_full: [n_layers][B][L][Hkv][d];
    scores [B][L] fp32, accumulated."""
    pool = make_pool(pool_k, pool_v)
    n_layers, B, L = k_full.shape[:3]
    st = _lib().acache_hkvd_scores(ctypes.byref(pool), _dev(shared_slots, torch.int32), int(L),
                                   _dev(k_full, pool_k.dtype), _dev(v_full, pool_k.dtype), int(B), int(layer_begin),
                                   int(n_layers), _dev(scores, torch.float32), _stream(stream))
    _check("acache_hkvd_scores", st)


def acache_lse_merge(lse_a, lse_b, lse, o_a=None, o_b=None, o=None, stream=None):
    """Merge two attentions over disjoint key sets.  lse_*: fp32 [..., H];
    o_*: [..., H, d] (all given or none)."""
    if o is not None:
        d = o.shape[-1]
        dt = o.dtype
        if o_a is None or o_b is None or o_a.dtype != dt or o_b.dtype != dt:
            raise ValueError("o_a, o_b and o must be given together with one dtype")
    else:
        d, dt = 16, torch.float32
    st = _lib().acache_lse_merge(_DT[dt], int(lse.numel()), int(d), _dev(o_a), _dev(lse_a, torch.float32),
                                 _dev(o_b), _dev(lse_b, torch.float32), _dev(o), _dev(lse, torch.float32),
                                 _stream(stream))
    _check("acache_lse_merge", st)


def acache_kv_footprint(seq_len, L, K, page_size, n_layers, n_kv_heads, head_dim, dtype="bf16"):
    """Bytes of the shared region, of all private regions and of a dense
    per-request cache (host arithmetic; seq_len is a host sequence)."""
    import numpy as np
    sl = np.ascontiguousarray(np.asarray(seq_len), dtype=np.int32)
    out = [ctypes.c_uint64() for _ in range(3)]
    dt = {"f32": 0, "bf16": 1}[dtype] if isinstance(dtype, str) else int(dtype)
    _check("acache_kv_footprint", _lib().acache_kv_footprint(
        len(sl), sl.ctypes.data_as(ctypes.c_void_p) if len(sl) else None, int(L), int(K), int(page_size),
        int(n_layers), int(n_kv_heads), int(head_dim), dt, *(ctypes.byref(x) for x in out)))
    return {"shared": out[0].value, "private": out[1].value, "dense": out[2].value}


def acache_validate_slots(slots, page_owner, n_pages, page_size, owner=None, distinct=True):
    """Host-side table check; slots/owner/page_owner are CPU int32 tensors or
    numpy arrays.  Returns (status, bad_index)."""
    import numpy as np

    def host(a):
        if a is None:
            return None, None
        arr = np.ascontiguousarray(a.cpu().numpy() if hasattr(a, "cpu") else a, dtype=np.int32)
        return arr, arr.ctypes.data_as(ctypes.c_void_p)

    s, sp = host(slots)
    o, op = host(owner)
    po, pop = host(page_owner)
    bad = _I(-1)
    st = _lib().acache_validate_slots(sp, len(s), op, pop, int(n_pages), int(page_size), int(bool(distinct)),
                                      ctypes.byref(bad))
    return st, bad.value
