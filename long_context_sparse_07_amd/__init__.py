"""Thin Python binding of liblsa.so, the MI355X hot path of LongCat Sparse Attention.

The functions carry the C ABI's names (lsa_index, lsa_block_means, lsa_select,
lsa_attend, lsa_workspace_clear) and only marshal arguments: they read shapes and
device pointers off torch tensors, allocate outputs/workspaces with torch (device
memory is the only thing torch provides here), pass the current HIP stream, and
raise on a non-zero status. All computation happens in the library's kernels;
there is no fallback path. See include/lsa.h for the contract of each call.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

__all__ = ["lib", "LSAError", "lsa_index", "lsa_block_means", "lsa_select", "lsa_index_select", "lsa_attend",
           "lsa_workspace_clear", "lsa_select_workspace_bytes", "lsa_attend_workspace_bytes",
           "LSA_BF16", "LSA_FP8_E4M3FN", "LSA_F32", "LSA_INDEX_TOKENS", "LSA_INDEX_BLOCKS",
           "LSA_WS_UNKNOWN", "LSA_WS_CLEAN", "LSA_WS_PRIMED", "lsa_select_attend", "lsa_index_select_attend",
           "lsa_cache_append", "lsa_attend_backward", "lsa_attend_noalloc", "lsa_index_target", "IndexTargetDesc", "IndexDesc", "BlockMeansDesc", "SelectDesc", "AttendDesc",
           "AttendBwdDesc", "CacheAppendDesc", "STATUS", "lsa_index_launch_events",
           "lsa_attend_launch_events"]

HERE = os.path.dirname(os.path.abspath(__file__))
# LSA_LIB_PATH selects another build of the same library (the host-sanitizer build that a
# CPU test runs the ABI checks against); by default the in-tree liblsa.so.
LIB_PATH = os.environ.get("LSA_LIB_PATH") or os.path.join(HERE, "liblsa.so")

LSA_BF16, LSA_FP8_E4M3FN, LSA_F32 = 1, 2, 3
LSA_INDEX_TOKENS, LSA_INDEX_BLOCKS = 0, 1
LSA_WS_UNKNOWN, LSA_WS_CLEAN, LSA_WS_PRIMED = 0, 1, 2
STATUS = {0: "LSA_OK", -1: "LSA_E_NULL", -2: "LSA_E_SHAPE", -3: "LSA_E_DTYPE", -4: "LSA_E_BUDGET",
          -5: "LSA_E_ALIGN", -6: "LSA_E_UNSUPPORTED", -7: "LSA_E_WORKSPACE", -8: "LSA_E_HIP"}


class IndexDesc(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("B", c_int32), ("T", c_int32), ("N", c_int32),
                ("ctx_len", c_void_p), ("H", c_int32), ("D", c_int32), ("q", c_void_p),
                ("w", c_void_p), ("k", c_void_p), ("k_dtype", c_int32), ("k_scale", c_void_p),
                ("kept", c_void_p), ("n_keep", c_int32), ("block_size", c_int32),
                ("n_blocks", c_int32), ("sink", c_int32), ("window", c_int32), ("scores", c_void_p),
                ("select_ws", c_void_p), ("select_ws_bytes", c_size_t), ("select_ws_state", c_int32),
                ("q_dtype", c_int32)]


class BlockMeansDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("N", c_int32), ("D", c_int32), ("k", c_void_p), ("k_dtype", c_int32),
                ("k_scale", c_void_p), ("block_size", c_int32), ("n_blocks", c_int32), ("kbar", c_void_p)]


class SelectDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("N", c_int32), ("ctx_len", c_void_p),
                ("scores", c_void_p), ("n_cols", c_int32), ("kept", c_void_p), ("n_keep", c_int32),
                ("block_size", c_int32), ("K", c_int32), ("sink", c_int32), ("window", c_int32),
                ("causal", c_int32), ("idx", c_void_p), ("workspace_state", c_int32)]


class CacheAppendDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("N", c_int32), ("D", c_int32), ("pos0", c_void_p),
                ("k_new", c_void_p), ("k_cache", c_void_p), ("k_dtype", c_int32), ("k_scale", c_void_p),
                ("n_rows", c_int32), ("rows_new", c_void_p * 2), ("rows_cache", c_void_p * 2),
                ("row_elems", c_int64 * 2), ("rows_stride_b", c_int64 * 2), ("rows_stride_n", c_int64 * 2),
                ("kbar", c_void_p), ("block_size", c_int32), ("n_blocks", c_int32)]


class AttendDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("N", c_int32), ("Hq", c_int32), ("Hkv", c_int32),
                ("d_qk", c_int32), ("d_v", c_int32), ("q", c_void_p), ("k", c_void_p),
                ("k_stride_b", c_int64), ("k_stride_n", c_int64), ("k_stride_h", c_int64),
                ("v", c_void_p), ("v_stride_b", c_int64), ("v_stride_n", c_int64), ("v_stride_h", c_int64),
                ("idx", c_void_p), ("K", c_int32), ("softmax_scale", c_float), ("out", c_void_p),
                ("out_dtype", c_int32), ("lse", c_void_p), ("n_layers", c_int32),
                ("layer_stride_q", c_int64), ("layer_stride_k", c_int64), ("layer_stride_v", c_int64),
                ("layer_stride_out", c_int64), ("layer_stride_lse", c_int64), ("n_splits", c_int32),
                ("block_table", c_void_p), ("page_size", c_int32), ("max_pages", c_int32), ("num_pages", c_int32),
                ("idx_shared", c_int32), ("ctx_len", c_void_p)]


class AttendBwdDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("N", c_int32), ("Hq", c_int32), ("Hkv", c_int32),
                ("d_qk", c_int32), ("d_v", c_int32), ("q", c_void_p), ("k", c_void_p),
                ("k_stride_b", c_int64), ("k_stride_n", c_int64), ("k_stride_h", c_int64),
                ("v", c_void_p), ("v_stride_b", c_int64), ("v_stride_n", c_int64), ("v_stride_h", c_int64),
                ("idx", c_void_p), ("K", c_int32), ("softmax_scale", c_float), ("out", c_void_p),
                ("lse", c_void_p), ("dout", c_void_p), ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p)]


class IndexTargetDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("N", c_int32), ("Hq", c_int32), ("Hkv", c_int32),
                ("d_qk", c_int32), ("q", c_void_p), ("k", c_void_p),
                ("k_stride_b", c_int64), ("k_stride_n", c_int64), ("k_stride_h", c_int64),
                ("idx", c_void_p), ("K", c_int32), ("softmax_scale", c_float), ("lse", c_void_p),
                ("scores", c_void_p), ("n_cols", c_int32), ("target", c_void_p), ("grad", c_void_p),
                ("loss", c_void_p)]


class LSAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded liblsa.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_07_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, desc in (("lsa_index", IndexDesc), ("lsa_block_means", BlockMeansDesc),
                           ("lsa_cache_append", CacheAppendDesc), ("lsa_index_target", IndexTargetDesc)):
            getattr(L, name).argtypes = [POINTER(desc), c_void_p]
            getattr(L, name).restype = c_int32
        L.lsa_select.argtypes = [POINTER(SelectDesc), c_void_p, c_size_t, c_void_p]
        L.lsa_select.restype = c_int32
        L.lsa_attend.argtypes = [POINTER(AttendDesc), c_void_p, c_size_t, c_void_p]
        L.lsa_attend.restype = c_int32
        L.lsa_index_select.argtypes = [POINTER(IndexDesc), c_int32, c_void_p, c_void_p, c_size_t, c_int32, c_void_p]
        L.lsa_index_select.restype = c_int32
        L.lsa_index_select_workspace_bytes.argtypes = [POINTER(IndexDesc), c_int32]
        L.lsa_index_select_workspace_bytes.restype = c_size_t
        L.lsa_attend_noalloc.argtypes = [POINTER(AttendDesc), c_void_p]
        L.lsa_attend_noalloc.restype = c_int32
        L.lsa_select_attend.argtypes = [POINTER(SelectDesc), POINTER(AttendDesc), c_void_p, c_size_t, c_void_p,
                                        c_size_t, c_void_p]
        L.lsa_select_attend.restype = c_int32
        L.lsa_select_workspace_bytes.argtypes = [POINTER(SelectDesc)]
        L.lsa_select_workspace_bytes.restype = c_size_t
        L.lsa_attend_workspace_bytes.argtypes = [POINTER(AttendDesc)]
        L.lsa_attend_workspace_bytes.restype = c_size_t
        L.lsa_attend_backward.argtypes = [POINTER(AttendBwdDesc), c_void_p, c_size_t, c_void_p]
        L.lsa_attend_backward.restype = c_int32
        L.lsa_attend_backward_workspace_bytes.argtypes = [POINTER(AttendBwdDesc)]
        L.lsa_attend_backward_workspace_bytes.restype = c_size_t
        L.lsa_workspace_clear.argtypes = [c_void_p, c_size_t, c_void_p]
        L.lsa_workspace_clear.restype = c_int32
        L.lsa_index_launch_events.argtypes = [c_void_p, c_void_p]
        L.lsa_index_launch_events.restype = c_int32
        L.lsa_attend_launch_events.argtypes = [c_void_p, c_void_p]
        L.lsa_attend_launch_events.restype = c_int32
        L.lsa_status_str.argtypes = [c_int32]
        L.lsa_status_str.restype = ctypes.c_char_p
        L.lsa_last_error.argtypes = []
        L.lsa_last_error.restype = ctypes.c_char_p
        L.lsa_version.argtypes = []
        L.lsa_version.restype = c_int32
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise LSAError(fn, rc, lib().lsa_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _kdtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return LSA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return LSA_FP8_E4M3FN
    if t.dtype == torch.float32:
        return LSA_F32
    raise TypeError(f"unsupported key dtype {t.dtype}")


# Workspaces are cached per (device, kind, shape key) and grown on demand. A select
# workspace is "clean" after a successful lsa_select with the same shape key (the
# library leaves its histogram/counters zeroed), which lets the next call skip its
# clearing kernel.
_ws = {}


def _workspace(kind: str, nbytes: int, device, shape_key=()):
    import torch
    key = (kind, str(device), shape_key)
    ent = _ws.get(key)
    if ent is None or ent[0].numel() < nbytes:
        ent = [torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device), False]
        _ws[key] = ent
    return ent


def _event_handle(ev):
    import torch
    if ev is None:
        return None
    if not ev.cuda_event:  # torch creates the event on its first record
        ev.record(torch.cuda.current_stream())
    return ev.cuda_event


def lsa_index_launch_events(start=None, stop=None):
    """The next token-indexer kernel launch (lsa_index, lsa_index_select) records its own
    start and end into these torch.cuda.Event objects (enable_timing=True); the events are
    created here if they have not been recorded yet. None, None clears the hook."""
    _check("lsa_index_launch_events", lib().lsa_index_launch_events(_event_handle(start), _event_handle(stop)))


def lsa_attend_launch_events(start=None, stop=None):
    """The next attention call (lsa_attend, lsa_attend_noalloc, lsa_select_attend) records
    the start of its attention kernel and the end of its last kernel (the split merge)
    into these torch.cuda.Event objects, as lsa_index_launch_events does for the indexer."""
    _check("lsa_attend_launch_events", lib().lsa_attend_launch_events(_event_handle(start), _event_handle(stop)))


def lsa_workspace_clear(buf, stream=None):
    _check("lsa_workspace_clear", lib().lsa_workspace_clear(buf.data_ptr(), buf.numel() * buf.element_size(), _stream(stream)))


def lsa_index(q, w, k, *, k_scale=None, ctx_len=None, kept=None, block_size=0, mode=LSA_INDEX_TOKENS,
              N=None, n_blocks=0, sink=0, window=0, scores=None, select_ws=None, select_ws_state=LSA_WS_UNKNOWN,
              q_fp8=False, stream=None):
    """Indexer scores. q bf16 [B,T,H,D], w fp32 [B,T,H]; k bf16/fp8 [B,N,D] (tokens) or
    fp32 block means [B,n_blocks,D] (mode=LSA_INDEX_BLOCKS, N = cache rows). With
    select_ws (a uint8 tensor), the selection workspace is primed for these scores.
    q_fp8: quantise each query row to fp8 and contract fp8 x fp8 (fp8 keys, D=128)."""
    import torch
    B, T, H, D = q.shape
    if mode == LSA_INDEX_TOKENS:
        N = k.shape[1] if N is None else N
        n_keep = kept.shape[-1] if kept is not None else 0
        n_out = n_keep * block_size if kept is not None else N
    else:
        n_blocks = n_blocks or k.shape[1]
        n_keep = 0
        n_out = n_blocks
    if scores is None:
        scores = torch.empty((B, T, n_out), dtype=torch.float32, device=q.device)
    d = IndexDesc(mode=mode, B=B, T=T, N=N, ctx_len=_ptr(ctx_len), H=H, D=D, q=_ptr(q), w=_ptr(w), k=_ptr(k),
                  k_dtype=_kdtype(k), k_scale=_ptr(k_scale), kept=_ptr(kept), n_keep=n_keep,
                  block_size=block_size, n_blocks=n_blocks, sink=sink, window=window, scores=_ptr(scores),
                  select_ws=_ptr(select_ws), select_ws_bytes=0 if select_ws is None else select_ws.numel(),
                  select_ws_state=select_ws_state, q_dtype=LSA_FP8_E4M3FN if q_fp8 else 0)
    _check("lsa_index", lib().lsa_index(ctypes.byref(d), _stream(stream)))
    return scores


def lsa_block_means(k, block_size, *, k_scale=None, n_blocks=None, kbar=None, stream=None):
    import torch
    B, N, D = k.shape
    n_blocks = N // block_size if n_blocks is None else n_blocks
    if kbar is None:
        kbar = torch.empty((B, n_blocks, D), dtype=torch.float32, device=k.device)
    d = BlockMeansDesc(B=B, N=N, D=D, k=_ptr(k), k_dtype=_kdtype(k), k_scale=_ptr(k_scale),
                       block_size=block_size, n_blocks=n_blocks, kbar=_ptr(kbar))
    _check("lsa_block_means", lib().lsa_block_means(ctypes.byref(d), _stream(stream)))
    return kbar


def _select_desc(scores, K, sink, window, N, ctx_len, kept, block_size, causal, idx):
    B, T, n_cols = scores.shape
    return SelectDesc(B=B, T=T, N=N, ctx_len=_ptr(ctx_len), scores=_ptr(scores), n_cols=n_cols,
                      kept=_ptr(kept), n_keep=kept.shape[-1] if kept is not None else 0,
                      block_size=block_size, K=K, sink=sink, window=window, causal=int(causal),
                      idx=_ptr(idx))


def lsa_select_workspace_bytes(scores, K, sink=0, window=0, *, N=None, kept=None, block_size=0, causal=True):
    d = _select_desc(scores, K, sink, window, N or scores.shape[-1], None, kept, block_size, causal, None)
    return lib().lsa_select_workspace_bytes(ctypes.byref(d))


def lsa_select(scores, K, sink=0, window=0, *, N=None, ctx_len=None, kept=None, block_size=0, causal=True,
               idx=None, workspace=None, workspace_state=LSA_WS_UNKNOWN, stream=None):
    """SI selection: idx int32 [B,T,K], ascending, -1 padded. With a caller workspace,
    workspace_state says what it holds (LSA_WS_PRIMED after lsa_index primed it)."""
    import torch
    B, T, n_cols = scores.shape
    N = n_cols if N is None else N
    if idx is None:
        idx = torch.empty((B, T, K), dtype=torch.int32, device=scores.device)
    d = _select_desc(scores, K, sink, window, N, ctx_len, kept, block_size, causal, idx)
    s = _stream(stream)
    need = lib().lsa_select_workspace_bytes(ctypes.byref(d))
    if workspace is not None:
        ws, ent = workspace, None
        d.workspace_state = workspace_state
    else:
        ent = _workspace("select", need, scores.device, (B, T, n_cols))
        ws = ent[0]
        d.workspace_state = 1 if ent[1] else 0
    _check("lsa_select", lib().lsa_select(ctypes.byref(d), ws.data_ptr(), ws.numel() * ws.element_size(), s))
    if ent is not None:
        ent[1] = True
    return idx


def lsa_index_select(q, w, k, K, sink, window, *, k_scale=None, ctx_len=None, kept=None, block_size=0,
                     scores=None, idx=None, q_fp8=False, with_scores=True, workspace=None, stream=None):
    """The indexer's scores and the causal selection from them (lsa_index_select): one C call
    (one launch where the shape allows) for flat rows; with a kept map (HI fine stage),
    lsa_index priming the selection workspace, then lsa_select on its scores. Returns
    (scores, idx); scores is None when with_scores is False and none was given (flat rows:
    the scores are then not written)."""
    import torch
    B, T = q.shape[0], q.shape[1]
    N = k.shape[1]
    n_cols = kept.shape[-1] * block_size if kept is not None else N
    if scores is None and (with_scores or kept is not None):
        scores = torch.empty((B, T, n_cols), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, T, K), dtype=torch.int32, device=q.device)
    if kept is None:
        H, D = q.shape[2], q.shape[3]
        d = IndexDesc(mode=LSA_INDEX_TOKENS, B=B, T=T, N=N, ctx_len=_ptr(ctx_len), H=H, D=D, q=_ptr(q), w=_ptr(w),
                      k=_ptr(k), k_dtype=_kdtype(k), k_scale=_ptr(k_scale), sink=sink, window=window,
                      scores=_ptr(scores), q_dtype=LSA_FP8_E4M3FN if q_fp8 else 0)
        need = lib().lsa_index_select_workspace_bytes(ctypes.byref(d), K)
        if workspace is not None:
            ws, ent, state = workspace, None, LSA_WS_UNKNOWN
        else:
            ent = _workspace("index_select", need, q.device, (B, T, N, H, D, d.k_dtype, d.q_dtype, scores is None))
            ws, state = ent[0], (LSA_WS_CLEAN if ent[1] else LSA_WS_UNKNOWN)
        _check("lsa_index_select", lib().lsa_index_select(ctypes.byref(d), K, idx.data_ptr(), ws.data_ptr(),
                                                          ws.numel(), state, _stream(stream)))
        if ent is not None:
            ent[1] = True
        return scores, idx
    d = _select_desc(scores, K, sink, window, N, ctx_len, kept, block_size, True, idx)
    need = lib().lsa_select_workspace_bytes(ctypes.byref(d))
    ent = _workspace("select", need, q.device, (B, T, n_cols))
    ws = ent[0]
    lsa_index(q, w, k, k_scale=k_scale, ctx_len=ctx_len, kept=kept, block_size=block_size, N=N, sink=sink,
              window=window, scores=scores, select_ws=ws, select_ws_state=LSA_WS_CLEAN if ent[1] else LSA_WS_UNKNOWN,
              q_fp8=q_fp8, stream=stream)
    ent[1] = False
    d.workspace_state = LSA_WS_PRIMED
    _check("lsa_select", lib().lsa_select(ctypes.byref(d), ws.data_ptr(), ws.numel(), _stream(stream)))
    ent[1] = True
    return scores, idx


def _attend_desc(q, k, v, idx, softmax_scale, out, lse, mla, n_splits, block_table=None, N=None, shared=False,
                 ctx_len=None):
    """q [L,B,T,Hq,dqk]; k,v [L,B,N,Hkv,d] (contiguous per layer). MLA: k [L,B,N,1,576], v=None.
    Paged (block_table int32 [B,max_pages]): k, v are page pools [L,num_pages,page_size,Hkv,d]
    and N (default max_pages * page_size) bounds the positions."""
    L, B, T, Hq, dqk = q.shape
    if mla:
        v = k
        dv = 512
    else:
        dv = v.shape[-1]
    K = idx.shape[-1]
    paged = {}
    if block_table is not None:
        num_pages, page_size, Hkv = k.shape[1], k.shape[2], k.shape[3]
        for t in (k, v):
            if t.shape[1:3] != k.shape[1:3] or t.stride(1) != page_size * t.stride(2):
                raise ValueError("paged k, v: pools [L, num_pages, page_size, Hkv, d] with whole pages")
        if str(block_table.dtype) != "torch.int32" or block_table.shape[0] != B or not block_table.is_contiguous():
            raise ValueError("block_table: contiguous int32 [B, max_pages]")
        max_pages = block_table.shape[1]
        N = max_pages * page_size if N is None else N
        paged = dict(block_table=_ptr(block_table), page_size=page_size, max_pages=max_pages, num_pages=num_pages)
        strides_k = (0, k.stride(2), k.stride(3))
        strides_v = (0, v.stride(2), v.stride(3))
    else:
        N, Hkv = k.shape[2], k.shape[3]
        strides_k = (k.stride(1), k.stride(2), k.stride(3))
        strides_v = (v.stride(1), v.stride(2), v.stride(3))
    return AttendDesc(B=B, T=T, N=N, Hq=Hq, Hkv=Hkv, d_qk=dqk, d_v=dv, q=_ptr(q), k=_ptr(k),
                      k_stride_b=strides_k[0], k_stride_n=strides_k[1], k_stride_h=strides_k[2],
                      v=_ptr(v), v_stride_b=strides_v[0], v_stride_n=strides_v[1], v_stride_h=strides_v[2],
                      idx=_ptr(idx), K=K, softmax_scale=softmax_scale, out=_ptr(out),
                      out_dtype=LSA_F32 if out is not None and out.dtype.is_floating_point and out.element_size() == 4 else LSA_BF16,
                      lse=_ptr(lse), n_layers=L, layer_stride_q=q.stride(0), layer_stride_k=k.stride(0),
                      layer_stride_v=v.stride(0), layer_stride_out=out.stride(0) if out is not None else 0,
                      layer_stride_lse=lse.stride(0) if lse is not None else 0, n_splits=n_splits,
                      idx_shared=int(bool(shared)), ctx_len=_ptr(ctx_len) if shared else None, **paged)


def lsa_attend(q, k, v, idx, softmax_scale, *, out=None, lse=None, out_dtype=None, with_lse=True,
               n_splits=0, workspace=None, block_table=None, N=None, shared=False, ctx_len=None, stream=None):
    """Sparse attention for L layers sharing idx. q bf16 [L,B,T,Hq,dqk]; k, v bf16
    [L,B,N,Hkv,d] (v=None: MLA latent rows, V = k[..., :512]); idx int32 [B,T,K].
    With block_table (int32 [B,max_pages]) k, v are page pools [L,num_pages,page_size,Hkv,d].
    shared=True: idx is int32 [B,K], one selection for all T tokens, token t masked to
    positions <= ctx_len[b] - T + t (ctx_len int32 [B] or None for N).
    Returns (out [L,B,T,Hq,dv], lse fp32 [L,B,T,Hq] or None)."""
    import torch
    L, B, T, Hq, dqk = q.shape
    mla = v is None
    dv = 512 if mla else v.shape[-1]
    if out is None:
        out = torch.empty((L, B, T, Hq, dv), dtype=out_dtype or torch.bfloat16, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((L, B, T, Hq), dtype=torch.float32, device=q.device)
    d = _attend_desc(q, k, v, idx, softmax_scale, out, lse, mla, n_splits, block_table, N, shared, ctx_len)
    s = _stream(stream)
    need = lib().lsa_attend_workspace_bytes(ctypes.byref(d))
    ws = workspace if workspace is not None else (_workspace("attend", need, q.device)[0] if need else None)
    _check("lsa_attend", lib().lsa_attend(ctypes.byref(d), _ptr(ws), 0 if ws is None else ws.numel(), s))
    return out, lse


def lsa_attend_noalloc(q, k, v, idx, softmax_scale, *, out=None, lse=None, out_dtype=None, with_lse=True,
                       n_splits=0, block_table=None, N=None, shared=False, ctx_len=None, stream=None):
    """lsa_attend without a workspace: the split partials go to the library's static
    per-GPU buffer (calls that overlap on one GPU race). Same arguments and results as
    lsa_attend (out and lse are allocated here only when not given)."""
    out, lse = _attend_outputs(q, v, out, lse, out_dtype, with_lse)
    d = _attend_desc(q, k, v, idx, softmax_scale, out, lse, v is None, n_splits, block_table, N, shared, ctx_len)
    _check("lsa_attend_noalloc", lib().lsa_attend_noalloc(ctypes.byref(d), _stream(stream)))
    return out, lse


def _attend_outputs(q, v, out, lse, out_dtype, with_lse):
    import torch
    L, B, T, Hq, dqk = q.shape
    dv = 512 if v is None else v.shape[-1]
    if out is None:
        out = torch.empty((L, B, T, Hq, dv), dtype=out_dtype or torch.bfloat16, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((L, B, T, Hq), dtype=torch.float32, device=q.device)
    return out, lse


def _select_attend_call(ds, da, sel_ent, q, stream):
    need_a = lib().lsa_attend_workspace_bytes(ctypes.byref(da))
    wa = _workspace("attend", need_a, q.device)[0] if need_a else None
    ws = sel_ent[0]
    _check("lsa_select_attend", lib().lsa_select_attend(ctypes.byref(ds), ctypes.byref(da), ws.data_ptr(), ws.numel(),
                                                        _ptr(wa), 0 if wa is None else wa.numel(), _stream(stream)))
    sel_ent[1] = True


def lsa_select_attend(scores, K, sink, window, q, k, v, softmax_scale, *, N=None, ctx_len=None, causal=True,
                      idx=None, out=None, lse=None, out_dtype=None, with_lse=True, n_splits=0, block_table=None,
                      stream=None):
    """lsa_select on scores, then lsa_attend on the positions it selects, as one chain
    (the attention kernel finishes the selection). Same arguments and results as the
    two calls (block_table: paged k, v as in lsa_attend); no kept map. Returns (idx, out, lse)."""
    import torch
    B, T, n_cols = scores.shape
    N = n_cols if N is None else N
    if idx is None:
        idx = torch.empty((B, T, K), dtype=torch.int32, device=scores.device)
    out, lse = _attend_outputs(q, v, out, lse, out_dtype, with_lse)
    ds = _select_desc(scores, K, sink, window, N, ctx_len, None, 0, causal, idx)
    da = _attend_desc(q, k, v, idx, softmax_scale, out, lse, v is None, n_splits, block_table, N)
    ent = _workspace("select", lib().lsa_select_workspace_bytes(ctypes.byref(ds)), scores.device, (B, T, n_cols))
    ds.workspace_state = LSA_WS_CLEAN if ent[1] else LSA_WS_UNKNOWN
    _select_attend_call(ds, da, ent, q, stream)
    return idx, out, lse


def lsa_index_select_attend(qI, w, kI, K, sink, window, q, k, v, softmax_scale, *, k_scale=None, ctx_len=None,
                            scores=None, idx=None, out=None, lse=None, out_dtype=None, with_lse=True, n_splits=0,
                            block_table=None, stream=None):
    """The whole flat decode path: lsa_index (priming the selection workspace), then
    lsa_select_attend on its scores. Returns (scores, idx, out, lse)."""
    import torch
    B, T = qI.shape[0], qI.shape[1]
    N = kI.shape[1]
    if scores is None:
        scores = torch.empty((B, T, N), dtype=torch.float32, device=qI.device)
    if idx is None:
        idx = torch.empty((B, T, K), dtype=torch.int32, device=qI.device)
    out, lse = _attend_outputs(q, v, out, lse, out_dtype, with_lse)
    ds = _select_desc(scores, K, sink, window, N, ctx_len, None, 0, True, idx)
    da = _attend_desc(q, k, v, idx, softmax_scale, out, lse, v is None, n_splits, block_table, N)
    ent = _workspace("select", lib().lsa_select_workspace_bytes(ctypes.byref(ds)), qI.device, (B, T, N))
    lsa_index(qI, w, kI, k_scale=k_scale, ctx_len=ctx_len, N=N, sink=sink, window=window, scores=scores,
              select_ws=ent[0], select_ws_state=LSA_WS_CLEAN if ent[1] else LSA_WS_UNKNOWN, stream=stream)
    ent[1] = False
    ds.workspace_state = LSA_WS_PRIMED
    _select_attend_call(ds, da, ent, q, stream)
    return scores, idx, out, lse


def lsa_attend_backward(q, k, v, idx, softmax_scale, out, lse, dout, *, dq=None, dk=None, dv=None,
                        workspace=None, stream=None):
    """Gradients of lsa_attend for one layer, selection fixed. q, out, dout bf16 [B,T,Hq,d];
    k, v bf16 [B,N,Hkv,d] (v=None: MLA latent rows); idx int32 [B,T,K] as lsa_select
    writes it; lse fp32 [B,T,Hq]. Returns fp32 (dq [B,T,Hq,d_qk], dk [B,N,Hkv,d_qk], dv
    [B,N,Hkv,d_v] or None for MLA, where dk is the latent row gradient). The call writes dk
    and dv only at the selected positions: buffers allocated here start at zero; buffers
    passed in keep their other rows."""
    import torch
    B, T, Hq, dqk = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    mla = v is None
    if mla:
        v = k
    dv_ = 512 if mla else v.shape[-1]
    dev = q.device
    dq = torch.empty((B, T, Hq, dqk), dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.zeros((B, N, Hkv, dqk), dtype=torch.float32, device=dev) if dk is None else dk
    if not mla and dv is None:
        dv = torch.zeros((B, N, Hkv, dv_), dtype=torch.float32, device=dev)
    d = AttendBwdDesc(B=B, T=T, N=N, Hq=Hq, Hkv=Hkv, d_qk=dqk, d_v=dv_, q=_ptr(q), k=_ptr(k),
                      k_stride_b=k.stride(0), k_stride_n=k.stride(1), k_stride_h=k.stride(2),
                      v=_ptr(v), v_stride_b=v.stride(0), v_stride_n=v.stride(1), v_stride_h=v.stride(2),
                      idx=_ptr(idx), K=idx.shape[-1], softmax_scale=softmax_scale, out=_ptr(out), lse=_ptr(lse),
                      dout=_ptr(dout), dq=_ptr(dq), dk=_ptr(dk), dv=_ptr(None if mla else dv))
    need = lib().lsa_attend_backward_workspace_bytes(ctypes.byref(d))
    ws = workspace if workspace is not None else (_workspace("attend_bwd", need, dev)[0] if need else None)
    _check("lsa_attend_backward", lib().lsa_attend_backward(ctypes.byref(d), _ptr(ws), 0 if ws is None else ws.numel(),
                                                            _stream(stream)))
    return dq, dk, (None if mla else dv)


def lsa_index_target(q, k, idx, softmax_scale, lse, scores, *, target=None, grad=None, loss=None, stream=None):
    """Indexer distillation target (one layer's attention). q bf16 [B,T,Hq,d_qk]; k bf16
    [B,N,Hkv,d_qk] (MLA latent rows: d_qk 576); idx int32 [B,T,K]; lse fp32 [B,T,Hq] from
    lsa_attend; scores fp32 [B,T,n_cols] (flat indexer scores). Returns (target [B,T,K],
    grad [B,T,K], loss [B,T]), fp32."""
    import torch
    B, T, Hq, dqk = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    K = idx.shape[-1]
    dev = q.device
    target = torch.empty((B, T, K), dtype=torch.float32, device=dev) if target is None else target
    grad = torch.empty((B, T, K), dtype=torch.float32, device=dev) if grad is None else grad
    loss = torch.empty((B, T), dtype=torch.float32, device=dev) if loss is None else loss
    d = IndexTargetDesc(B=B, T=T, N=N, Hq=Hq, Hkv=Hkv, d_qk=dqk, q=_ptr(q), k=_ptr(k), k_stride_b=k.stride(0),
                        k_stride_n=k.stride(1), k_stride_h=k.stride(2), idx=_ptr(idx), K=K,
                        softmax_scale=softmax_scale, lse=_ptr(lse), scores=_ptr(scores), n_cols=scores.shape[-1],
                        target=_ptr(target), grad=_ptr(grad), loss=_ptr(loss))
    _check("lsa_index_target", lib().lsa_index_target(ctypes.byref(d), _stream(stream)))
    return target, grad, loss


def lsa_cache_append(k_new, k_cache, *, k_scale=None, rows=(), pos0=None, kbar=None, block_size=0, stream=None):
    """Append T new tokens per sequence. k_new bf16 [B,T,D]; k_cache fp8 (with k_scale fp32
    [B,N]) or bf16 [B,N,D]; rows: up to two (new [B,T,...] bf16 contiguous, cache
    [B,N,...] bf16) pairs; pos0 int32 [B] (rows already cached; None = N - T); kbar fp32
    [B,n_blocks,D] updated for the blocks this append completes."""
    B, T, D = k_new.shape
    N = k_cache.shape[1]
    d = CacheAppendDesc(B=B, T=T, N=N, D=D, pos0=_ptr(pos0), k_new=_ptr(k_new), k_cache=_ptr(k_cache),
                        k_dtype=_kdtype(k_cache), k_scale=_ptr(k_scale), n_rows=len(rows), kbar=_ptr(kbar),
                        block_size=block_size if kbar is not None else 0,
                        n_blocks=kbar.shape[1] if kbar is not None else 0)
    for i, (rn, rc) in enumerate(rows):
        d.rows_new[i] = rn.data_ptr()
        d.rows_cache[i] = rc.data_ptr()
        d.row_elems[i] = rn[0, 0].numel()
        d.rows_stride_b[i] = rc.stride(0)
        d.rows_stride_n[i] = rc.stride(1)
    _check("lsa_cache_append", lib().lsa_cache_append(ctypes.byref(d), _stream(stream)))
