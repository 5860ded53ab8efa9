"""Thin Python binding of libkvss (include/kvss.h), same names as the C ABI.

Argument marshalling only: tensors are checked for device, dtype and contiguity, their device
pointers and torch's current HIP stream are handed to the library, and missing outputs or
workspaces are allocated with torch. Every step of the computation runs in the library's HIP
kernels; there is no fallback. Loading fails loudly if libkvss.so has not been built.
"""

import ctypes
import functools
import inspect
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvss.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "kvss.h")

KVSS_OK, KVSS_EINVAL, KVSS_EUNSUPPORTED, KVSS_EWORKSPACE, KVSS_EHIP = 0, -1, -2, -3, -4
KVSS_F32, KVSS_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: KVSS_F32, torch.bfloat16: KVSS_BF16}


class KvssError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"kvss error {code}: {message}")
        self.code = code


class kvss_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_U64 = ctypes.c_uint64
_KV = ctypes.POINTER(kvss_kv)

_SIGNATURES = {
    "kvss_last_error": (ctypes.c_char_p, []),
    "kvss_version": (_I, []),
    "kvss_verify_workspace_bytes": (_Z, [_KV, _I, _I]),
    "verify_attn_full": (_I, [_KV, _P, _I, _I, _F, _P, _P, _P, _Z, _P]),
    "verify_attn_full_noalloc": (_I, [_KV, _P, _I, _I, _F, _P, _P, _P]),
    "kvss_draft_workspace_bytes": (_Z, [_KV, _I, _I, _I]),
    "draft_attn_sparse": (_I, [_KV, _P, _I, _P, _P, _I, _P, _I, _F, _P, _P, _P, _Z, _P]),
    "kvss_streaming_set": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "kvss_snapkv_workspace_bytes": (_Z, [_KV, _I, _I, _I]),
    "snapkv_select": (_I, [_KV, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _Z, _P]),
    "kvss_accept_workspace_bytes": (_Z, [_I, _I, _I]),
    "spec_accept": (_I, [_P, _P, _P, _I, _I, _I, _F, _U64, _U64, _P, _P, _P, _P, _Z, _P]),
    "kvss_stream_read": (_I, [_P, _Z, _P, _P]),
    "kvss_kv_append": (_I, [_KV, _P, _P, _I, _P, _P]),
    "kvss_topk_workspace_bytes": (_Z, [_KV, _I, _I]),
    "kvss_sample_workspace_bytes": (_Z, [_I, _I]),
    "draft_sample": (_I, [_P, _I, _I, _F, _U64, _U64, _I, _P, _P, _P, _Z, _P]),
    "draft_attn_topk": (_I, [_KV, _P, _I, _I, _F, _P, _P, _P, _P, _P, _Z, _P]),
    "kvss_draft_cache_build": (_I, [_KV, _P, _P, _I, _P, _I, _KV, _P, _P]),
    "kvss_philox4x32_10": (_I, [_P, ctypes.c_int64, _U64, _P, _P]),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with kv_sparse_speculative_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def declared_functions():
    """Function names declared with KVSS_API in include/kvss.h."""
    text = open(HEADER).read()
    return re.findall(r"KVSS_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def _check(rc):
    if rc != KVSS_OK:
        raise KvssError(rc, lib().kvss_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on_call_stream(fn):
    """Run a wrapper with its `stream` argument (when given) as torch's current stream, so that
    the outputs and the workspace the wrapper allocates, and the fills of those it zeroes, are
    ordered on the stream the library's kernels run on; memory the wrapper drops on return
    then goes back to that stream's pool, which the allocator hands out only to later work on
    the same stream."""
    idx = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def call(*args, **kwargs):
        stream = kwargs.get("stream", args[idx] if len(args) > idx else None)
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return call


def _need(t, name, dtype=None, device=True, shape=None):
    """Check a tensor the library reads or writes through a raw pointer: contiguous, of the
    given dtype, on the device and, when `shape` is given, of exactly that shape (the kernels
    index it by the call's sizes, so a smaller buffer would be read or written out of bounds)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class PagedKV:
    """A paged per-layer KV cache: k, v [num_blocks, Hkv, block_size, D] (bf16 or f32),
    block_table int32 [B, max_blocks], kv_lens int32 [B] and a host bound max_kv_len."""

    def __init__(self, k, v, block_table, kv_lens, max_kv_len):
        for t, n in ((k, "k"), (v, "v")):
            _need(t, n)
        _need(block_table, "block_table", torch.int32)
        if k.dim() != 4 or block_table.dim() != 2:
            raise ValueError("k, v must be [num_blocks, Hkv, block_size, D]; block_table [B, max_blocks]")
        _need(kv_lens, "kv_lens", torch.int32, shape=(block_table.shape[0],))
        if k.dtype not in _DTYPE_CODE or v.dtype != k.dtype or v.shape != k.shape:
            raise ValueError("k and v must share shape and a bf16 / f32 dtype")
        self.k, self.v, self.block_table, self.kv_lens = k, v, block_table, kv_lens
        self.max_kv_len = int(max_kv_len)
        self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim = k.shape
        self.batch, self.max_blocks = block_table.shape
        self.dtype = k.dtype
        self._desc = kvss_kv(k.data_ptr(), v.data_ptr(), block_table.data_ptr(),
                             kv_lens.data_ptr(), self.batch, self.num_kv_heads, self.head_dim,
                             self.block_size, self.max_blocks, self.num_blocks, self.max_kv_len,
                             _DTYPE_CODE[self.dtype])

    def with_lens(self, kv_lens, max_kv_len):
        return PagedKV(self.k, self.v, self.block_table, kv_lens, max_kv_len)

    def desc(self):
        return self._desc


def _workspace(nbytes, workspace, device):
    """The caller's workspace (size checked by the library) or a new one of nbytes, allocated
    on the stream the call runs on (see `_on_call_stream`)."""
    if workspace is None:
        if nbytes == 0:
            return None, 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _need(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


@_on_call_stream
def verify_attn_full(kv, q, scale=None, out=None, lse=None, want_lse=True, workspace=None,
                     stream=None):
    """q [B, Hq, T, D] -> (out [B, Hq, T, D] f32, lse [B, Hq, T] f32 or None)."""
    _need(q, "q", kv.dtype)
    if q.dim() != 4 or q.shape[0] != kv.batch or q.shape[3] != kv.head_dim:
        raise ValueError("q must be [batch, num_q_heads, T, head_dim] of the cache")
    B, Hq, T, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, Hq, T, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, shape=(B, Hq, T, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq, T))
    d = kv.desc()
    nbytes = lib().kvss_verify_workspace_bytes(ctypes.byref(d), Hq, T)
    workspace, wsb = _workspace(nbytes, workspace, q.device)
    _check(lib().verify_attn_full(ctypes.byref(d), q.data_ptr(), Hq, T, scale, out.data_ptr(),
                                  _ptr(lse), _ptr(workspace), wsb, _stream(stream)))
    return out, lse


@_on_call_stream
def verify_attn_full_noalloc(kv, q, scale=None, out=None, lse=None, want_lse=True, stream=None):
    """verify_attn_full with the split partials in the library's own device scratch (no
    workspace). q [B, Hq, T, D] -> (out, lse or None); out / lse are allocated here only when
    not given, so a caller that passes both allocates nothing."""
    _need(q, "q", kv.dtype)
    if q.dim() != 4 or q.shape[0] != kv.batch or q.shape[3] != kv.head_dim:
        raise ValueError("q must be [batch, num_q_heads, T, head_dim] of the cache")
    B, Hq, T, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, Hq, T, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, shape=(B, Hq, T, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq, T))
    _check(lib().verify_attn_full_noalloc(ctypes.byref(kv.desc()), q.data_ptr(), Hq, T, scale,
                                          out.data_ptr(), _ptr(lse), _stream(stream)))
    return out, lse


@_on_call_stream
def draft_attn_sparse(kv, q, sel_idx, sel_count, tail_lo, max_tail, scale=None, out=None,
                      lse=None, want_lse=True, workspace=None, stream=None):
    """q [B, Hq, D]; sel_idx int32 [B, Hkv, k_max]; sel_count, tail_lo int32 [B]."""
    _need(q, "q", kv.dtype)
    if q.dim() != 3 or q.shape[0] != kv.batch or q.shape[2] != kv.head_dim:
        raise ValueError("q must be [batch, num_q_heads, head_dim] of the cache")
    B, Hq, D = q.shape
    k_max = 0 if sel_idx is None else sel_idx.shape[-1]
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", torch.int32, shape=(B, kv.num_kv_heads, k_max))
        _need(sel_count, "sel_count", torch.int32, shape=(B,))
    _need(tail_lo, "tail_lo", torch.int32, shape=(B,))
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, shape=(B, Hq, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq))
    d = kv.desc()
    nbytes = lib().kvss_draft_workspace_bytes(ctypes.byref(d), Hq, k_max, int(max_tail))
    workspace, wsb = _workspace(nbytes, workspace, q.device)
    _check(lib().draft_attn_sparse(ctypes.byref(d), q.data_ptr(), Hq, _ptr(sel_idx),
                                   _ptr(sel_count), k_max, tail_lo.data_ptr(), int(max_tail),
                                   scale, out.data_ptr(), _ptr(lse), _ptr(workspace), wsb,
                                   _stream(stream)))
    return out, lse


@_on_call_stream
def kvss_streaming_set(kv_lens, num_kv_heads, sink, window, sel_idx=None, sel_count=None,
                       tail_lo=None, stream=None):
    """StreamingLLM set -> (sel_idx [B, Hkv, sink], sel_count [B], tail_lo [B]) int32."""
    _need(kv_lens, "kv_lens", torch.int32)
    B = kv_lens.shape[0]
    dev = kv_lens.device
    if sel_idx is None:
        sel_idx = torch.empty((B, num_kv_heads, sink), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty(B, dtype=torch.int32, device=dev)
    if tail_lo is None:
        tail_lo = torch.empty(B, dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, shape=(B, num_kv_heads, sink))
    _need(sel_count, "sel_count", torch.int32, shape=(B,))
    _need(tail_lo, "tail_lo", torch.int32, shape=(B,))
    _check(lib().kvss_streaming_set(kv_lens.data_ptr(), B, num_kv_heads, sink, window,
                                    sel_idx.data_ptr(), sel_count.data_ptr(), tail_lo.data_ptr(),
                                    _stream(stream)))
    return sel_idx, sel_count, tail_lo


@_on_call_stream
def snapkv_select(kv, q_obs, w, pool_kernel, budget, scale=None, scores_out=None,
                  want_scores=False, sel_idx=None, sel_count=None, workspace=None, stream=None):
    """kv.kv_lens = prompt lengths; q_obs [B, Hq, w, D] -> (sel_idx, sel_count, scores|None)."""
    _need(q_obs, "q_obs", kv.dtype)
    if q_obs.dim() != 4 or q_obs.shape[0] != kv.batch or q_obs.shape[3] != kv.head_dim:
        raise ValueError("q_obs must be [batch, num_q_heads, w, head_dim] of the cache")
    B, Hq, w_, D = q_obs.shape
    if w_ != w:
        raise ValueError("q_obs window does not match w")
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dev = q_obs.device
    if sel_idx is None:
        sel_idx = torch.empty((B, kv.num_kv_heads, budget - w), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty(B, dtype=torch.int32, device=dev)
    if scores_out is None and want_scores:
        scores_out = torch.zeros((B, kv.num_kv_heads, max(kv.max_kv_len - w, 0)),
                                 dtype=torch.float32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, shape=(B, kv.num_kv_heads, budget - w))
    _need(sel_count, "sel_count", torch.int32, shape=(B,))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32,
              shape=(B, kv.num_kv_heads, max(kv.max_kv_len - w, 0)))
    d = kv.desc()
    nbytes = lib().kvss_snapkv_workspace_bytes(ctypes.byref(d), Hq, w, budget)
    workspace, wsb = _workspace(nbytes, workspace, dev)
    _check(lib().snapkv_select(ctypes.byref(d), q_obs.data_ptr(), Hq, w, pool_kernel, budget,
                               scale, sel_idx.data_ptr(), sel_count.data_ptr(), _ptr(scores_out),
                               _ptr(workspace), wsb, _stream(stream)))
    return sel_idx, sel_count, scores_out


@_on_call_stream
def spec_accept(target_logits, draft_logits, draft_tokens, temperature, seed=0, offset=0,
                row_stats=None, want_stats=False, out_tokens=None, num_accepted=None,
                workspace=None, stream=None):
    """target [B, gamma+1, V], draft [B, gamma, V] f32; tokens int32 [B, gamma]
    -> (out_tokens [B, gamma+1], num_accepted [B], row_stats [B, 2gamma+1, 4] or None)."""
    _need(target_logits, "target_logits", torch.float32)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [batch, gamma + 1, vocab]")
    B, T, V = target_logits.shape
    gamma = T - 1
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, shape=(B, gamma, V))
    elif float(temperature) != 0.0 and gamma > 0:
        raise ValueError("draft_logits are required when temperature > 0 and gamma > 0")
    _need(draft_tokens, "draft_tokens", torch.int32, shape=(B, gamma))
    dev = target_logits.device
    if out_tokens is None:
        out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev)
    n_acc = num_accepted
    if n_acc is None:
        n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    if row_stats is None and want_stats:
        row_stats = torch.zeros((B, 2 * gamma + 1, 4), dtype=torch.float32, device=dev)
    _need(out_tokens, "out_tokens", torch.int32, shape=(B, T))
    _need(n_acc, "num_accepted", torch.int32, shape=(B,))
    if row_stats is not None:
        _need(row_stats, "row_stats", torch.float32, shape=(B, 2 * gamma + 1, 4))
    nbytes = lib().kvss_accept_workspace_bytes(B, gamma, V)
    workspace, wsb = _workspace(nbytes, workspace, dev)
    _check(lib().spec_accept(target_logits.data_ptr(), _ptr(draft_logits), draft_tokens.data_ptr(),
                             B, gamma, V, float(temperature), int(seed) & (2**64 - 1),
                             int(offset) & (2**64 - 1), out_tokens.data_ptr(), n_acc.data_ptr(),
                             _ptr(row_stats), _ptr(workspace), wsb, _stream(stream)))
    return out_tokens, n_acc, row_stats


@_on_call_stream
def kvss_stream_read(buf, sink, stream=None):
    """Measurement reference: stream-read every byte of the device tensor `buf`."""
    _need(buf, "buf")
    _need(sink, "sink")
    _check(lib().kvss_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                  _stream(stream)))


@_on_call_stream
def kvss_philox4x32_10(counters, seed, out=None, stream=None):
    """The library's Philox4x32-10 on counters int32/uint32-bit words [n, 4] (device, stored as
    torch.int32); returns the output words [n, 4] as torch.int32 bit patterns."""
    _need(counters, "counters", torch.int32)
    if counters.dim() != 2 or counters.shape[1] != 4:
        raise ValueError("counters must be [n, 4]")
    if out is None:
        out = torch.empty_like(counters)
    _need(out, "out", torch.int32, shape=tuple(counters.shape))
    _check(lib().kvss_philox4x32_10(counters.data_ptr(), counters.shape[0], int(seed) & (2**64 - 1),
                                    out.data_ptr(), _stream(stream)))
    return out


@_on_call_stream
def kvss_kv_append(kv, k_new, v_new, start, stream=None):
    """Write k_new / v_new [B, Hkv, T, D] at logical positions start[b] + t of the paged cache."""
    _need(k_new, "k_new", kv.dtype)
    _need(v_new, "v_new", kv.dtype)
    _need(start, "start", torch.int32, shape=(kv.batch,))
    B, H, T, D = k_new.shape
    if v_new.shape != k_new.shape or B != kv.batch or H != kv.num_kv_heads or D != kv.head_dim:
        raise ValueError("k_new / v_new must be [batch, num_kv_heads, T, head_dim] of the cache")
    _check(lib().kvss_kv_append(ctypes.byref(kv.desc()), k_new.data_ptr(), v_new.data_ptr(), T,
                                start.data_ptr(), _stream(stream)))


@_on_call_stream
def kvss_draft_cache_build(src, sel_idx, sel_count, tail_lo, max_tail, dst, dst_lens=None,
                           stream=None):
    """Compact draft cache: dst receives each (b, g)'s listed rows then the tail of src;
    returns dst_lens int32 [B]."""
    k_max = 0 if sel_idx is None else sel_idx.shape[-1]
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", torch.int32, shape=(src.batch, src.num_kv_heads, k_max))
        _need(sel_count, "sel_count", torch.int32, shape=(src.batch,))
    _need(tail_lo, "tail_lo", torch.int32, shape=(src.batch,))
    if dst_lens is None:
        dst_lens = torch.empty(src.batch, dtype=torch.int32, device=tail_lo.device)
    _need(dst_lens, "dst_lens", torch.int32, shape=(src.batch,))
    _check(lib().kvss_draft_cache_build(ctypes.byref(src.desc()), _ptr(sel_idx), _ptr(sel_count),
                                        k_max, tail_lo.data_ptr(), int(max_tail),
                                        ctypes.byref(dst.desc()), dst_lens.data_ptr(),
                                        _stream(stream)))
    return dst_lens


@_on_call_stream
def draft_attn_topk(kv, q, k, scale=None, out=None, lse=None, want_lse=True, sel_idx=None,
                    sel_count=None, workspace=None, stream=None):
    """Dynamic Top-K draft: q [B, Hq, D] -> (out [B, Hq, D], lse [B, Hq] or None); the kept
    positions go to sel_idx [B, Hkv, k] / sel_count [B] when given."""
    _need(q, "q", kv.dtype)
    if q.dim() != 3 or q.shape[0] != kv.batch or q.shape[2] != kv.head_dim:
        raise ValueError("q must be [batch, num_q_heads, head_dim] of the cache")
    B, Hq, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, shape=(B, Hq, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq))
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", torch.int32, shape=(B, kv.num_kv_heads, int(k)))
    if sel_count is not None:
        _need(sel_count, "sel_count", torch.int32, shape=(B,))
    d = kv.desc()
    nbytes = lib().kvss_topk_workspace_bytes(ctypes.byref(d), Hq, int(k))
    workspace, wsb = _workspace(nbytes, workspace, q.device)
    _check(lib().draft_attn_topk(ctypes.byref(d), q.data_ptr(), Hq, int(k), scale, out.data_ptr(),
                                 _ptr(lse), _ptr(sel_idx), _ptr(sel_count), _ptr(workspace), wsb,
                                 _stream(stream)))
    return out, lse


@_on_call_stream
def draft_sample(logits, temperature, seed=0, offset=0, step=0, tokens=None, row_stats=None,
                 want_stats=False, workspace=None, stream=None):
    """Draft token per sequence from logits [B, V] f32 -> (tokens int32 [B], row_stats or None)."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [batch, vocab]")
    B, V = logits.shape
    dev = logits.device
    if tokens is None:
        tokens = torch.empty(B, dtype=torch.int32, device=dev)
    if row_stats is None and want_stats:
        row_stats = torch.zeros((B, 4), dtype=torch.float32, device=dev)
    _need(tokens, "tokens", torch.int32, shape=(B,))
    if row_stats is not None:
        _need(row_stats, "row_stats", torch.float32, shape=(B, 4))
    nbytes = lib().kvss_sample_workspace_bytes(B, V)
    workspace, wsb = _workspace(nbytes, workspace, dev)
    _check(lib().draft_sample(logits.data_ptr(), B, V, float(temperature), int(seed) & (2**64 - 1),
                              int(offset) & (2**64 - 1), int(step), tokens.data_ptr(),
                              _ptr(row_stats), _ptr(workspace), wsb, _stream(stream)))
    return tokens, row_stats

