"""ctypes binding of libdblock (``include/dblock.h``), argument marshalling only.

Every step of the iteration runs in the library's HIP kernels; this module
checks tensor dtypes/shapes/devices, passes raw device pointers and sizes, and
raises ``DblockError`` on a non-zero status.  PyTorch provides the device
memory and the stream (the current torch stream unless one is given).

There is no fallback: if ``libdblock.so`` has not been built, loading fails
with an ImportError.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdblock.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADER = os.path.join(INCLUDE, "dblock.h")
PROBE_HEADER = os.path.join(INCLUDE, "dblock_probe.h")

DBLK_OK = 0
STATUS_NAMES = {0: "DBLK_OK", 1: "DBLK_ERR_NULL", 2: "DBLK_ERR_SHAPE", 3: "DBLK_ERR_ALIGN",
                4: "DBLK_ERR_WORKSPACE", 5: "DBLK_ERR_UNSUPPORTED", 6: "DBLK_ERR_LAUNCH"}

_c_void_p, _i32, _f32, _size = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t

class DecodeArgs(ctypes.Structure):
    """dblk_decode_args of include/dblock.h (same field order and C types)."""
    _fields_ = [(n, _c_void_p) for n in ("q", "k_prefix", "v_prefix", "k_block", "v_block",
                                          "k_suffix", "v_suffix", "prefix_len")] + \
               [(n, _i32) for n in ("B", "H", "L", "D", "P_cap", "S", "S_cap")] + \
               [("scale", _f32), ("attn_out", _c_void_p), ("h", _c_void_p), ("W", _c_void_p),
                ("d", _i32), ("V", _i32), ("conf", _c_void_p), ("argmax", _c_void_p),
                ("tokens", _c_void_p), ("mask", _c_void_p), ("threshold", _f32),
                ("eos_id", _i32), ("max_iters", _i32), ("commit_iter", _c_void_p),
                ("n_iters", _c_void_p), ("finished", _c_void_p)]


class KVSegment(ctypes.Structure):
    """dblk_kv_segment of include/dblock.h (same field order and C types)."""
    _fields_ = [("k", _c_void_p), ("v", _c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64), ("len", _i32),
                ("len_per_b", _c_void_p)]


class AttendArgs(ctypes.Structure):
    """dblk_attend_args of include/dblock.h (same field order and C types)."""
    _fields_ = [("B", _i32), ("H", _i32), ("L", _i32), ("D", _i32), ("q", _c_void_p),
                ("q_stride_b", ctypes.c_int64), ("q_stride_l", ctypes.c_int64),
                ("q_stride_h", ctypes.c_int64), ("prefix", KVSegment), ("block", KVSegment),
                ("suffix", KVSegment), ("scale", _f32), ("out", _c_void_p),
                ("o_stride_b", ctypes.c_int64), ("o_stride_l", ctypes.c_int64),
                ("o_stride_h", ctypes.c_int64)]


_SIGS = {
    "dblk_status_string": (ctypes.c_char_p, [_i32]),
    "dblk_abi_version": (_i32, []),
    "dblk_attend_workspace_size": (_size, [_i32] * 6),
    "dblk_attend": (_i32, [_c_void_p] * 7 + [_c_void_p] + [_i32] * 7 + [_f32, _c_void_p,
                                                                     _c_void_p, _size, _c_void_p]),
    "dblk_attend_segments_workspace_size": (_size, [ctypes.POINTER(AttendArgs)]),
    "dblk_attend_segments": (_i32, [ctypes.POINTER(AttendArgs), _c_void_p, _size, _c_void_p]),
    "dblk_lmhead_workspace_size": (_size, [_i32] * 3),
    "dblk_lmhead_confidence": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p,
                                      _c_void_p, _c_void_p, _size, _c_void_p]),
    "dblk_threshold_commit": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                     _f32, _c_void_p, _c_void_p]),
    "dblk_lmhead_confidence_commit": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p,
                                             _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _f32,
                                             _c_void_p, _c_void_p, _size, _c_void_p]),
    "dblk_lmhead_confidence_commit_noalloc": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p,
                                                     _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                                     _f32, _c_void_p, _c_void_p]),
    "dblk_threshold_commit_eos": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                         _f32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "dblk_decode_block_workspace_size": (_size, [ctypes.POINTER(DecodeArgs)]),
    "dblk_decode_block": (_i32, [ctypes.POINTER(DecodeArgs), _c_void_p, _size, _c_void_p]),
    "dblk_decode_block_run": (_i32, [ctypes.POINTER(DecodeArgs), _i32, _c_void_p, _c_void_p,
                                     _size, _c_void_p, ctypes.POINTER(_i32)]),
    "dblk_cache_append": (_i32, [_c_void_p] * 5 + [_i32] * 5 + [_c_void_p, _c_void_p]),
    "dblk_probe_read": (_i32, [_c_void_p, _size, _i32, _i32, _c_void_p, _c_void_p]),
}

_lib = None


class DblockError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


def header_symbols(path: Optional[str] = None):
    """Names of the functions declared in include/*.h (or in one header)."""
    paths = [path] if path else sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)
                                       if f.endswith(".h"))
    txt = "\n".join(open(p).read() for p in paths)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|int32_t)\s*(dblk_\w+)\s*\(",
                                 txt, re.M)))


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libdblock.so is not built ({p}); run "
                          "`python -m block_wise_decoding_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().dblk_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != DBLK_OK:
        raise DblockError(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ------------------------------------------------------------------ workspace

def attend_workspace_size(B, H, L, D, P_cap, S) -> int:
    return int(load_library().dblk_attend_workspace_size(B, H, L, D, P_cap, S))


def lmhead_workspace_size(M, d, V) -> int:
    return int(load_library().dblk_lmhead_workspace_size(M, d, V))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled device workspace (torch's allocator returns 512-byte aligned blocks)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def dblk_attend(q, k_prefix, v_prefix, k_block, v_block, k_suffix, v_suffix, prefix_len, out,
                workspace=None, scale: float = 0.0, stream=None, S: Optional[int] = None):
    """Non-causal attention of the block over the dual cache (include/dblock.h).

    q, out [B][L][H][D]; k/v_prefix [B][H][P_cap][D]; k/v_block [B][H][L][D];
    k/v_suffix [B][H][S_cap][D] (all bf16); prefix_len int32 [B] or None.
    S: suffix rows attended (default S_cap, the buffers' row count).
    """
    B, L, H, D = q.shape
    _need(q, "q", torch.bfloat16)
    P_cap = k_prefix.shape[2]
    S_cap = k_suffix.shape[2]
    S = S_cap if S is None else int(S)
    for n, t, s in (("k_prefix", k_prefix, (B, H, P_cap, D)), ("v_prefix", v_prefix, (B, H, P_cap, D)),
                    ("k_block", k_block, (B, H, L, D)), ("v_block", v_block, (B, H, L, D)),
                    ("k_suffix", k_suffix, (B, H, S_cap, D)), ("v_suffix", v_suffix, (B, H, S_cap, D)),
                    ("out", out, (B, L, H, D))):
        _need(t, n, torch.bfloat16, s)
    if prefix_len is not None:
        _need(prefix_len, "prefix_len", torch.int32, (B,))
    if workspace is None:
        workspace = alloc_workspace(attend_workspace_size(B, H, L, D, P_cap, S), q.device)
    st = load_library().dblk_attend(
        _ptr(q), _ptr(k_prefix), _ptr(v_prefix), _ptr(k_block), _ptr(v_block), _ptr(k_suffix),
        _ptr(v_suffix), _ptr(prefix_len), B, H, L, D, P_cap, S, S_cap, float(scale), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream, q.device))
    _check("dblk_attend", st)
    return out


def _view(t: torch.Tensor, name: str, ndim: int = 4):
    """Checks a bf16 device view whose last dimension is contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != ndim or (t.shape[-1] > 1 and t.stride(-1) != 1):
        raise ValueError(f"{name} must be a {ndim}-d view with a contiguous last dimension")


def kv_segment(k=None, v=None, len_per_b=None, rows: Optional[int] = None) -> KVSegment:
    """One cache segment: k, v bf16 views [B][H][T][D] with equal strides (any
    layout whose D is contiguous, e.g. a head-interleaved [B][T][H][D] cache
    permuted to [B][H][T][D]); len_per_b int32 [B] device tensor or None;
    rows: rows available per (b, h), default T.  None for k: an empty segment."""
    if k is None:
        return KVSegment(None, None, 0, 0, 0, 0, None)
    _view(k, "k"); _view(v, "v")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v of a segment must have the same shape and strides")
    if len_per_b is not None:
        _need(len_per_b, "len_per_b", torch.int32, (k.shape[0],))
    n = k.shape[2] if rows is None else int(rows)
    if n > k.shape[2]:
        raise ValueError("rows exceeds the segment's row count")
    seg = KVSegment(_ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2), n, _ptr(len_per_b))
    seg._keep = (k, v, len_per_b)          # the structure holds raw pointers into these
    return seg


def attend_args(q, prefix: KVSegment, block: KVSegment, suffix: KVSegment, out,
                scale: float = 0.0) -> AttendArgs:
    """dblk_attend_args for q and out bf16 views [B][L][H][D] (any strides, D contiguous).

    The returned structure references every tensor it points into, so a
    temporary passed here stays alive as long as the structure does."""
    _view(q, "q"); _view(out, "out")
    if tuple(q.shape) != tuple(out.shape):
        raise ValueError("q and out must have the same shape")
    B, L, H, D = q.shape
    a = AttendArgs(B, H, L, D, _ptr(q), q.stride(0), q.stride(1), q.stride(2), prefix, block,
                   suffix, float(scale), _ptr(out), out.stride(0), out.stride(1), out.stride(2))
    # the structure holds raw pointers: it keeps the tensors they point into
    # alive for as long as it exists (the segments are copied in by value)
    a._keep = (q, out) + tuple(getattr(sg, "_keep", ()) for sg in (prefix, block, suffix))
    return a


def attend_segments_workspace_size(args: AttendArgs) -> int:
    return int(load_library().dblk_attend_segments_workspace_size(ctypes.byref(args)))


def dblk_attend_segments(args: AttendArgs, workspace=None, stream=None, device=None):
    """Non-causal attention over strided cache segments (include/dblock.h).

    args from attend_args() (pointers into the tensors: keep them alive);
    workspace zero-filled uint8, sized by attend_segments_workspace_size(args)
    (allocated here if None)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    if workspace is None:
        workspace = alloc_workspace(attend_segments_workspace_size(args), device)
    st = load_library().dblk_attend_segments(ctypes.byref(args), _ptr(workspace),
                                             workspace.numel(), _stream(stream, device))
    _check("dblk_attend_segments", st)
    return workspace


def dblk_lmhead_confidence(h, W, conf, argmax, workspace=None, stream=None):
    """LM head + full-vocabulary confidence and argmax (include/dblock.h).

    h [M][d] bf16, W [V][d] bf16, conf [M] float32 (out), argmax [M] int32 (out).
    """
    M, d = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16)
    _need(W, "W", torch.bfloat16, (V, d))
    _need(conf, "conf", torch.float32, (M,))
    _need(argmax, "argmax", torch.int32, (M,))
    if workspace is None:
        workspace = alloc_workspace(lmhead_workspace_size(M, d, V), h.device)
    st = load_library().dblk_lmhead_confidence(
        _ptr(h), _ptr(W), M, d, V, _ptr(conf), _ptr(argmax), _ptr(workspace),
        workspace.numel(), _stream(stream, h.device))
    _check("dblk_lmhead_confidence", st)
    return conf, argmax


def dblk_threshold_commit(conf, argmax, tokens, mask, threshold: float, n_committed=None,
                          stream=None):
    """One threshold-parallel-decoder step, in place on tokens/mask (include/dblock.h).

    conf float32 [B][L], argmax int32 [B][L], tokens int32 [B][L], mask uint8
    [B][L] (nonzero = masked), n_committed int32 [B] or None.
    """
    B, L = conf.shape
    _need(conf, "conf", torch.float32)
    _need(argmax, "argmax", torch.int32, (B, L))
    _need(tokens, "tokens", torch.int32, (B, L))
    _need(mask, "mask", torch.uint8, (B, L))
    if n_committed is not None:
        _need(n_committed, "n_committed", torch.int32, (B,))
    st = load_library().dblk_threshold_commit(
        _ptr(conf), _ptr(argmax), _ptr(tokens), _ptr(mask), B, L, float(threshold),
        _ptr(n_committed), _stream(stream, conf.device))
    _check("dblk_threshold_commit", st)
    return tokens, mask


def dblk_lmhead_confidence_commit(h, W, conf, argmax, tokens, mask, threshold: float,
                                  n_committed=None, workspace=None, stream=None):
    """LM head + confidence + one decoder step, in place on tokens/mask (include/dblock.h).

    h [B*L][d] bf16, W [V][d] bf16, conf float32 [B][L] (out), argmax int32 [B][L]
    (out), tokens int32 [B][L], mask uint8 [B][L], n_committed int32 [B] or None.
    """
    B, L = tokens.shape
    M, d = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, (B * L, d))
    _need(W, "W", torch.bfloat16, (V, d))
    _need(conf, "conf", torch.float32, (B, L))
    _need(argmax, "argmax", torch.int32, (B, L))
    _need(tokens, "tokens", torch.int32, (B, L))
    _need(mask, "mask", torch.uint8, (B, L))
    if n_committed is not None:
        _need(n_committed, "n_committed", torch.int32, (B,))
    if workspace is None:
        workspace = alloc_workspace(lmhead_workspace_size(M, d, V), h.device)
    st = load_library().dblk_lmhead_confidence_commit(
        _ptr(h), _ptr(W), d, V, _ptr(conf), _ptr(argmax), _ptr(tokens), _ptr(mask), B, L,
        float(threshold), _ptr(n_committed), _ptr(workspace), workspace.numel(),
        _stream(stream, h.device))
    _check("dblk_lmhead_confidence_commit", st)
    return tokens, mask


NOALLOC_SCRATCH_BYTES = 16 << 20     # DBLK_NOALLOC_SCRATCH_BYTES of include/dblock.h


def dblk_lmhead_confidence_commit_noalloc(h, W, conf, argmax, tokens, mask, threshold: float,
                                          n_committed=None, stream=None):
    """dblk_lmhead_confidence_commit with the library's per-GPU scratch instead
    of a workspace: allocates nothing (include/dblock.h).  Calls that may
    overlap on one GPU race."""
    B, L = tokens.shape
    M, d = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, (B * L, d))
    _need(W, "W", torch.bfloat16, (V, d))
    _need(conf, "conf", torch.float32, (B, L))
    _need(argmax, "argmax", torch.int32, (B, L))
    _need(tokens, "tokens", torch.int32, (B, L))
    _need(mask, "mask", torch.uint8, (B, L))
    if n_committed is not None:
        _need(n_committed, "n_committed", torch.int32, (B,))
    st = load_library().dblk_lmhead_confidence_commit_noalloc(
        _ptr(h), _ptr(W), d, V, _ptr(conf), _ptr(argmax), _ptr(tokens), _ptr(mask), B, L,
        float(threshold), _ptr(n_committed), _stream(stream, h.device))
    _check("dblk_lmhead_confidence_commit_noalloc", st)
    return tokens, mask


def dblk_threshold_commit_eos(conf, argmax, tokens, mask, threshold: float, eos_id: int,
                              n_committed=None, finished=None, stream=None):
    """Decoder step with end-of-text handling, in place on tokens/mask (include/dblock.h).

    As dblk_threshold_commit; then still-masked positions after the row's first
    committed eos_id become eos_id.  finished uint8 [B] or None.
    """
    B, L = conf.shape
    _need(conf, "conf", torch.float32)
    _need(argmax, "argmax", torch.int32, (B, L))
    _need(tokens, "tokens", torch.int32, (B, L))
    _need(mask, "mask", torch.uint8, (B, L))
    if n_committed is not None:
        _need(n_committed, "n_committed", torch.int32, (B,))
    if finished is not None:
        _need(finished, "finished", torch.uint8, (B,))
    st = load_library().dblk_threshold_commit_eos(
        _ptr(conf), _ptr(argmax), _ptr(tokens), _ptr(mask), B, L, float(threshold), int(eos_id),
        _ptr(n_committed), _ptr(finished), _stream(stream, conf.device))
    _check("dblk_threshold_commit_eos", st)
    return tokens, mask


def decode_args(q, k_prefix, v_prefix, k_block, v_block, k_suffix, v_suffix, prefix_len,
                attn_out, h, W, conf, argmax, tokens, mask, threshold: float, *, eos_id: int = -1,
                max_iters: int = 0, commit_iter=None, n_iters=None, finished=None,
                scale: float = 0.0, S: Optional[int] = None) -> DecodeArgs:
    """Checks the tensors of a block decode and fills a DecodeArgs (pointers into them:
    keep the tensors alive while the structure is used)."""
    B, L, H, D = q.shape
    P_cap = k_prefix.shape[2]
    S_cap = k_suffix.shape[2]
    S = S_cap if S is None else int(S)
    M, d = h.shape
    V = W.shape[0]
    for n, t, sh in (("q", q, (B, L, H, D)), ("k_prefix", k_prefix, (B, H, P_cap, D)),
                     ("v_prefix", v_prefix, (B, H, P_cap, D)), ("k_block", k_block, (B, H, L, D)),
                     ("v_block", v_block, (B, H, L, D)), ("k_suffix", k_suffix, (B, H, S_cap, D)),
                     ("v_suffix", v_suffix, (B, H, S_cap, D)), ("attn_out", attn_out, (B, L, H, D)),
                     ("h", h, (B * L, d)), ("W", W, (V, d))):
        _need(t, n, torch.bfloat16, sh)
    if prefix_len is not None:
        _need(prefix_len, "prefix_len", torch.int32, (B,))
    _need(conf, "conf", torch.float32, (B, L))
    _need(argmax, "argmax", torch.int32, (B, L))
    _need(tokens, "tokens", torch.int32, (B, L))
    _need(mask, "mask", torch.uint8, (B, L))
    if commit_iter is not None:
        _need(commit_iter, "commit_iter", torch.int32, (B, L))
    if n_iters is not None:
        _need(n_iters, "n_iters", torch.int32, (B,))
    if finished is not None:
        _need(finished, "finished", torch.uint8, (B,))
    return DecodeArgs(_ptr(q), _ptr(k_prefix), _ptr(v_prefix), _ptr(k_block), _ptr(v_block),
                      _ptr(k_suffix), _ptr(v_suffix), _ptr(prefix_len), B, H, L, D, P_cap, S,
                      S_cap, float(scale), _ptr(attn_out), _ptr(h), _ptr(W), d, V, _ptr(conf),
                      _ptr(argmax), _ptr(tokens), _ptr(mask), float(threshold), int(eos_id),
                      int(max_iters), _ptr(commit_iter), _ptr(n_iters), _ptr(finished))


def decode_block_workspace_size(args: DecodeArgs) -> int:
    return int(load_library().dblk_decode_block_workspace_size(ctypes.byref(args)))


def dblk_decode_block(args: DecodeArgs, workspace=None, stream=None, device=None):
    """Enqueue the iterations of one block, no host synchronisation (include/dblock.h).

    args from decode_args(); workspace zero-filled uint8, sized by
    decode_block_workspace_size(args) (allocated here if None).
    """
    device = device or torch.device("cuda", torch.cuda.current_device())
    if workspace is None:
        workspace = alloc_workspace(decode_block_workspace_size(args), device)
    st = load_library().dblk_decode_block(ctypes.byref(args), _ptr(workspace), workspace.numel(),
                                          _stream(stream, device))
    _check("dblk_decode_block", st)
    return workspace


_HOST_ACTIVE = {}


def _host_active_buffer(device) -> torch.Tensor:
    """One pinned int32 [2] buffer per device, alive until the process ends.

    dblk_decode_block_run returns while the chunk queued behind the last one
    it checked may still be running, and that chunk's copy still writes into
    host_active; a buffer freed on return could by then belong to another
    tensor.  A module-level buffer outlives every such copy.  Calls on one
    device share it, so they must not overlap (they also share the stream's
    order, which keeps them apart when issued on one stream)."""
    key = torch.device(device).index if torch.device(device).index is not None else \
        torch.cuda.current_device()
    buf = _HOST_ACTIVE.get(key)
    if buf is None:
        buf = torch.zeros(2, dtype=torch.int32, pin_memory=True)
        _HOST_ACTIVE[key] = buf
    return buf


def dblk_decode_block_run(args: DecodeArgs, chunk: int, workspace=None, host_active=None,
                          stream=None, device=None) -> int:
    """Decode one block to completion, `chunk` iterations queued ahead of the
    host's completion check (include/dblock.h).  Waits for device progress;
    returns the number of iterations enqueued.  host_active: pinned int32 [2]
    host tensor that stays alive until the stream has finished this call's
    work (default: a per-device buffer kept by this module)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    if workspace is None:
        workspace = alloc_workspace(decode_block_workspace_size(args), device)
    if host_active is None:
        host_active = _host_active_buffer(device)
    if host_active.is_cuda or not host_active.is_pinned() or host_active.numel() < 2 \
            or host_active.dtype != torch.int32:
        raise ValueError("host_active must be a pinned host int32 tensor of >= 2 elements")
    n = _i32(0)
    st = load_library().dblk_decode_block_run(ctypes.byref(args), int(chunk),
                                              host_active.data_ptr(), _ptr(workspace),
                                              workspace.numel(), _stream(stream, device),
                                              ctypes.byref(n))
    _check("dblk_decode_block_run", st)
    return int(n.value)


def dblk_cache_append(k_prefix, v_prefix, k_block, v_block, prefix_len, appended=None,
                      stream=None):
    """Append the block's K/V after each sequence's prefix, advance prefix_len (include/dblock.h).

    k/v_prefix [B][H][P_cap][D] (in/out), k/v_block [B][H][L][D] bf16;
    prefix_len int32 [B] (in/out); appended int32 [B] or None.
    """
    B, H, P_cap, D = k_prefix.shape
    L = k_block.shape[2]
    for n, t, sh in (("k_prefix", k_prefix, (B, H, P_cap, D)), ("v_prefix", v_prefix, (B, H, P_cap, D)),
                     ("k_block", k_block, (B, H, L, D)), ("v_block", v_block, (B, H, L, D))):
        _need(t, n, torch.bfloat16, sh)
    _need(prefix_len, "prefix_len", torch.int32, (B,))
    if appended is not None:
        _need(appended, "appended", torch.int32, (B,))
    st = load_library().dblk_cache_append(
        _ptr(k_prefix), _ptr(v_prefix), _ptr(k_block), _ptr(v_block), _ptr(prefix_len), B, H, L,
        D, P_cap, _ptr(appended), _stream(stream, k_prefix.device))
    _check("dblk_cache_append", st)
    return prefix_len


def dblk_probe_read(buf: torch.Tensor, nontemporal: bool, grid: int, sink: torch.Tensor,
                    stream=None):
    """HBM read-ceiling probe (include/dblock_probe.h): stream ``buf`` once.

    buf: contiguous device tensor of a multiple of 32768 bytes; sink: int32
    device tensor of at least grid*256 elements (written, value meaningless).
    """
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _need(sink, "sink", torch.int32)
    if sink.numel() < grid * 256:
        raise ValueError("sink must hold grid*256 elements")
    st = load_library().dblk_probe_read(_ptr(buf), buf.numel() * buf.element_size(),
                                        int(bool(nontemporal)), int(grid), _ptr(sink),
                                        _stream(stream, buf.device))
    _check("dblk_probe_read", st)
