"""ctypes binding of libattn (include/attn.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of ``libattn.so``;
this module checks tensor metadata, allocates outputs with torch on the
tensors' device, passes raw device pointers and torch's current HIP stream,
and turns a non-zero status into an exception. There is no fallback: if the
library is missing or the tensors are not on a GPU, calls raise.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

F32, F16, BF16 = 0, 1, 2
_DTYPE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_MISALIGNED = -3
ERR_LAUNCH = -4
ERR_WORKSPACE = -5

_lib = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "attn_abi_version": (_i, []),
    "attn_status_string": (ctypes.c_char_p, [_i]),
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_fwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "attn_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_fwd_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "attn_fwd_num_splits": (_i, [_i, _i, _i, _i, _i, _i, _i]),
    "attn_check_args": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i]),
    "hadamard_quant": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "quant_per_tensor": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "attn_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "attn_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_fwd_persistent": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "rope_hadamard_quant": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_mfma_stream": (_i, [_i, _i, _vp, _sz, ctypes.POINTER(ctypes.c_double), _vp]),
}


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = load().attn_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")


def load():
    """Load libattn.so once and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m exact_attention_47_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, status):
    if status != OK:
        raise AttnError(fn, status)


def _need_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def abi_version() -> int:
    return load().attn_abi_version()


def mfma_stream(kind: int, iters: int, sink=None, device=None) -> float:
    """Enqueue ``attn_mfma_stream`` on the current stream; returns the launch's floating-point operations.

    ``kind`` 0 is the bf16 32x32x16 instruction, 1 the fp8 32x32x64 one, 2 the bf16 16x16x32 one. ``sink``
    (float32, one value per thread: 2 * CUs * 256) is allocated when not given; time the call with events on
    the current stream.
    """
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if sink is None:
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.empty(2 * n_cu * 256, dtype=torch.float32, device=dev)
    _need_gpu(sink)
    flop = ctypes.c_double(0.0)
    _check("attn_mfma_stream", load().attn_mfma_stream(int(kind), int(iters), _ptr(sink),
                                                       sink.numel() * sink.element_size(), ctypes.byref(flop),
                                                       _stream(sink.device)))
    return float(flop.value)


def workspace_size(B, H, S_q, S_k, D, num_splits=0) -> int:
    return int(load().attn_fwd_workspace_size(B, H, S_q, S_k, D, num_splits))


def num_splits(B, H, S_q, S_k, D, num_splits=0, dtype=BF16) -> int:
    """The split count attn_fwd (or attn_fwd_ex with num_splits) uses for these sizes and element type."""
    return int(load().attn_fwd_num_splits(B, H, S_q, S_k, D, int(dtype), num_splits))


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, num_splits=None, workspace=None):
    """O, LSE = attention(q, k, v) for [B, H, S, D] tensors on the GPU.

    ``num_splits=None`` calls ``attn_fwd`` (automatic split); an integer calls
    ``attn_fwd_ex`` with that request and the given (or a freshly allocated)
    workspace.
    """
    _need_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v must share one of float32/float16/bfloat16")
    B, H, S_q, D = q.shape
    S_k = k.shape[2]
    if tuple(k.shape) != (B, H, S_k, D) or tuple(v.shape) != (B, H, S_k, D):
        raise ValueError("k and v must be [B, H, S_k, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    _need_gpu(out, lse)
    lib = load()
    st = _stream(q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, S_q, S_k, D, int(causal),
            float(scale), _DTYPE[q.dtype])
    if num_splits is None:
        _check("attn_fwd", lib.attn_fwd(*args, st))
    else:
        need = lib.attn_fwd_workspace_size(B, H, S_q, S_k, D, int(num_splits))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check("attn_fwd_ex", lib.attn_fwd_ex(*args, int(num_splits), _ptr(workspace), wsz, st))
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20   # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h


def fwd_noalloc(q, k, v, causal=False, scale=None, out=None, lse=None):
    """``fwd`` through ``attn_fwd_noalloc``: the library allocates nothing during the call.

    A key-range split stages its partial results in the library's fixed device scratch array
    (NOALLOC_SCRATCH_BYTES per GPU) instead of a fresh allocation; shapes whose split needs more
    raise AttnError (ATTN_ERR_WORKSPACE). ``out`` and ``lse`` given by the caller keep this call
    free of allocations on the Python side as well.
    """
    _need_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v must share one of float32/float16/bfloat16")
    B, H, S_q, D = q.shape
    S_k = k.shape[2]
    if tuple(k.shape) != (B, H, S_k, D) or tuple(v.shape) != (B, H, S_k, D):
        raise ValueError("k and v must be [B, H, S_k, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    _need_gpu(out, lse)
    _check("attn_fwd_noalloc", load().attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, S_q, S_k, D, int(causal), float(scale),
        _DTYPE[q.dtype], _stream(q.device)))
    return out, lse


def fwd_persistent(q, k, v, causal=False, scale=None, out=None, lse=None, num_workgroups=0):
    """``fwd`` on a persistent grid of ``num_workgroups`` workgroups (0 = one per CU).

    bf16 / fp16, D 64 or 128, no key-range split; same outputs as ``fwd``.
    """
    _need_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise ValueError("q, k, v must share one of float32/float16/bfloat16")
    B, H, S_q, D = q.shape
    S_k = k.shape[2]
    if tuple(k.shape) != (B, H, S_k, D) or tuple(v.shape) != (B, H, S_k, D):
        raise ValueError("k and v must be [B, H, S_k, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    _need_gpu(out, lse)
    _check("attn_fwd_persistent", load().attn_fwd_persistent(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, S_q, S_k, D, int(causal), float(scale),
        _DTYPE[q.dtype], int(num_workgroups), _stream(q.device)))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, max_seqlen_k=None, causal=False,
               scale=None, out=None, lse=None, validate=True):
    """O [total_q, H, D], LSE [H, total_q] for a packed batch of sequences.

    ``q`` is [total_q, H, D], ``k``/``v`` are [total_k, H, D]; sequence b owns
    rows ``cu_seqlens_q[b]:cu_seqlens_q[b+1]`` (int32 GPU tensors of B+1
    entries). The kernel reads the offsets on the device and trusts them, so
    with ``validate`` (the default) they are copied to the host once and
    checked here; the maxima are taken from them when not given.
    """
    _need_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [total, H, D]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must share float16 or bfloat16")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if tuple(k.shape) != (total_k, H, D) or tuple(v.shape) != (total_k, H, D):
        raise ValueError("k and v must be [total_k, H, D] matching q")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D with the same B+1 >= 2 entries")
    B = cu_seqlens_q.numel() - 1
    if validate or max_seqlen_q is None or max_seqlen_k is None:
        cq, ck = cu_seqlens_q.cpu(), cu_seqlens_k.cpu()
        for cu, total, name in ((cq, total_q, "q"), (ck, total_k, "k")):
            if int(cu[0]) != 0 or int(cu[-1]) != total or bool((cu[1:] < cu[:-1]).any()):
                raise ValueError(f"cu_seqlens_{name} must start at 0, not decrease and end at {total}")
        lq, lk = int((cq[1:] - cq[:-1]).max()), int((ck[1:] - ck[:-1]).max())
        if max_seqlen_q is None:
            max_seqlen_q = lq
        if max_seqlen_k is None:
            max_seqlen_k = lk
        if lq > max_seqlen_q or lk > max_seqlen_k:
            raise ValueError("a sequence is longer than max_seqlen")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    _need_gpu(out, lse)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or tuple(lse.shape) != (H, total_q) \
            or lse.dtype != torch.float32:
        raise ValueError("out must be like q and lse float32 [H, total_q]")
    if total_q == 0:
        return out, lse
    st = _stream(q.device)
    _check("attn_fwd_varlen", load().attn_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, H,
        total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D, int(causal), float(scale), _DTYPE[q.dtype],
        st))
    return out, lse


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None):
    """(dQ, dK, dV) of attention for [B, H, S, D] tensors, given the forward output O and its LSE."""
    _need_gpu(q, k, v, o, lse, dout)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype) or q.dtype not in (torch.float16,
                                                                                         torch.bfloat16):
        raise ValueError("q, k, v, o, dout must share float16 or bfloat16")
    B, H, S_q, D = q.shape
    S_k = k.shape[2]
    if tuple(k.shape) != (B, H, S_k, D) or tuple(v.shape) != (B, H, S_k, D):
        raise ValueError("k and v must be [B, H, S_k, D] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must be like q")
    if tuple(lse.shape) != (B, H, S_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, S_q]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need_gpu(dq, dk, dv)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or not (
            dq.dtype == dk.dtype == dv.dtype == q.dtype):
        raise ValueError("dq, dk, dv must be like q, k, v")
    _check("attn_bwd", load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, S_q, S_k, D, int(causal), float(scale),
                                       _DTYPE[q.dtype], _stream(q.device)))
    return dq, dk, dv


def check_args(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S_q, S_k, D, causal, scale, dtype) -> int:
    """Host-only validation (no launch): the status attn_fwd would return."""
    return load().attn_check_args(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S_q, S_k, D, causal,
                                  ctypes.c_float(scale), dtype)


def hadamard_quant(x, signs, block_rows=64, apply_hadamard=True, out=None):
    """(codes uint8 [B,H,S,D], scales float32 [B,H,ceil(S/block_rows)]); out=(codes, scales) reuses buffers."""
    _need_gpu(x, signs)
    if x.dim() != 4 or x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("x must be a [B, H, S, D] bfloat16/float16 tensor")
    if signs.dtype != torch.int8 or signs.shape != (x.shape[3],):
        raise ValueError("signs must be int8 [D]")
    B, H, S, D = x.shape
    nb = -(-S // block_rows)
    if out is None:
        x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    else:
        x8, scales = out
        if (x8.shape != x.shape or x8.dtype != torch.uint8 or scales.shape != (B, H, nb)
                or scales.dtype != torch.float32 or not (x8.is_contiguous() and scales.is_contiguous())):
            raise ValueError("out must be contiguous (uint8 [B,H,S,D], float32 [B,H,ceil(S/block_rows)])")
        _need_gpu(x8, scales)
    st = _stream(x.device)
    _check("hadamard_quant", load().hadamard_quant(_ptr(x), _ptr(x8), _ptr(scales), _ptr(signs), B, H, S,
                                                   D, block_rows, int(bool(apply_hadamard)),
                                                   _DTYPE[x.dtype], st))
    return x8, scales


def rope_hadamard_quant(x, signs, cos, sin, mode=0, block_rows=64, out=None):
    """Rotary embedding (tables cos/sin float32 [S, D/2] on the GPU; mode 0 interleaved pairs,
    1 half pairs) followed by hadamard_quant, in one pass: (codes uint8 [B,H,S,D], scales)."""
    _need_gpu(x, signs, cos, sin)
    if x.dim() != 4 or x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be a float16/bfloat16 [B, H, S, D] tensor")
    B, H, S, D = x.shape
    if signs.dtype != torch.int8 or signs.shape != (D,):
        raise ValueError("signs must be int8 [D]")
    if cos.dtype != torch.float32 or sin.dtype != torch.float32 or tuple(cos.shape) != (S, D // 2) \
            or tuple(sin.shape) != (S, D // 2):
        raise ValueError("cos and sin must be float32 [S, D/2]")
    nb = (S + block_rows - 1) // block_rows
    if out is None:
        x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    else:
        x8, scales = out
        if (x8.shape != x.shape or x8.dtype != torch.uint8 or scales.shape != (B, H, nb)
                or scales.dtype != torch.float32):
            raise ValueError("out must be (uint8 like x, float32 [B, H, nblk])")
        _need_gpu(x8, scales)
    _check("rope_hadamard_quant", load().rope_hadamard_quant(
        _ptr(x), _ptr(x8), _ptr(scales), _ptr(signs), _ptr(cos), _ptr(sin), B, H, S, D, block_rows, int(mode),
        _DTYPE[x.dtype], _stream(x.device)))
    return x8, scales


def quant_per_tensor(x, transposed=False, out=None):
    """(codes uint8 [B,H,S,D] or [B,H,D,S], scale float32 [1]); out=(codes, scale) reuses buffers."""
    _need_gpu(x)
    if x.dim() != 4 or x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("x must be a [B, H, S, D] bfloat16/float16 tensor")
    B, H, S, D = x.shape
    shape = (B, H, D, S) if transposed else (B, H, S, D)
    if out is None:
        x8 = torch.empty(shape, dtype=torch.uint8, device=x.device)
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        x8, scale = out
        if (x8.shape != shape or x8.dtype != torch.uint8 or scale.numel() != 1
                or scale.dtype != torch.float32 or not x8.is_contiguous()):
            raise ValueError("out must be (contiguous uint8 codes of the output shape, float32 [1])")
        _need_gpu(x8, scale)
    st = _stream(x.device)
    _check("quant_per_tensor", load().quant_per_tensor(_ptr(x), _ptr(x8), _ptr(scale), B, H, S, D,
                                                       _DTYPE[x.dtype], int(bool(transposed)), st))
    return x8, scale


def fwd_fp8(q8, k8, v8, q_scales, k_scales, v_scale, causal=False, scale=None, block_rows=64,
            v_transposed=False, out=None, lse=None):
    """O (bfloat16), LSE from E4M3 inputs and their scales."""
    _need_gpu(q8, k8, v8, q_scales, k_scales, v_scale)
    B, H, S_q, D = q8.shape
    S_k = k8.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, S_q, D), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q8.device)
    st = _stream(q8.device)
    _check("attn_fwd_fp8", load().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scales), _ptr(k_scales),
                                               _ptr(v_scale), _ptr(out), _ptr(lse), B, H, S_q, S_k, D,
                                               int(causal), float(scale), block_rows, int(bool(v_transposed)),
                                               st))
    return out, lse
