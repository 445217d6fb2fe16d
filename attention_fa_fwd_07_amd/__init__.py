"""Python binding of libfa_mi355x (FlashAttention forward, MI355X / gfx950).

Argument marshalling only: every step of the attention forward runs in the
HIP kernels of ``libfa_mi355x.so``. torch supplies device memory and the
current stream. There is no fallback: if the library is missing or the
tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

# status codes (include/fa_mi355x.h)
FA_OK = 0
FA_ERR_NULL_POINTER = 1
FA_ERR_BAD_SHAPE = 2
FA_ERR_UNSUPPORTED_HEAD_DIM = 3
FA_ERR_UNSUPPORTED_DTYPE = 4
FA_ERR_UNSUPPORTED_LAYOUT = 5
FA_ERR_UNSUPPORTED_DROPOUT = 6
FA_ERR_BAD_SCALE = 7
FA_ERR_MISALIGNED = 8
FA_ERR_ALIASING = 9
FA_ERR_HIP = 10
FA_ERR_WORKSPACE = 11
FA_ERR_UNSUPPORTED_MASK = 12
FA_ERR_SCRATCH = 13

FA_LAYOUT_BNSD = 0
FA_LAYOUT_BSHD = 1
FA_F16, FA_BF16, FA_FP8_E4M3, FA_F32 = 0, 1, 2, 3
FA_MASK_NONE, FA_MASK_CAUSAL_TOP_LEFT, FA_MASK_CAUSAL_BOTTOM_RIGHT = 0, 1, 2

EXPORTS = ("fa_fwd", "fa_fwd_ex", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
           "fa_fwd_splitkv_noalloc",
           "fa_fwd_varlen", "fa_fwd_dropout", "fa_bwd", "fa_bwd_dropout", "fa_bwd_workspace_size", "fa_status_str",
           "fa_abi_version")

_lib = None


class FaError(RuntimeError):
    """A launch failure reported by the library (FA_ERR_HIP)."""


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa_mi355x.so and declare its C signatures."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m attention_fa_fwd_07_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp,            # q k v o lse
                           i64, i64, i64, i64, i64,       # B H Sq Sk D
                           ctypes.c_int, ctypes.c_float,  # layout scale
                           ctypes.c_int, ctypes.c_float,  # causal keep_prob
                           ctypes.c_int, ctypes.c_int,    # in_dtype o_dtype
                           vp, vp, vp,                    # descale q k v
                           vp]                            # stream
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = lib.fa_fwd.argtypes[:-1] + [ctypes.c_int, vp, i64, vp]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = lib.fa_fwd.argtypes[:-1] + [ctypes.c_int, vp]
    lib.fa_fwd_ex.restype = ctypes.c_int
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                              ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                              ctypes.c_int, ctypes.c_int, vp, vp, vp,
                              ctypes.c_int, vp, i64, vp]
    lib.fa_fwd_varlen.restype = ctypes.c_int
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp,         # q k v o lse cu_q cu_k
                                  i64, i64, i64, i64, i64, i64, i64,  # B H H_kv tq tk maxq D
                                  ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                  ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
    lib.fa_fwd_dropout.restype = ctypes.c_int
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                   ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                   ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                   vp, vp, vp, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp,          # q k v o dout lse
                           vp, vp, vp,                      # dq dk dv
                           i64, i64, i64, i64, i64, i64,    # B H H_kv Sq Sk D
                           ctypes.c_float, ctypes.c_int,    # scale mask
                           ctypes.c_int, ctypes.c_int,      # in_dtype grad_dtype
                           vp, i64, vp]                     # workspace size stream
    lib.fa_bwd_dropout.restype = ctypes.c_int
    lib.fa_bwd_dropout.argtypes = lib.fa_bwd.argtypes[:17] + [ctypes.c_float, ctypes.c_uint64,
                                                              ctypes.c_uint64] + lib.fa_bwd.argtypes[17:]
    lib.fa_bwd_workspace_size.restype = i64
    lib.fa_bwd_workspace_size.argtypes = [i64, i64, i64]
    lib.fa_fwd_splitkv_workspace_size.restype = i64
    lib.fa_fwd_splitkv_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_abi_version.restype = ctypes.c_int
    lib.fa_abi_version.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().fa_status_str(code).decode()


def fa_fwd_raw(q, k, v, o, lse, B, H, Sq, Sk, D, layout, scale, causal, keep_prob,
               in_dtype, o_dtype, descale_q, descale_k, descale_v, stream) -> int:
    """The C entry point with integer pointers; returns the status code."""
    return load_library().fa_fwd(q, k, v, o, lse, B, H, Sq, Sk, D, layout, scale,
                                 causal, keep_prob, in_dtype, o_dtype,
                                 descale_q, descale_k, descale_v, stream)


def fa_fwd_splitkv_raw(q, k, v, o, lse, B, H, Sq, Sk, D, layout, scale, causal, keep_prob,
                       in_dtype, o_dtype, descale_q, descale_k, descale_v, num_splits,
                       workspace, workspace_size, stream) -> int:
    """The split-KV C entry point with integer pointers; returns the status code."""
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, H, Sq, Sk, D, layout, scale,
                                         causal, keep_prob, in_dtype, o_dtype, descale_q,
                                         descale_k, descale_v, num_splits, workspace,
                                         workspace_size, stream)


def fa_fwd_splitkv_noalloc_raw(q, k, v, o, lse, B, H, Sq, Sk, D, layout, scale, causal, keep_prob,
                               in_dtype, o_dtype, descale_q, descale_k, descale_v, num_splits,
                               stream) -> int:
    """The split-KV C entry point that allocates nothing (its workspace is a
    static device array of the library); integer pointers, returns the status."""
    return load_library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D, layout, scale,
                                                 causal, keep_prob, in_dtype, o_dtype, descale_q,
                                                 descale_k, descale_v, num_splits, stream)


def fa_fwd_ex_raw(q, k, v, o, lse, B, H, H_kv, Sq, Sk, D, layout, scale, mask, keep_prob,
                  in_dtype, o_dtype, descale_q, descale_k, descale_v, num_splits, workspace,
                  workspace_size, stream) -> int:
    """The general C entry point with integer pointers; returns the status code."""
    return load_library().fa_fwd_ex(q, k, v, o, lse, B, H, H_kv, Sq, Sk, D, layout, scale, mask,
                                    keep_prob, in_dtype, o_dtype, descale_q, descale_k,
                                    descale_v, num_splits, workspace, workspace_size, stream)


def fa_fwd_varlen_raw(q, k, v, o, lse, cu_q, cu_k, B, H, H_kv, total_q, total_k, max_seqlen_q,
                      D, scale, mask, keep_prob, in_dtype, o_dtype, descale_q, descale_k,
                      descale_v, stream) -> int:
    """The packed variable-length C entry point with integer pointers."""
    return load_library().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, H_kv, total_q,
                                        total_k, max_seqlen_q, D, scale, mask, keep_prob,
                                        in_dtype, o_dtype, descale_q, descale_k, descale_v,
                                        stream)


def fa_fwd_dropout_raw(q, k, v, o, lse, B, H, H_kv, Sq, Sk, D, layout, scale, mask, keep_prob,
                       seed, offset, in_dtype, o_dtype, descale_q, descale_k, descale_v,
                       stream) -> int:
    """The dropout C entry point with integer pointers; returns the status code."""
    return load_library().fa_fwd_dropout(q, k, v, o, lse, B, H, H_kv, Sq, Sk, D, layout, scale,
                                         mask, keep_prob, seed, offset, in_dtype, o_dtype,
                                         descale_q, descale_k, descale_v, stream)


def fa_bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Sq, Sk, D, scale, mask,
               in_dtype, grad_dtype, workspace, workspace_size, stream) -> int:
    """The backward C entry point with integer pointers; returns the status code."""
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Sq, Sk, D,
                                 scale, mask, in_dtype, grad_dtype, workspace, workspace_size,
                                 stream)


def fa_bwd_dropout_raw(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Sq, Sk, D, scale, mask,
                       keep_prob, seed, offset, in_dtype, grad_dtype, workspace, workspace_size,
                       stream) -> int:
    """The backward-with-dropout C entry point with integer pointers."""
    return load_library().fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, Sq, Sk,
                                         D, scale, mask, keep_prob, seed, offset, in_dtype,
                                         grad_dtype, workspace, workspace_size, stream)


def bwd_workspace_size(B, H, Sq) -> int:
    """Workspace bytes fa_bwd needs (-1: rejected sizes)."""
    return load_library().fa_bwd_workspace_size(B, H, Sq)


def splitkv_workspace_size(B, H, Sq, Sk, D, causal=False, num_splits=0) -> int:
    """Workspace bytes fa_fwd_splitkv needs (0: a single range; -1: rejected sizes)."""
    return load_library().fa_fwd_splitkv_workspace_size(B, H, Sq, Sk, D, 1 if causal else 0,
                                                        num_splits)


def _dtype_code(dt) -> int:
    import torch
    table = {torch.float16: FA_F16, torch.bfloat16: FA_BF16,
             torch.float8_e4m3fn: FA_FP8_E4M3, torch.float32: FA_F32}
    if dt not in table:
        raise ValueError(f"unsupported dtype {dt}")
    return table[dt]


def _check_status(code: int) -> None:
    if code == FA_OK:
        return
    name = status_str(code)
    if code == FA_ERR_HIP:
        raise FaError(name)
    raise ValueError(name)


def fa_fwd(q, k, v, *, scale: float | None = None, causal: bool = False,
           keep_prob: float = 1.0, o_dtype=None, descale_q=None, descale_k=None,
           descale_v=None, out=None, lse=None, stream=None, layout: str = "BNSD",
           seed: int | None = None, rng_offset: int = 0):
    """Attention forward over BNSD tensors on the GPU.

    q [B,H,Sq,D], k/v [B,H_kv,Sk,D] contiguous GPU tensors (fp16, bf16 or
    float8_e4m3fn; H_kv divides H: query head h uses key/value head
    h // (H / H_kv)). ``causal``: False, True (= "top_left": key j visible to
    query i iff j <= i) or "bottom_right" (iff j <= i + Sk - Sq).
    ``layout="BSHD"``: q, o [B,Sq,H,D] and k, v [B,Sk,H_kv,D] instead (lse
    stays [B,H,Sq]). fp8 inputs need ``descale_*``: one-element fp32 GPU
    tensors (value = code * descale). Returns (o, lse): o [B,H,Sq,D] in
    ``o_dtype`` (default: fp16 for fp16/fp8 inputs, bf16 for bf16 inputs),
    lse [B,H,Sq] fp32 (natural-log logsumexp of the scaled, masked scores).
    ``keep_prob`` < 1 applies dropout (fa_fwd_dropout) with the mask drawn
    from ``seed`` (required then) and ``rng_offset``.
    """
    if keep_prob != 1.0:
        if seed is None:
            raise ValueError("dropout (keep_prob < 1) needs a seed")
        return _call(q, k, v, scale, causal, keep_prob, o_dtype, descale_q, descale_k,
                     descale_v, out, lse, stream, None, None, layout,
                     dropout=(int(seed), int(rng_offset)))
    return _call(q, k, v, scale, causal, keep_prob, o_dtype, descale_q, descale_k, descale_v,
                 out, lse, stream, None, None, layout)


def _check_buffer(name, t, shape, dtypes, device):
    """A caller-supplied buffer must be a contiguous GPU tensor on ``device``
    with exactly ``shape`` and a dtype in ``dtypes``: the C ABI takes bare
    pointers and cannot check sizes, so a short or misplaced buffer would be
    written or read out of bounds."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")


def _check_inputs(names_tensors):
    """q, k, v (and the like): contiguous GPU tensors on one device."""
    dev = None
    for name, t in names_tensors:
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} must be on {dev}, not {t.device}")
    return dev


def _check_descales(ds, dev):
    import torch
    for name, t in zip(("descale_q", "descale_k", "descale_v"), ds):
        if t is not None:
            _check_buffer(name, t, tuple(t.shape), (torch.float32,), dev)
            if t.numel() != 1:
                raise ValueError(f"{name} must hold exactly one float32")


def _check_workspace(ws, dev):
    import torch
    if ws is not None:
        _check_buffer("workspace", ws, (ws.numel(),), (torch.uint8,), dev)


def _mask_code(causal) -> int:
    if causal is False or causal is None:
        return FA_MASK_NONE
    if causal is True or causal == "top_left":
        return FA_MASK_CAUSAL_TOP_LEFT
    if causal == "bottom_right":
        return FA_MASK_CAUSAL_BOTTOM_RIGHT
    raise ValueError(f"causal must be False, True, 'top_left' or 'bottom_right', not {causal!r}")


def fa_fwd_splitkv(q, k, v, *, num_splits: int = 0, scale: float | None = None,
                   causal: bool = False, keep_prob: float = 1.0, o_dtype=None, descale_q=None,
                   descale_k=None, descale_v=None, out=None, lse=None, workspace=None,
                   stream=None, layout: str = "BNSD"):
    """fa_fwd with the keys of each query block split into ``num_splits``
    ranges (0: chosen by the library, 1 unless the plain grid would leave
    most of the GPU idle), merged by logsumexp. ``workspace``:
    an optional uint8 GPU tensor of at least ``splitkv_workspace_size(...)``
    bytes (allocated here when not given)."""
    return _call(q, k, v, scale, causal, keep_prob, o_dtype, descale_q, descale_k, descale_v,
                 out, lse, stream, int(num_splits), workspace, layout)


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, *,
                  scale: float | None = None, causal: bool = False, keep_prob: float = 1.0,
                  o_dtype=None, descale_q=None, descale_k=None, descale_v=None, out=None,
                  lse=None, stream=None):
    """Attention forward over a batch of sequences of different lengths.

    q [total_q,H,D], k/v [total_k,H_kv,D]: the sequences packed one after
    the other (contiguous GPU tensors); ``cu_seqlens_q``/``cu_seqlens_k``:
    int32 GPU tensors of B+1 offsets from 0 to total_q (total_k), sequence b
    owning rows cu[b]..cu[b+1]-1; ``max_seqlen_q``: the longest query
    length. Each sequence is attended on its own (``causal`` as in fa_fwd,
    per sequence). Returns (o [total_q,H,D], lse [H,total_q] fp32).
    """
    import torch
    dev = _check_inputs((("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                         ("cu_seqlens_k", cu_seqlens_k)))
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [total, heads, D]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of the same length B+1")
    tq, H, D = q.shape
    tk, Hkv = k.shape[0], k.shape[1]
    if tuple(k.shape) != (tk, Hkv, D) or tuple(v.shape) != (tk, Hkv, D):
        raise ValueError("k and v must be [total_k, H_kv, D] with q's D")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B = cu_seqlens_q.shape[0] - 1
    if o_dtype is None:
        o_dtype = out.dtype if out is not None else (
            torch.bfloat16 if q.dtype == torch.bfloat16 else torch.float16)
    if o_dtype not in (torch.float16, torch.bfloat16, torch.float32):
        raise ValueError(f"o_dtype must be float16, bfloat16 or float32, not {o_dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is not None:
        _check_buffer("out", out, q.shape, (o_dtype,), dev)
    if lse is not None:
        _check_buffer("lse", lse, (H, tq), (torch.float32,), dev)
    _check_descales((descale_q, descale_k, descale_v), dev)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=o_dtype, device=dev)
    if lse is None:
        lse = torch.empty((H, tq), dtype=torch.float32, device=dev)
    dq = descale_q.data_ptr() if descale_q is not None else None
    dk = descale_k.data_ptr() if descale_k is not None else None
    dv = descale_v.data_ptr() if descale_v is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check_status(fa_fwd_varlen_raw(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, Hkv, tq, tk, int(max_seqlen_q),
        D, float(scale), _mask_code(causal), float(keep_prob), _dtype_code(q.dtype),
        _dtype_code(out.dtype), dq, dk, dv, stream))
    return out, lse


def fa_bwd(q, k, v, o, dout, lse, *, scale: float | None = None, causal: bool = False,
           grad_dtype=None, dq=None, dk=None, dv=None, workspace=None, stream=None,
           keep_prob: float = 1.0, seed: int | None = None, rng_offset: int = 0):
    """Gradients (dq, dk, dv) of the attention forward for the cotangent
    ``dout``, from the forward's output ``o`` and ``lse``.

    q, o, dout [B,H,Sq,D] and k, v [B,H_kv,Sk,D]: contiguous BNSD GPU tensors
    of one dtype (fp16 or bf16); lse [B,H,Sq] fp32. ``causal`` as in fa_fwd.
    ``grad_dtype``: dtype of the gradients (default: the input dtype; or
    float32). ``workspace``: an optional uint8 GPU tensor of at least
    ``bwd_workspace_size(B, H, Sq)`` bytes (allocated here when not given).
    ``keep_prob`` < 1: the backward of fa_fwd with dropout; ``seed`` and
    ``rng_offset`` must be the forward's.
    """
    import torch
    dev = _check_inputs((("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse)))
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, D) or tuple(v.shape) != (B, Hkv, Sk, D):
        raise ValueError("k and v must be [B, H_kv, Sk, D] with q's B and D")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Sq]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise ValueError("q, k, v, o, dout must share a dtype")
    if grad_dtype is None:
        grad_dtype = dq.dtype if dq is not None else q.dtype
    if grad_dtype not in (q.dtype, torch.float32):
        raise ValueError("grad_dtype must be the input dtype or float32")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    for name, t, shp in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, v.shape)):
        if t is not None:
            _check_buffer(name, t, shp, (grad_dtype,), dev)
    _check_workspace(workspace, dev)
    if dq is None:
        dq = torch.empty(tuple(q.shape), dtype=grad_dtype, device=dev)
    if dk is None:
        dk = torch.empty(tuple(k.shape), dtype=grad_dtype, device=dev)
    if dv is None:
        dv = torch.empty(tuple(v.shape), dtype=grad_dtype, device=dev)
    need = bwd_workspace_size(B, H, Sq)
    if need < 0:
        raise ValueError("FA_ERR_BAD_SHAPE")
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    base = workspace.data_ptr()
    ws = (base + 255) // 256 * 256
    ws_size = workspace.numel() - (ws - base)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    shape = (B, H, Hkv, Sq, Sk, D, float(scale), _mask_code(causal))
    tail = (_dtype_code(q.dtype), _dtype_code(dq.dtype), ws, ws_size, stream)
    if keep_prob != 1.0:
        if seed is None:
            raise ValueError("dropout (keep_prob < 1) needs the forward's seed")
        _check_status(fa_bwd_dropout_raw(*ptrs, *shape, float(keep_prob),
                                         int(seed) & ((1 << 64) - 1),
                                         int(rng_offset) & ((1 << 64) - 1), *tail))
    else:
        _check_status(fa_bwd_raw(*ptrs, *shape, *tail))
    return dq, dk, dv


def _call(q, k, v, scale, causal, keep_prob, o_dtype, descale_q, descale_k, descale_v,
          out, lse, stream, num_splits, workspace, layout="BNSD", dropout=None):
    import torch
    dev = _check_inputs((("q", q), ("k", k), ("v", v)))
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    if layout == "BNSD":
        lay = FA_LAYOUT_BNSD
        B, H, Sq, D = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        kv_shape = (B, Hkv, Sk, D)
    elif layout == "BSHD":
        lay = FA_LAYOUT_BSHD
        B, Sq, H, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
        kv_shape = (B, Sk, Hkv, D)
    else:
        raise ValueError(f"layout must be 'BNSD' or 'BSHD', not {layout!r}")
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"k and v must be {layout} with q's B and D")
    mask = _mask_code(causal)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    in_code = _dtype_code(q.dtype)
    if o_dtype is None:
        o_dtype = out.dtype if out is not None else (
            torch.bfloat16 if q.dtype == torch.bfloat16 else torch.float16)
    if o_dtype not in (torch.float16, torch.bfloat16, torch.float32):
        raise ValueError(f"o_dtype must be float16, bfloat16 or float32, not {o_dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is not None:
        _check_buffer("out", out, q.shape, (o_dtype,), dev)
    if lse is not None:
        _check_buffer("lse", lse, (B, H, Sq), (torch.float32,), dev)
    _check_descales((descale_q, descale_k, descale_v), dev)
    _check_workspace(workspace, dev)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=o_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    dq = descale_q.data_ptr() if descale_q is not None else None
    dk = descale_k.data_ptr() if descale_k is not None else None
    dv = descale_v.data_ptr() if descale_v is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    tail = (float(keep_prob), in_code, _dtype_code(out.dtype), dq, dk, dv)
    if dropout is not None:
        _check_status(fa_fwd_dropout_raw(*ptrs, B, H, Hkv, Sq, Sk, D, lay, float(scale), mask,
                                         float(keep_prob), dropout[0] & ((1 << 64) - 1),
                                         dropout[1] & ((1 << 64) - 1), *tail[1:], stream))
        return out, lse
    general = Hkv != H or mask == FA_MASK_CAUSAL_BOTTOM_RIGHT or lay != FA_LAYOUT_BNSD
    args = ptrs + (B, H, Sq, Sk, D, FA_LAYOUT_BNSD, float(scale), 1 if mask else 0) + tail
    if num_splits is None and not general:
        _check_status(fa_fwd_raw(*args, stream))
        return out, lse
    ns = 1 if num_splits is None else num_splits
    need = splitkv_workspace_size(B, H, Sq, Sk, D, mask != FA_MASK_NONE, ns)
    if need < 0:
        raise ValueError("FA_ERR_BAD_SHAPE")
    if workspace is None and need > 0:
        # 256 extra bytes so the start can be aligned to 256
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    if workspace is not None:
        base = workspace.data_ptr()
        ws = (base + 255) // 256 * 256
        ws_size = workspace.numel() - (ws - base)
    else:
        ws, ws_size = None, 0
    if general:
        ex = ptrs + (B, H, Hkv, Sq, Sk, D, lay, float(scale), mask) + tail
        _check_status(fa_fwd_ex_raw(*ex, ns, ws, ws_size, stream))
    else:
        _check_status(fa_fwd_splitkv_raw(*args, ns, ws, ws_size, stream))
    return out, lse
