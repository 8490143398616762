"""Python binding of libattn.so (argument marshalling only).

Every step of the attention forward pass runs in the library's HIP kernels;
this module only checks tensor metadata, passes device pointers, sizes and
the current HIP stream through ctypes, and turns error codes into
exceptions. torch provides device memory and streams, nothing else. There is
no fallback: if the library is missing or a call is rejected, an exception is
raised.

The names follow include/attn.h: ``attn_fwd``, ``attn_fwd_lse``, ``attn_fwd_fp8``,
``attn_fwd_split``, ``attn_fwd_split_noalloc``, ``attn_split_workspace``, ``attn_split_suggest``,
``attn_fwd_strided``, ``attn_bwd``, ``attn_bwd_workspace``, ``attn_fwd_fp8_lse``,
``attn_bwd_fp8``, ``attn_bwd_fp8_workspace``, ``attn_strerror``; :func:`fwd`, :func:`fwd_lse` and :func:`bwd` are the
tensor-level convenience wrappers.
"""

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_F16, ATTN_FP8_E4M3, ATTN_FP8_E5M2 = 0, 1, 2, 3, 4
FP8_STATE_BYTES = 16 + 4 * 1024   # one delayed-scaling state (see include/attn.h)
FP8_GRAD_DTYPE = torch.float8_e5m2   # gradient input of attn_bwd_fp8
DTYPE_CODE = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16,
              torch.float8_e4m3fn: ATTN_FP8_E4M3}
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_GROUP",
          -4: "ATTN_ERR_HEAD_DIM", -5: "ATTN_ERR_DTYPE", -6: "ATTN_ERR_ALIGN", -7: "ATTN_ERR_ALIAS",
          -8: "ATTN_ERR_SCALE", -9: "ATTN_ERR_HIP", -10: "ATTN_ERR_CAUSAL", -11: "ATTN_ERR_SPLIT",
          -12: "ATTN_ERR_WORKSPACE", -13: "ATTN_ERR_STRIDE", -14: "ATTN_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h
EXPORTS = ("attn_fwd", "attn_fwd_lse", "attn_fwd_fp8", "attn_fwd_fp8_lse", "attn_fwd_split", "attn_fwd_split_noalloc", "attn_split_workspace", "attn_split_suggest",
           "attn_fwd_strided", "attn_bwd", "attn_bwd_workspace", "attn_bwd_fp8", "attn_bwd_fp8_workspace",
           "attn_bwd_fp8_dev", "attn_fp8_state_bytes", "attn_fp8_state_init", "attn_fp8_quantize", "attn_fp8_update",
           "attn_fwd_fp8_dev", "attn_strerror")
# causal argument: 0 none, 1 lower triangle (top-left), 2 bottom-right (Sq <= Skv)
CAUSAL_CODE = {False: 0, True: 1, "top_left": 1, "bottom_right": 2, 0: 0, 1: 1, 2: 2}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded libattn.so with argument types set (loads it once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m scaled_dot_product_09_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.attn_fwd.restype = i
        L.attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.attn_fwd_lse.restype = i
        L.attn_fwd_fp8_lse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, f, f, f, vp]
        L.attn_fwd_fp8_lse.restype = i
        L.attn_bwd_fp8.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, f, f, f, f, vp, ctypes.c_size_t, vp]
        L.attn_bwd_fp8.restype = i
        L.attn_bwd_fp8_workspace.argtypes = [i, i, i, i, i, i]
        L.attn_bwd_fp8_workspace.restype = ctypes.c_size_t
        L.attn_bwd_fp8_dev.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.attn_bwd_fp8_dev.restype = i
        L.attn_fp8_state_bytes.argtypes = []
        L.attn_fp8_state_bytes.restype = ctypes.c_size_t
        L.attn_fp8_state_init.argtypes = [vp, i, i, vp]
        L.attn_fp8_state_init.restype = i
        L.attn_fp8_quantize.argtypes = [vp, i, vp, ctypes.c_int64, vp, vp]
        L.attn_fp8_quantize.restype = i
        L.attn_fp8_update.argtypes = [vp, i, vp]
        L.attn_fp8_update.restype = i
        L.attn_fwd_fp8_dev.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, vp, vp]
        L.attn_fwd_fp8_dev.restype = i
        L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, f, f, f, vp]
        L.attn_fwd_fp8.restype = i
        L.attn_fwd_split.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, ctypes.c_size_t, vp]
        L.attn_fwd_split.restype = i
        L.attn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp]
        L.attn_fwd_split_noalloc.restype = i
        L.attn_split_workspace.argtypes = [i, i, i, i, i]
        L.attn_split_workspace.restype = ctypes.c_size_t
        L.attn_split_suggest.argtypes = [i, i, i, i, i, i, i]
        L.attn_split_suggest.restype = i
        L.attn_fwd_strided.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, vp, vp, f, i, i, vp]
        L.attn_fwd_strided.restype = i
        L.attn_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
        L.attn_bwd.restype = i
        L.attn_bwd_workspace.argtypes = [i, i, i]
        L.attn_bwd_workspace.restype = ctypes.c_size_t
        L.attn_strerror.argtypes = [i]
        L.attn_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_strerror(status):
    return lib().attn_strerror(int(status)).decode()


def attn_fwd(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, stream):
    """Raw C call: pointers as ints, returns the status code."""
    return lib().attn_fwd(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal), int(dtype), stream)


def attn_fwd_lse(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, stream):
    """Raw C call of the forward with the row log-sum-exp output, returns the status code."""
    return lib().attn_fwd_lse(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal), int(dtype),
                              stream)


def attn_fwd_fp8(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, q_descale, k_descale, v_descale, stream):
    """Raw C call of the E4M3 entry point, returns the status code."""
    return lib().attn_fwd_fp8(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal),
                              float(q_descale), float(k_descale), float(v_descale), stream)


def attn_fwd_split(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, n_split, workspace,
                   workspace_bytes, stream):
    """Raw C call of the split-key entry point, returns the status code."""
    return lib().attn_fwd_split(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal), int(dtype),
                                int(n_split), workspace, int(workspace_bytes), stream)


def attn_fwd_split_noalloc(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, n_split, stream):
    """Raw C call of the allocation-free split-key entry point, returns the status code."""
    return lib().attn_fwd_split_noalloc(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal),
                                        int(dtype), int(n_split), stream)


def attn_split_workspace(B, Hq, Sq, D, n_split):
    return int(lib().attn_split_workspace(B, Hq, Sq, D, n_split))


def attn_split_suggest(B, Hq, Hkv, Sq, Skv, D, causal):
    return int(lib().attn_split_suggest(B, Hq, Hkv, Sq, Skv, D, int(causal)))


def attn_fwd_strided(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, q_strides, k_strides, v_strides, out_strides,
                     scale, causal, dtype, stream):
    """Raw C call of the strided entry point (strides: 3 ints each), returns the status code."""
    arr = [(ctypes.c_int64 * 3)(*map(int, st)) for st in (q_strides, k_strides, v_strides, out_strides)]
    return lib().attn_fwd_strided(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, *[ctypes.addressof(a) for a in arr],
                                  float(scale), int(causal), int(dtype), stream)


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, workspace,
             workspace_bytes, stream):
    """Raw C call of the backward pass, returns the status code."""
    return lib().attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal),
                          int(dtype), workspace, int(workspace_bytes), stream)


def attn_bwd_workspace(B, Hq, Sq):
    return int(lib().attn_bwd_workspace(B, Hq, Sq))


def attn_fwd_fp8_lse(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, q_descale, k_descale, v_descale,
                     stream):
    """Raw C call of the E4M3 forward with the row log-sum-exp output, returns the status code."""
    return lib().attn_fwd_fp8_lse(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal),
                                  float(q_descale), float(k_descale), float(v_descale), stream)


def attn_bwd_fp8(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, q_descale,
                 k_descale, v_descale, do_descale, workspace, workspace_bytes, stream):
    """Raw C call of the FP8 (E4M3 inputs, E5M2 gradient) backward pass, returns the status code."""
    return lib().attn_bwd_fp8(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, float(scale),
                              int(causal), float(q_descale), float(k_descale), float(v_descale),
                              float(do_descale), workspace, int(workspace_bytes), stream)


def attn_bwd_fp8_workspace(B, Hq, Hkv, Sq, Skv, D):
    return int(lib().attn_bwd_fp8_workspace(B, Hq, Hkv, Sq, Skv, D))


def attn_bwd_fp8_dev(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, q_descale,
                     k_descale, v_descale, do_descale, workspace, workspace_bytes, stream):
    """Raw C call of the FP8 backward with device-side factor pointers, returns the status code."""
    return lib().attn_bwd_fp8_dev(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, float(scale),
                                  int(causal), q_descale, k_descale, v_descale, do_descale, workspace,
                                  int(workspace_bytes), stream)


def attn_fp8_state_bytes():
    return int(lib().attn_fp8_state_bytes())


def attn_fp8_state_init(states, n_states, fmt, stream):
    return lib().attn_fp8_state_init(states, int(n_states), int(fmt), stream)


def attn_fp8_quantize(x, x_dtype, codes, n, state, stream):
    return lib().attn_fp8_quantize(x, int(x_dtype), codes, int(n), state, stream)


def attn_fp8_update(states, n_states, stream):
    return lib().attn_fp8_update(states, int(n_states), stream)


def attn_fwd_fp8_dev(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, q_descale, k_descale, v_descale,
                     stream):
    """Raw C call of the E4M3 forward with device-side factor pointers, returns the status code."""
    return lib().attn_fwd_fp8_dev(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, float(scale), int(causal), q_descale,
                                  k_descale, v_descale, stream)


def _check(st):
    if st != 0:
        raise AttnError(st, attn_strerror(st))


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D torch tensor (B, S, H, D)")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported or mixed dtypes {q.dtype}, {k.dtype}, {v.dtype}")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")


def _causal_code(causal):
    if causal not in CAUSAL_CODE:
        raise ValueError(f"causal must be one of {sorted(map(str, CAUSAL_CODE))}")
    return CAUSAL_CODE[causal]


def fwd_lse(q, k, v, *, causal=False, scale=None, out=None, lse=None, stream=None, descales=None):
    """(out, lse): the forward of :func:`fwd` plus the float32 row log-sum-exp
    lse[b, h, i] = log sum_j exp(scale q.k) over the visible keys, shape
    (B, Hq, Sq). Contiguous float32 / bfloat16 / float16 tensors, or
    float8_e4m3fn with ``descales`` = (q, k, v) factors (bfloat16 output)."""
    _check_qkv(q, k, v)
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd_lse takes contiguous (B, S, H, D) tensors")
    fp8 = q.dtype == torch.float8_e4m3fn
    if fp8 and descales is None:
        raise ValueError("E4M3 inputs need descales=(q_descale, k_descale, v_descale)")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    causal = _causal_code(causal)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out_dtype = torch.bfloat16 if fp8 else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and device, in the output dtype")
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, Hq, Sq) tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if fp8:
        _check(attn_fwd_fp8_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                B, Hq, Hkv, Sq, Skv, D, scale, causal, *descales, stream))
    else:
        _check(attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, Sq, Skv, D, scale, causal, DTYPE_CODE[q.dtype], stream))
    return out, lse


def fwd(q, k, v, *, causal=False, scale=None, out=None, descales=None, stream=None, n_split=None,
        workspace=None):
    """out = softmax(scale * q k^T [+ causal mask]) v on torch device tensors.

    q: (B, Sq, Hq, D), k and v: (B, Skv, Hkv, D), same dtype (float32,
    bfloat16, float16 or float8_e4m3fn) on one GPU. Non-contiguous views
    (last axis contiguous; e.g. transposed (B, H, S, D) storage or slices of a
    packed buffer) go through attn_fwd_strided (float32 / bfloat16 / float16;
    ``out`` may be such a view too). ``causal``:
    False, True (lower triangle, top-left aligned) or "bottom_right" (the
    queries are the last Sq of Skv positions; needs Sq <= Skv). ``scale``
    defaults to 1 / sqrt(D). E4M3 inputs need ``descales`` = (q, k, v)
    dequantisation factors and produce a bfloat16 output. ``n_split`` (an
    int, or "auto" for the library's suggestion) selects the split-key path
    for bfloat16 / float16, with ``workspace`` a uint8 device tensor of at
    least attn_split_workspace(...) bytes (allocated here if None). The
    kernels are enqueued on ``stream`` (default: torch's current stream);
    nothing is synchronised.
    """
    _check_qkv(q, k, v)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}'s last (head-dimension) axis must be contiguous")
    dense = q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    causal = _causal_code(causal)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code = DTYPE_CODE[q.dtype]
    out_dtype = torch.bfloat16 if code == ATTN_FP8_E4M3 else q.dtype
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or out.device != q.device or out.stride(3) != 1:
        raise ValueError("out must have q's shape, q's device, the output dtype and a contiguous last axis")
    dense = dense and out.is_contiguous()
    if not dense:
        if code == ATTN_FP8_E4M3 or n_split is not None:
            raise ValueError("strided layouts are supported for float32 / bfloat16 / float16 without n_split")
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                              q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3],
                              scale, causal, code, stream)
        _check(st)
        return out
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if n_split is not None:
        if code not in (ATTN_BF16, ATTN_F16):
            raise ValueError("the split-key path takes bfloat16 or float16 inputs")
        if n_split == "auto":
            n_split = attn_split_suggest(B, Hq, Hkv, Sq, Skv, D, causal)
        need = attn_split_workspace(B, Hq, Sq, D, n_split)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
            raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
        st = attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                            scale, causal, code, n_split, workspace.data_ptr(), workspace.numel(), stream)
    elif code == ATTN_FP8_E4M3:
        if descales is None:
            raise ValueError("E4M3 inputs need descales=(q_descale, k_descale, v_descale)")
        st = attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                          scale, causal, *descales, stream)
    else:
        st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                      scale, causal, code, stream)
    _check(st)
    return out


def bwd(q, k, v, out, dout, lse, *, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
        stream=None, descales=None):
    """(dq, dk, dv): gradients of sum(dout * out) for out = fwd(q, k, v).

    ``out`` and ``lse`` come from :func:`fwd_lse` on the same inputs with the
    same ``causal`` and ``scale``; ``dout`` has out's shape. Contiguous
    bfloat16 / float16 tensors on one GPU; the gradients have the inputs'
    shapes and dtype. FP8: q, k, v float8_e4m3fn, out bfloat16, dout
    float8_e5m2, ``descales`` = (q, k, v, dout) factors; bfloat16 gradients
    (attn_bwd_fp8). ``workspace`` is a uint8 device tensor of at least
    attn_bwd_workspace(B, Hq, Sq) (FP8: attn_bwd_fp8_workspace(...)) bytes,
    allocated here if None.
    """
    _check_qkv(q, k, v)
    fp8 = q.dtype == torch.float8_e4m3fn
    if not fp8 and q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("the backward pass takes bfloat16, float16 or E4M3 (with an E5M2 dout) tensors")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse)):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be contiguous and on q's device")
    out_dtype = torch.bfloat16 if fp8 else q.dtype
    do_dtype = FP8_GRAD_DTYPE if fp8 else q.dtype
    if out.shape != q.shape or dout.shape != q.shape or out.dtype != out_dtype or dout.dtype != do_dtype:
        raise ValueError("out and dout must have q's shape; out in the forward's output dtype, dout in q's "
                         "dtype (float8_e5m2 for E4M3 inputs)")
    if fp8 and (descales is None or len(descales) != 4):
        raise ValueError("E4M3 inputs need descales=(q_descale, k_descale, v_descale, dout_descale)")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 (B, Hq, Sq) tensor")
    causal = _causal_code(causal)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    grads = []
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g is None:
            g = torch.empty(ref.shape, dtype=out_dtype, device=ref.device)
        elif g.shape != ref.shape or g.dtype != out_dtype or g.device != ref.device or not g.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor of its input's shape and device, in the "
                             "gradient dtype")
        grads.append(g)
    need = attn_bwd_fp8_workspace(B, Hq, Hkv, Sq, Skv, D) if fp8 else attn_bwd_workspace(B, Hq, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dq, dk, dv = grads
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    if fp8:
        _check(attn_bwd_fp8(*ptrs, B, Hq, Hkv, Sq, Skv, D, scale, causal, *descales, workspace.data_ptr(),
                            workspace.numel(), stream))
    else:
        _check(attn_bwd(*ptrs, B, Hq, Hkv, Sq, Skv, D, scale, causal, DTYPE_CODE[q.dtype], workspace.data_ptr(),
                        workspace.numel(), stream))
    return dq, dk, dv


# ---- FP8 delayed scaling (state in device memory) -------------------------------------------

FP8_FORMAT = {torch.float8_e4m3fn: ATTN_FP8_E4M3, torch.float8_e5m2: ATTN_FP8_E5M2}
FP8_TORCH = {ATTN_FP8_E4M3: torch.float8_e4m3fn, ATTN_FP8_E5M2: torch.float8_e5m2}


def fp8_states(n, fmt, device="cuda:0", stream=None):
    """n delayed-scaling states (a uint8 device tensor of shape (n, FP8_STATE_BYTES)),
    initialised for format ATTN_FP8_E4M3 or ATTN_FP8_E5M2."""
    st = torch.empty((n, FP8_STATE_BYTES), dtype=torch.uint8, device=device)
    if stream is None:
        stream = torch.cuda.current_stream(st.device).cuda_stream
    _check(attn_fp8_state_init(st.data_ptr(), n, fmt, stream))
    return st


def fp8_scale_inv_ptr(state):
    """Device pointer to a state's scale_inv word (its dequantisation factor)."""
    return state.data_ptr() + 4


def fp8_quantize(x, state, fmt, *, out=None, stream=None):
    """FP8 codes of x (float32 / bfloat16 / float16, contiguous) cast with the
    state's current scale; records amax(|x|) in the state's history. ``fmt``
    (ATTN_FP8_E4M3 / ATTN_FP8_E5M2) must be the state's format: it only picks
    the torch dtype of the result (the kernel reads the format from the state)."""
    if not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous GPU tensor")
    code = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(x.dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if out is None:
        out = torch.empty(x.shape, dtype=FP8_TORCH[fmt], device=x.device)
    elif out.dtype != FP8_TORCH[fmt] or out.shape != x.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous FP8 tensor of x's shape in the state's format")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(attn_fp8_quantize(x.data_ptr(), code, out.data_ptr(), x.numel(), state.data_ptr(), stream))
    return out


def fp8_update(states, stream=None):
    """Scale update of every state in a (n, FP8_STATE_BYTES) tensor (or one state row)."""
    n = 1 if states.dim() == 1 else states.shape[0]
    if stream is None:
        stream = torch.cuda.current_stream(states.device).cuda_stream
    _check(attn_fp8_update(states.data_ptr(), n, stream))


def fwd_fp8_dev(q, k, v, states, *, causal=False, scale=None, out=None, lse=None, with_lse=False, stream=None):
    """The E4M3 forward with the q, k, v dequantisation factors read on the
    device from three scaling states (rows of a state tensor). Returns
    (out, lse or None)."""
    _check_qkv(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise ValueError("fwd_fp8_dev takes float8_e4m3fn q, k, v")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    causal = _causal_code(causal)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(attn_fwd_fp8_dev(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Sq, Skv, D, scale, causal,
                            *(fp8_scale_inv_ptr(s) for s in states), stream))
    return out, lse


def bwd_fp8_dev(q, k, v, out, dout, lse, states, *, causal=False, scale=None, workspace=None, stream=None):
    """The FP8 backward (E4M3 q, k, v; E5M2 dout) with the four factors read on
    the device from scaling states (q, k, v, dout). Returns bf16 (dq, dk, dv)."""
    _check_qkv(q, k, v)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    causal = _causal_code(causal)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.bfloat16, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.bfloat16, device=q.device)
    need = attn_bwd_fp8_workspace(B, Hq, Hkv, Sq, Skv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(attn_bwd_fp8_dev(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                            scale, causal, *(fp8_scale_inv_ptr(s) for s in states), workspace.data_ptr(),
                            workspace.numel(), stream))
    return dq, dk, dv
