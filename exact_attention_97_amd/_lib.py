"""ctypes binding of libattn97.so (the C ABI in include/attn97.h).

Argument marshalling only: every step of attention runs in the HIP kernels.
PyTorch supplies device memory and the current HIP stream.  If the library
is missing, every call raises; there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn97.so")

# status codes (attn_status)
ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_VALUE",
    8: "ATTN_ERR_SCRATCH_LIMIT",
}
NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES
EXP_MODES = {"native": 0, "poly": 1, "mixed": 2}
BWD_MODES = {"atomic": 0, "split": 1}

# every symbol include/attn97.h declares
EXPORTS = (
    "attn_default_opts", "attn_fwd", "attn_bwd_workspace_bytes", "attn_bwd", "attn_strerror",
    "attn_exp2_eval", "attn_prof_enable", "attn_prof_reset", "attn_prof_collect", "attn_version",
    "attn_fwd_splitkv_workspace_bytes", "attn_fwd_splitkv",
    "attn_fp8_buffer_bytes", "attn_fp8_buffer_offsets", "attn_fp8_quantize", "attn_fwd_fp8",
    "attn_set_variant", "attn_fp8_dot_eval", "attn_bwd_noalloc",
)
FP8_REGIONS = ("q8", "k8", "v8t", "qs", "ks", "vs", "scratch")


class AttnOpts(ctypes.Structure):
    _fields_ = [("exp_mode", ctypes.c_int), ("poly_fraction", ctypes.c_float), ("rescale_tau", ctypes.c_float),
                ("bwd_mode", ctypes.c_int)]


class AttnError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(code, code)} ({text})")
        self.code = code


_lib = None


def load():
    """Load libattn97.so (once) and declare its prototypes; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run exact_attention_97_amd/build_lib.py "
            "(or __graft_entry__.build()); the attention library has no fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    optp = ctypes.POINTER(AttnOpts)
    lib.attn_default_opts.argtypes = [optp]
    lib.attn_default_opts.restype = None
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, optp, vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, optp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, optp, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, optp, vp]
    lib.attn_bwd_noalloc.restype = i
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_exp2_eval.argtypes = [vp, vp, ctypes.c_long, i, vp]
    lib.attn_exp2_eval.restype = i
    lib.attn_prof_enable.argtypes = [i]
    lib.attn_prof_enable.restype = i
    lib.attn_prof_reset.argtypes = []
    lib.attn_prof_reset.restype = i
    lib.attn_prof_collect.argtypes = [ctypes.c_char_p, ctypes.POINTER(i), ctypes.POINTER(ctypes.c_double)]
    lib.attn_prof_collect.restype = i
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.attn_fwd_splitkv_workspace_bytes.restype = sz
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, optp, vp]
    lib.attn_fwd_splitkv.restype = i
    lib.attn_fp8_buffer_bytes.argtypes = [i, i, i, i]
    lib.attn_fp8_buffer_bytes.restype = sz
    lib.attn_fp8_buffer_offsets.argtypes = [i, i, i, i, ctypes.POINTER(sz)]
    lib.attn_fp8_buffer_offsets.restype = i
    lib.attn_fp8_quantize.argtypes = [vp, vp, vp, vp, vp, sz, i, i, i, i, vp]
    lib.attn_fp8_quantize.restype = i
    lib.attn_fwd_fp8.argtypes = [vp, sz, vp, vp, i, i, i, i, f, i, optp, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fp8_dot_eval.argtypes = [vp, vp, vp, ctypes.c_long, vp]
    lib.attn_fp8_dot_eval.restype = i
    lib.attn_set_variant.argtypes = [ctypes.c_char_p, i]
    lib.attn_set_variant.restype = i
    _lib = lib
    return lib


def _check(fn, code):
    if code != ATTN_OK:
        raise AttnError(fn, code, load().attn_strerror(code).decode())


def make_opts(exp_mode="native", rescale_tau=8.0, bwd_mode="split", poly_fraction=0.5) -> AttnOpts:
    o = AttnOpts()
    o.exp_mode = EXP_MODES[exp_mode] if isinstance(exp_mode, str) else int(exp_mode)
    o.poly_fraction = float(poly_fraction)
    o.rescale_tau = float(rescale_tau)
    o.bwd_mode = BWD_MODES[bwd_mode] if isinstance(bwd_mode, str) else int(bwd_mode)
    return o


def _stream_ptr(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_qkv(*ts):
    import torch

    shape = ts[0].shape
    for t in ts:
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous bfloat16 CUDA/HIP tensors")
        if t.shape != shape or t.dim() != 4:
            raise ValueError(f"attention tensors must share one [B,H,S,D] shape, got {[tuple(x.shape) for x in ts]}")
    return shape


def attn_fwd(q, k, v, scale=None, causal=False, exp_mode="native", rescale_tau=8.0,
             out=None, lse=None, stream=None, poly_fraction=0.5):
    """Forward pass; returns (O bf16 [B,H,S,D], LSE fp32 [B,H,S])."""
    import torch

    lib = load()
    B, H, S, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    opts = make_opts(exp_mode, rescale_tau, poly_fraction=poly_fraction)
    _check("attn_fwd", lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, S, D, float(scale), int(bool(causal)),
                                    ctypes.byref(opts), _stream_ptr(stream)))
    return out, lse


def fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, causal=False, num_splits=0):
    return int(load().attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, int(bool(causal)), int(num_splits)))


def attn_fwd_splitkv(q, k, v, scale=None, causal=False, num_splits=0, exp_mode="native", rescale_tau=8.0,
                     workspace=None, out=None, lse=None, stream=None, poly_fraction=0.5):
    """Split-KV forward: q [B,H,Sq,D], k/v [B,H,Sk,D]; returns (O bf16 [B,H,Sq,D], LSE fp32 [B,H,Sq])."""
    import torch

    lib = load()
    for t in (q, k, v):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("attention tensors must be contiguous 4-d bfloat16 CUDA/HIP tensors")
    B, H, Sq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError(f"k and v must be [B,H,Sk,D] matching q {tuple(q.shape)}, got {tuple(k.shape)}")
    Sk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    need = fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, causal, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    opts = make_opts(exp_mode, rescale_tau, poly_fraction=poly_fraction)
    _check("attn_fwd_splitkv", lib.attn_fwd_splitkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), B, H, Sq, Sk, D, float(scale), int(bool(causal)),
        int(num_splits), ctypes.byref(opts), _stream_ptr(stream)))
    return out, lse


def fp8_buffer_bytes(B, H, S, D):
    return int(load().attn_fp8_buffer_bytes(B, H, S, D))


def fp8_buffer_views(buf, B, H, S, D):
    """Views of the regions of an FP8 buffer (layout of include/attn97.h): dict name -> tensor."""
    import torch

    offs = (ctypes.c_size_t * 7)()
    _check("attn_fp8_buffer_offsets", load().attn_fp8_buffer_offsets(B, H, S, D, offs))
    Sp = (S + 127) // 128 * 128
    BH = B * H
    shapes = {"q8": ((BH, Sp, D), torch.uint8), "k8": ((BH, Sp, D), torch.uint8), "v8t": ((BH, D, Sp), torch.uint8),
              "qs": ((BH, Sp), torch.float32), "ks": ((BH,), torch.float32), "vs": ((BH, D), torch.float32)}
    out = {}
    for n, name in enumerate(FP8_REGIONS[:6]):
        shape, dt = shapes[name]
        nbytes = math.prod(shape) * (4 if dt == torch.float32 else 1)
        out[name] = buf[offs[n]:offs[n] + nbytes].view(dt).view(shape)
    return out


def fp8_quantize(q, k, v, signs=None, buf=None, stream=None):
    """Transform (with signs, a float32 [D] device tensor of +-1) and quantize Q, K, V to E4M3; returns the buffer."""
    import torch

    lib = load()
    B, H, S, D = _check_qkv(q, k, v)
    need = fp8_buffer_bytes(B, H, S, D)
    if buf is None:
        buf = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if signs is not None and (signs.dtype != torch.float32 or not signs.is_cuda or signs.numel() != D):
        raise ValueError("signs must be a float32 device tensor of D elements")
    _check("attn_fp8_quantize", lib.attn_fp8_quantize(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), None if signs is None else signs.data_ptr(), buf.data_ptr(),
        buf.numel(), B, H, S, D, _stream_ptr(stream)))
    return buf


def attn_fwd_fp8_quantized(buf, B, H, S, D, scale=None, causal=False, rescale_tau=8.0, out=None, lse=None,
                           device=None, stream=None):
    """FP8 forward from a quantized buffer; returns (O bf16 [B,H,S,D], LSE fp32 [B,H,S])."""
    import torch

    lib = load()
    dev = buf.device if device is None else device
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    opts = make_opts(rescale_tau=rescale_tau)
    _check("attn_fwd_fp8", lib.attn_fwd_fp8(buf.data_ptr(), buf.numel(), out.data_ptr(), lse.data_ptr(), B, H, S, D,
                                            float(scale), int(bool(causal)), ctypes.byref(opts),
                                            _stream_ptr(stream)))
    return out, lse


def attn_fwd_fp8(q, k, v, signs=None, scale=None, causal=False, rescale_tau=8.0, buf=None, out=None, lse=None,
                 stream=None):
    """FP8 forward with incoherent processing: quantize then attend; returns (O, LSE)."""
    B, H, S, D = _check_qkv(q, k, v)
    buf = fp8_quantize(q, k, v, signs, buf, stream)
    return attn_fwd_fp8_quantized(buf, B, H, S, D, scale, causal, rescale_tau, out, lse, q.device, stream)


def bwd_workspace_bytes(B, H, S, D, causal=False, bwd_mode="split"):
    opts = make_opts(bwd_mode=bwd_mode)
    return int(load().attn_bwd_workspace_bytes(B, H, S, D, int(bool(causal)), ctypes.byref(opts)))


def attn_bwd(q, k, v, o, do, lse, scale=None, causal=False, bwd_mode="split",
             workspace=None, dq=None, dk=None, dv=None, stream=None):
    """Backward pass; returns (dQ, dK, dV), bf16 [B,H,S,D]."""
    import torch

    lib = load()
    B, H, S, D = _check_qkv(q, k, v, o, do)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    opts = make_opts(bwd_mode=bwd_mode)
    need = int(lib.attn_bwd_workspace_bytes(B, H, S, D, int(bool(causal)), ctypes.byref(opts)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check("attn_bwd", lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    B, H, S, D, float(scale), int(bool(causal)), ctypes.byref(opts),
                                    _stream_ptr(stream)))
    return dq, dk, dv


def fp8_dot_eval(a, bt, stream=None):
    """The FP8 forward's score product on E4M3 codes: a, bt uint8 device tensors
    [n, 32, 128] (bt holds B transposed); returns C = a @ bt^T, fp32 [n, 32, 32]."""
    import torch

    for t in (a, bt):
        if not t.is_cuda or t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 3 \
                or tuple(t.shape[1:]) != (32, 128):
            raise ValueError("a and bt must be contiguous uint8 device tensors [n, 32, 128]")
    if a.shape != bt.shape:
        raise ValueError("a and bt must have the same shape")
    c = torch.empty((a.shape[0], 32, 32), dtype=torch.float32, device=a.device)
    _check("attn_fp8_dot_eval", load().attn_fp8_dot_eval(a.data_ptr(), bt.data_ptr(), c.data_ptr(), a.shape[0],
                                                         _stream_ptr(stream)))
    return c


def attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, bwd_mode="split", stream=None):
    """Backward pass with the library's fixed device scratch as its workspace
    (attn_bwd_noalloc): the caller passes every input and output (dq, dk, dv
    bf16 [B,H,S,D]); nothing is allocated.  Returns (dq, dk, dv)."""
    import torch

    lib = load()
    B, H, S, D = _check_qkv(q, k, v, o, do, dq, dk, dv)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    opts = make_opts(bwd_mode=bwd_mode)
    _check("attn_bwd_noalloc", lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                    do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                                    dv.data_ptr(), B, H, S, D, float(scale), int(bool(causal)),
                                                    ctypes.byref(opts), _stream_ptr(stream)))
    return dq, dk, dv


def exp2_eval(x, mode="native", stream=None):
    """The kernels' exp2 applied elementwise to a contiguous float32 device tensor."""
    import torch

    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    y = torch.empty_like(x)
    m = EXP_MODES[mode] if isinstance(mode, str) else int(mode)
    _check("attn_exp2_eval", load().attn_exp2_eval(x.data_ptr(), y.data_ptr(), x.numel(), m, _stream_ptr(stream)))
    return y


def set_variant(kernel, variant):
    """Select a measured kernel variant ("fwd", "bwd_dq"); -1 = back to the environment's choice."""
    _check("attn_set_variant", load().attn_set_variant(kernel.encode(), int(variant)))


def prof_enable(on=True):
    _check("attn_prof_enable", load().attn_prof_enable(int(bool(on))))


def prof_reset():
    _check("attn_prof_reset", load().attn_prof_reset())


def prof_collect(kernel):
    """(launch count, summed milliseconds) of one library kernel since the last reset."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check("attn_prof_collect", load().attn_prof_collect(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def version():
    return load().attn_version().decode()
