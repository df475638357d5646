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
}
EXP_MODES = {"native": 0, "poly": 1, "mixed": 2}
BWD_MODES = {"atomic": 0, "split": 1}

# every symbol include/attn97.h declares
EXPORTS = (
    "attn_default_opts", "attn_fwd", "attn_bwd_workspace_bytes", "attn_bwd", "attn_strerror",
    "attn_exp2_eval", "attn_prof_enable", "attn_prof_reset", "attn_prof_collect", "attn_version",
    "attn_fwd_splitkv_workspace_bytes", "attn_fwd_splitkv",
)


class AttnOpts(ctypes.Structure):
    _fields_ = [("exp_mode", ctypes.c_int), ("rescale_tau", ctypes.c_float), ("bwd_mode", ctypes.c_int)]


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
    _lib = lib
    return lib


def _check(fn, code):
    if code != ATTN_OK:
        raise AttnError(fn, code, load().attn_strerror(code).decode())


def make_opts(exp_mode="native", rescale_tau=8.0, bwd_mode="split") -> AttnOpts:
    o = AttnOpts()
    o.exp_mode = EXP_MODES[exp_mode] if isinstance(exp_mode, str) else int(exp_mode)
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
             out=None, lse=None, stream=None):
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
    opts = make_opts(exp_mode, rescale_tau)
    _check("attn_fwd", lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, S, D, float(scale), int(bool(causal)),
                                    ctypes.byref(opts), _stream_ptr(stream)))
    return out, lse


def fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, causal=False, num_splits=0):
    return int(load().attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, int(bool(causal)), int(num_splits)))


def attn_fwd_splitkv(q, k, v, scale=None, causal=False, num_splits=0, exp_mode="native", rescale_tau=8.0,
                     workspace=None, out=None, lse=None, stream=None):
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
    opts = make_opts(exp_mode, rescale_tau)
    _check("attn_fwd_splitkv", lib.attn_fwd_splitkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), B, H, Sq, Sk, D, float(scale), int(bool(causal)),
        int(num_splits), ctypes.byref(opts), _stream_ptr(stream)))
    return out, lse


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


def exp2_eval(x, mode="native", stream=None):
    """The kernels' exp2 applied elementwise to a contiguous float32 device tensor."""
    import torch

    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    y = torch.empty_like(x)
    m = EXP_MODES[mode] if isinstance(mode, str) else int(mode)
    _check("attn_exp2_eval", load().attn_exp2_eval(x.data_ptr(), y.data_ptr(), x.numel(), m, _stream_ptr(stream)))
    return y


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
