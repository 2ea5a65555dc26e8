"""ctypes binding of libssm.so (include/ssm.h).  Argument marshalling only: every step of
the scan runs in the library's HIP kernels.  PyTorch supplies device memory and the
current HIP stream.  There is no fallback: a missing library raises."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSM_SANITIZE=1 selects the host-sanitized build (build.py --sanitize; CPU test runs only).
LIB_PATH = os.path.join(_HERE, "libssm_san.so" if os.environ.get("SSM_SANITIZE") == "1" else "libssm.so")

SSM_F32, SSM_BF16 = 0, 1
ABI_VERSION = 2
MAX_STATE = 16
CONV_W = 4

STATUS = {0: "SSM_OK", 1: "SSM_ERR_NULL", 2: "SSM_ERR_SHAPE", 3: "SSM_ERR_DTYPE", 4: "SSM_ERR_ALIGN",
          5: "SSM_ERR_ALIAS", 6: "SSM_ERR_WORKSPACE", 7: "SSM_ERR_LAUNCH", 8: "SSM_ERR_SCRATCH"}


class SsmError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_inner", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("d_conv", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("chunk_hint", ctypes.c_int32)]


class Params(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("Dskip", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libssm.so and declare its entry points (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run python selective_state_space_causal_amd/build.py "
                          "(hipcc for gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.ssm_abi_version.restype = ctypes.c_int
    lib.ssm_abi_version.argtypes = []
    lib.ssm_status_str.restype = ctypes.c_char_p
    lib.ssm_status_str.argtypes = [ctypes.c_int]
    lib.ssm_prefill_workspace_bytes.restype = sz
    lib.ssm_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    lib.ssm_prefill.restype = ctypes.c_int
    lib.ssm_prefill.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params)] + [vp] * 11 + [sz, vp]
    lib.ssm_decode_step.restype = ctypes.c_int
    lib.ssm_decode_step.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params)] + [vp] * 9
    i64, cint = ctypes.c_int64, ctypes.c_int
    lib.ssm_prefill_pool.restype = ctypes.c_int
    lib.ssm_prefill_pool.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params)] + [vp] * 7 + [i64, cint] + \
        [vp] * 4
    lib.ssm_decode_step_pool.restype = ctypes.c_int
    lib.ssm_decode_step_pool.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params)] + [vp] * 6 + [i64] + \
        [vp] * 4
    lib.ssm_q8_num_blocks.restype = i64
    lib.ssm_q8_num_blocks.argtypes = [i64, ctypes.c_int32]
    lib.ssm_q8_quantize.restype = ctypes.c_int
    lib.ssm_q8_quantize.argtypes = [i64, ctypes.c_int32, ctypes.c_int32] + [vp] * 4
    lib.ssm_q8_dequant_sum.restype = ctypes.c_int
    lib.ssm_q8_dequant_sum.argtypes = [i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp]
    lib.ssm_proj_create.restype = ctypes.c_int
    lib.ssm_proj_create.argtypes = [ctypes.POINTER(vp)]
    lib.ssm_proj_destroy.restype = None
    lib.ssm_proj_destroy.argtypes = [vp]
    lib.ssm_proj_workspace_bytes.restype = sz
    lib.ssm_proj_workspace_bytes.argtypes = []
    lib.ssm_proj.restype = ctypes.c_int
    lib.ssm_proj.argtypes = [vp, ctypes.c_int32, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp,
                             sz, vp]
    lib.ssm_conv_silu.restype = ctypes.c_int
    lib.ssm_conv_silu.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params), vp, vp, vp, vp]
    lib.ssm_conv_xproj.restype = ctypes.c_int
    lib.ssm_conv_xproj.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params), vp, vp, vp, ctypes.c_int64,
                                   vp, vp, vp, vp]
    lib.ssm_decode_fused_workspace_bytes.restype = sz
    lib.ssm_decode_fused_workspace_bytes.argtypes = [ctypes.POINTER(Dims), i64]
    lib.ssm_decode_fused.restype = ctypes.c_int
    lib.ssm_decode_fused.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params), vp, vp, i64] + [vp] * 5 + \
        [vp, sz, vp]
    lib.ssm_decode_fused_noalloc.restype = ctypes.c_int
    lib.ssm_decode_fused_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Params), vp, vp, i64] + \
        [vp] * 5 + [vp]
    lib.ssm_calib_issue.restype = ctypes.c_int
    lib.ssm_calib_issue.argtypes = [cint, i64, ctypes.c_int32, i64, vp, vp, vp]
    lib.ssm_calib_copy.restype = ctypes.c_int
    lib.ssm_calib_copy.argtypes = [vp, vp, sz, vp]
    lib.ssm_calib_read.restype = ctypes.c_int
    lib.ssm_calib_read.argtypes = [vp, sz, vp, vp]
    lib.ssm_calib_read_sink_floats.restype = sz
    lib.ssm_calib_read_sink_floats.argtypes = []
    if lib.ssm_abi_version() != ABI_VERSION:
        raise ImportError(f"libssm ABI {lib.ssm_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()  # ctypes passes the integer as a void*


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return SSM_F32
    if dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"io tensors must be float32 or bfloat16, got {dtype}")


def _check(t: Optional[torch.Tensor], name: str, shape, dtype, device, optional=False):
    """Shape, dtype, GPU device and contiguity of a tensor handed to the library (the cheap tests
    first; messages are built only on a mismatch)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.shape == shape and t.dtype == dtype and t.is_cuda and t.get_device() == device.index and t.is_contiguous():
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    raise ValueError(f"{name} must be a contiguous tensor on {device} (a GPU)")


def make_params(params: dict) -> Params:
    return Params(params["A"].data_ptr(), params["Dskip"].data_ptr(), params["dt_bias"].data_ptr(),
                  params["conv_w"].data_ptr(),
                  None if params.get("conv_b") is None else params["conv_b"].data_ptr())


def _check_params(params: dict, D: int, N: int, device):
    f32 = torch.float32
    _check(params["A"], "A", (D, N), f32, device)
    _check(params["Dskip"], "Dskip", (D,), f32, device)
    _check(params["dt_bias"], "dt_bias", (D,), f32, device)
    _check(params["conv_w"], "conv_w", (D, CONV_W), f32, device)
    _check(params.get("conv_b"), "conv_b", (D,), f32, device, optional=True)


def stream_handle(stream=None, device=None) -> int:
    """The HIP stream to enqueue on: `stream`, else the current stream of `device` (the
    tensors' device), so kernels run where the tensors live."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream  # ctypes passes the integer as a void*


def workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype=torch.bfloat16, chunk_hint=0) -> int:
    d = Dims(batch, seqlen, d_inner, d_state, CONV_W, _io_code(io_dtype), chunk_hint)
    return int(load().ssm_prefill_workspace_bytes(ctypes.byref(d)))


def prefill(x, dt, z, Bm, Cm, params: dict, h0=None, conv0=None, *, chunk_hint: int = 0,
            y=None, h_out=None, conv_out=None, workspace=None, stream=None):
    """ssm_prefill.  x, dt, z [B, D, L] and Bm, Cm [B, L, N] (io dtype, on the GPU); z may be
    None.  Returns (y, h_out, conv_out); outputs are allocated when not given."""
    lib = load()
    Bsz, D, L = x.shape
    N = params["A"].shape[1]
    dev, io = x.device, x.dtype
    for t, n in ((x, "x"), (dt, "dt"), (z, "z")):
        _check(t, n, (Bsz, D, L), io, dev, optional=(n == "z"))
    _check(Bm, "Bm", (Bsz, L, N), io, dev)
    _check(Cm, "Cm", (Bsz, L, N), io, dev)
    _check(h0, "h0", (Bsz, D, N), torch.float32, dev, optional=True)
    _check(conv0, "conv0", (Bsz, D, CONV_W - 1), torch.float32, dev, optional=True)
    _check_params(params, D, N, dev)
    y = torch.empty_like(x) if y is None else y
    h_out = torch.empty(Bsz, D, N, dtype=torch.float32, device=dev) if h_out is None else h_out
    conv_out = torch.empty(Bsz, D, CONV_W - 1, dtype=torch.float32, device=dev) if conv_out is None else conv_out
    _check(y, "y", (Bsz, D, L), io, dev)   # given outputs are written in full: their sizes must match
    _check(h_out, "h_out", (Bsz, D, N), torch.float32, dev)
    _check(conv_out, "conv_out", (Bsz, D, CONV_W - 1), torch.float32, dev)
    d = Dims(Bsz, L, D, N, CONV_W, _io_code(io), chunk_hint)
    need = int(lib.ssm_prefill_workspace_bytes(ctypes.byref(d)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p = make_params(params)
    st = lib.ssm_prefill(ctypes.byref(d), ctypes.byref(p), _ptr(x), _ptr(dt), _ptr(z), _ptr(Bm), _ptr(Cm),
                         _ptr(h0), _ptr(conv0), _ptr(y), _ptr(h_out), _ptr(conv_out), _ptr(workspace),
                         ws_bytes, stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_prefill", st, lib.ssm_status_str(st).decode())
    return y, h_out, conv_out


def decode_step(x_t, dt_t, z_t, B_t, C_t, params: dict, h, conv, *, y_t=None, stream=None):
    """ssm_decode_step: x_t, dt_t, z_t [B, D]; B_t, C_t [B, N]; h [B, D, N] and conv [B, D, 3]
    are updated in place.  Returns y_t [B, D]."""
    lib = load()
    Bsz, D = x_t.shape
    N = params["A"].shape[1]
    dev, io = x_t.device, x_t.dtype
    for t, n in ((x_t, "x_t"), (dt_t, "dt_t"), (z_t, "z_t")):
        _check(t, n, (Bsz, D), io, dev, optional=(n == "z_t"))
    _check(B_t, "B_t", (Bsz, N), io, dev)
    _check(C_t, "C_t", (Bsz, N), io, dev)
    _check(h, "h", (Bsz, D, N), torch.float32, dev)
    _check(conv, "conv", (Bsz, D, CONV_W - 1), torch.float32, dev)
    _check_params(params, D, N, dev)
    y_t = torch.empty_like(x_t) if y_t is None else y_t
    _check(y_t, "y_t", (Bsz, D), io, dev)
    d = Dims(Bsz, 1, D, N, CONV_W, _io_code(io), 0)
    p = make_params(params)
    st = lib.ssm_decode_step(ctypes.byref(d), ctypes.byref(p), _ptr(x_t), _ptr(dt_t), _ptr(z_t), _ptr(B_t),
                             _ptr(C_t), _ptr(y_t), _ptr(h), _ptr(conv), stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_decode_step", st, lib.ssm_status_str(st).decode())
    return y_t


def _check_index(t, name, B, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != (B,) or t.dtype != torch.int32 or not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape ({B},) on {device}")


def prefill_pool(x, dt, z, Bm, Cm, params: dict, slots, h_pool, conv_pool, *, seqlens=None, resume=False,
                 chunk_hint: int = 0, y=None, stream=None):
    """ssm_prefill_pool: rows write their final state into h_pool[slots[b]] / conv_pool[slots[b]]
    (resume=True starts from those entries); seqlens [B] int32 gives per-row lengths.  Returns y."""
    lib = load()
    Bsz, D, L = x.shape
    N = params["A"].shape[1]
    dev, io = x.device, x.dtype
    for t, n in ((x, "x"), (dt, "dt"), (z, "z")):
        _check(t, n, (Bsz, D, L), io, dev, optional=(n == "z"))
    _check(Bm, "Bm", (Bsz, L, N), io, dev)
    _check(Cm, "Cm", (Bsz, L, N), io, dev)
    _check_index(slots, "slots", Bsz, dev)
    _check_index(seqlens, "seqlens", Bsz, dev, optional=True)
    S = h_pool.shape[0]
    _check(h_pool, "h_pool", (S, D, N), torch.float32, dev)
    _check(conv_pool, "conv_pool", (S, D, CONV_W - 1), torch.float32, dev)
    _check_params(params, D, N, dev)
    y = torch.empty_like(x) if y is None else y
    _check(y, "y", (Bsz, D, L), io, dev)
    d = Dims(Bsz, L, D, N, CONV_W, _io_code(io), chunk_hint)
    p = make_params(params)
    st = lib.ssm_prefill_pool(ctypes.byref(d), ctypes.byref(p), _ptr(x), _ptr(dt), _ptr(z), _ptr(Bm), _ptr(Cm),
                              _ptr(seqlens), _ptr(slots), S, int(bool(resume)), _ptr(y), _ptr(h_pool),
                              _ptr(conv_pool), stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_prefill_pool", st, lib.ssm_status_str(st).decode())
    return y


def decode_step_pool(x_t, dt_t, z_t, B_t, C_t, params: dict, slots, h_pool, conv_pool, *, y_t=None, stream=None):
    """ssm_decode_step_pool: row b updates h_pool[slots[b]] / conv_pool[slots[b]] in place.  Returns y_t."""
    lib = load()
    Bsz, D = x_t.shape
    N = params["A"].shape[1]
    dev, io = x_t.device, x_t.dtype
    for t, n in ((x_t, "x_t"), (dt_t, "dt_t"), (z_t, "z_t")):
        _check(t, n, (Bsz, D), io, dev, optional=(n == "z_t"))
    _check(B_t, "B_t", (Bsz, N), io, dev)
    _check(C_t, "C_t", (Bsz, N), io, dev)
    _check_index(slots, "slots", Bsz, dev)
    S = h_pool.shape[0]
    _check(h_pool, "h_pool", (S, D, N), torch.float32, dev)
    _check(conv_pool, "conv_pool", (S, D, CONV_W - 1), torch.float32, dev)
    _check_params(params, D, N, dev)
    y_t = torch.empty_like(x_t) if y_t is None else y_t
    _check(y_t, "y_t", (Bsz, D), io, dev)
    d = Dims(Bsz, 1, D, N, CONV_W, _io_code(io), 0)
    p = make_params(params)
    st = lib.ssm_decode_step_pool(ctypes.byref(d), ctypes.byref(p), _ptr(x_t), _ptr(dt_t), _ptr(z_t), _ptr(B_t),
                                  _ptr(C_t), _ptr(slots), S, _ptr(y_t), _ptr(h_pool), _ptr(conv_pool),
                                  stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_decode_step_pool", st, lib.ssm_status_str(st).decode())
    return y_t


# ---- block int8 codec of include/ssm_codec.h ----

Q8_MAX_PARTS = 16


def q8_num_blocks(n: int, block: int) -> int:
    """Scales per tensor of n elements: ceil(n / block) (0 for invalid arguments)."""
    return int(load().ssm_q8_num_blocks(n, block))


def q8_quantize(x, block: int = 128, *, q=None, scales=None, stream=None):
    """x (any shape, contiguous, float32 or bfloat16, on the GPU) -> (q int8 [x.numel()],
    scales float32 [ceil(numel / block)])."""
    lib = load()
    if x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    n = x.numel()
    nb = q8_num_blocks(n, block)
    if q is None:
        q = torch.empty(n, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(max(nb, 1), dtype=torch.float32, device=x.device)
    _check(q, "q", (n,), torch.int8, x.device)
    _check(scales, "scales", (max(nb, 1),), torch.float32, x.device)
    st = lib.ssm_q8_quantize(n, block, _io_code(x.dtype), _ptr(x), _ptr(q), _ptr(scales),
                             stream_handle(stream, x.device))
    if st != 0:
        raise SsmError("ssm_q8_quantize", st, lib.ssm_status_str(st).decode())
    return q, scales


def q8_dequant_sum(q_parts, scale_parts, block: int = 128, dtype=torch.bfloat16, *, y=None, stream=None):
    """Sum of the dequantized parts: y[i] = sum_p q_parts[p][i] * scale_parts[p][i // block]."""
    lib = load()
    parts = len(q_parts)
    if parts != len(scale_parts) or parts < 1:
        raise ValueError("q_parts and scale_parts must be non-empty lists of equal length")
    n = q_parts[0].numel()
    dev = q_parts[0].device
    nb = q8_num_blocks(n, block)
    for i in range(parts):
        _check(q_parts[i], f"q_parts[{i}]", (n,), torch.int8, dev)
        _check(scale_parts[i], f"scale_parts[{i}]", (max(nb, 1),), torch.float32, dev)
    if y is None:
        y = torch.empty(n, dtype=dtype, device=dev)
    _check(y, "y", (n,), dtype, dev)
    qa = (ctypes.c_void_p * parts)(*[t.data_ptr() for t in q_parts])
    sa = (ctypes.c_void_p * parts)(*[t.data_ptr() for t in scale_parts])
    st = lib.ssm_q8_dequant_sum(n, block, _io_code(dtype), parts, qa, sa, _ptr(y), stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_q8_dequant_sum", st, lib.ssm_status_str(st).decode())
    return y


# ---- channel-sliced projections and the conv front of include/ssm_proj.h ----

PROJ_IN, PROJ_X, PROJ_DT, PROJ_OUT = 0, 1, 2, 3


class Projector:
    """A projection context (hipBLASLt handle + per-shape algorithm cache) with its device
    workspace.  Layouts: IN / DT map token-major in [B, L, K] to channel-major out [B, M, L];
    X / OUT map channel-major in [B, K, L] to token-major out [B, L, M]; W is [M, K]."""

    def __init__(self, device="cuda"):
        self.lib = load()
        h = ctypes.c_void_p()
        st = self.lib.ssm_proj_create(ctypes.byref(h))
        if st != 0:
            raise SsmError("ssm_proj_create", st, self.lib.ssm_status_str(st).decode())
        self.handle = h
        self.ws_bytes = int(self.lib.ssm_proj_workspace_bytes())
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def close(self):
        if self.handle is not None and self.handle.value:
            self.lib.ssm_proj_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __call__(self, kind: int, x, w, *, out=None, out_dtype=None, stream=None):
        lib = self.lib
        if kind not in (PROJ_IN, PROJ_X, PROJ_DT, PROJ_OUT):
            raise ValueError(f"unknown projection kind {kind}")
        M, K = w.shape
        token_major_in = kind in (PROJ_IN, PROJ_DT)
        if token_major_in:
            Bn, L, K2 = x.shape
        else:
            Bn, K2, L = x.shape
        if K2 != K:
            raise ValueError(f"in_features mismatch: input has {K2}, weight has {K}")
        if out_dtype is None:
            out_dtype = x.dtype if out is None else out.dtype
        shape = (Bn, M, L) if token_major_in else (Bn, L, M)
        if out is None:
            out = torch.empty(shape, dtype=out_dtype, device=x.device)
        _check(x, "x", tuple(x.shape), x.dtype, x.device)
        _check(w, "w", (M, K), x.dtype, x.device)
        _check(out, "out", shape, out_dtype, x.device)
        st = lib.ssm_proj(self.handle, kind, Bn, L, K, M, _io_code(x.dtype), _io_code(out_dtype), _ptr(x), _ptr(w),
                          _ptr(out), _ptr(self.ws), self.ws_bytes, stream_handle(stream, x.device))
        if st != 0:
            raise SsmError("ssm_proj", st, lib.ssm_status_str(st).decode())
        return out


def conv_silu(x, params: dict, conv0=None, *, u=None, stream=None):
    """u = silu(conv(x)) for x [B, D, L] (the scan's front end, materialised)."""
    lib = load()
    Bn, D, L = x.shape
    if u is None:
        u = torch.empty_like(x)
    _check(u, "u", (Bn, D, L), x.dtype, x.device)
    _check(conv0, "conv0", (Bn, D, CONV_W - 1), torch.float32, x.device, optional=True)
    d = Dims(Bn, L, D, 1, CONV_W, _io_code(x.dtype), 0)
    p = Params(None, None, None, params["conv_w"].data_ptr(),
               None if params.get("conv_b") is None else params["conv_b"].data_ptr())
    st = lib.ssm_conv_silu(ctypes.byref(d), ctypes.byref(p), _ptr(x), _ptr(conv0), _ptr(u),
                           stream_handle(stream, x.device))
    if st != 0:
        raise SsmError("ssm_conv_silu", st, lib.ssm_status_str(st).decode())
    return u


def conv_xproj(x, params: dict, w, rank: int, conv0=None, *, lowrank=None, Bm=None, Cm=None, stream=None):
    """The conv front fused into x_proj: for x [B, D, L] bf16 and the stacked x_proj rows
    w [rank + 2 N, D], returns (lowrank [B, L, rank], Bm [B, L, N], Cm [B, L, N]) of
    x_proj(silu(conv(x)))."""
    lib = load()
    Bn, D, L = x.shape
    M = w.shape[0]
    N = (M - rank) // 2
    if w.dim() != 2 or w.shape[1] != D or rank < 1 or N < 1 or rank + 2 * N != M:
        raise ValueError(f"w must be [rank + 2 N, {D}] with rank={rank}; got {tuple(w.shape)}")
    _check(w, "w", (M, D), x.dtype, x.device)
    _check(conv0, "conv0", (Bn, D, CONV_W - 1), torch.float32, x.device, optional=True)
    outs = []
    for t, name, width in ((lowrank, "lowrank", rank), (Bm, "Bm", N), (Cm, "Cm", N)):
        if t is None:
            t = torch.empty(Bn, L, width, dtype=x.dtype, device=x.device)
        _check(t, name, (Bn, L, width), x.dtype, x.device)
        outs.append(t)
    d = Dims(Bn, L, D, N, CONV_W, _io_code(x.dtype), 0)
    p = Params(None, None, None, params["conv_w"].data_ptr(),
               None if params.get("conv_b") is None else params["conv_b"].data_ptr())
    st = lib.ssm_conv_xproj(ctypes.byref(d), ctypes.byref(p), _ptr(x), _ptr(conv0), _ptr(w), rank,
                            _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), stream_handle(stream, x.device))
    if st != 0:
        raise SsmError("ssm_conv_xproj", st, lib.ssm_status_str(st).decode())
    return tuple(outs)


# ---- the fused per-token layer stages (include/ssm_layer.h) ----

def decode_fused_workspace_bytes(batch: int, d_inner: int, rank: int, d_state: int = 16,
                                 io_dtype=torch.bfloat16) -> int:
    d = Dims(batch, 1, d_inner, d_state, CONV_W, _io_code(io_dtype), 0)
    return int(load().ssm_decode_fused_workspace_bytes(ctypes.byref(d), rank))


def decode_fused(x_t, z_t, params: dict, w_x, w_dt, rank: int, h, conv, *, y_t=None, workspace=None, stream=None):
    """ssm_decode_fused: x_t, z_t [B, D] (z_t may be None), w_x [rank + 2N, D], w_dt [D, rank];
    h [B, D, N] and conv [B, D, 3] are updated in place.  Returns y_t [B, D]."""
    lib = load()
    Bsz, D = x_t.shape
    N = params["A"].shape[1]
    dev, io = x_t.device, x_t.dtype
    _check(x_t, "x_t", (Bsz, D), io, dev)
    _check(z_t, "z_t", (Bsz, D), io, dev, optional=True)
    _check(w_x, "w_x", (rank + 2 * N, D), io, dev)
    _check(w_dt, "w_dt", (D, rank), io, dev)
    _check(h, "h", (Bsz, D, N), torch.float32, dev)
    _check(conv, "conv", (Bsz, D, CONV_W - 1), torch.float32, dev)
    _check_params(params, D, N, dev)
    y_t = torch.empty_like(x_t) if y_t is None else y_t
    _check(y_t, "y_t", (Bsz, D), io, dev)
    d = Dims(Bsz, 1, D, N, CONV_W, _io_code(io), 0)
    need = int(lib.ssm_decode_fused_workspace_bytes(ctypes.byref(d), rank))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    p = make_params(params)
    st = lib.ssm_decode_fused(ctypes.byref(d), ctypes.byref(p), _ptr(w_x), _ptr(w_dt), rank, _ptr(x_t), _ptr(z_t),
                              _ptr(y_t), _ptr(h), _ptr(conv), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_decode_fused", st, lib.ssm_status_str(st).decode())
    return y_t


def decode_fused_noalloc(x_t, z_t, params: dict, w_x, w_dt, rank: int, h, conv, *, y_t=None, stream=None):
    """ssm_decode_fused_noalloc: as decode_fused, with the library's fixed per-GPU scratch instead
    of a workspace (nothing is allocated; y_t must be given for no allocation at all)."""
    lib = load()
    Bsz, D = x_t.shape
    N = params["A"].shape[1]
    dev, io = x_t.device, x_t.dtype
    _check(x_t, "x_t", (Bsz, D), io, dev)
    _check(z_t, "z_t", (Bsz, D), io, dev, optional=True)
    _check(w_x, "w_x", (rank + 2 * N, D), io, dev)
    _check(w_dt, "w_dt", (D, rank), io, dev)
    _check(h, "h", (Bsz, D, N), torch.float32, dev)
    _check(conv, "conv", (Bsz, D, CONV_W - 1), torch.float32, dev)
    _check_params(params, D, N, dev)
    y_t = torch.empty_like(x_t) if y_t is None else y_t
    _check(y_t, "y_t", (Bsz, D), io, dev)
    d = Dims(Bsz, 1, D, N, CONV_W, _io_code(io), 0)
    p = make_params(params)
    st = lib.ssm_decode_fused_noalloc(ctypes.byref(d), ctypes.byref(p), _ptr(w_x), _ptr(w_dt), rank, _ptr(x_t),
                                      _ptr(z_t), _ptr(y_t), _ptr(h), _ptr(conv), stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_decode_fused_noalloc", st, lib.ssm_status_str(st).decode())
    return y_t


# ---- rate calibration (include/ssm_calib.h) ----

CALIB_KINDS = {"fma": 0, "exp": 1, "mix": 2, "mul": 3, "fmac": 4, "fma3": 5, "dpp": 6, "split": 7, "mixi": 8}
CALIB_STAMP_WORDS = 8
CALIB_THREADS = 256


def calib_issue(kind: int, workgroups: int, iters: int, split: int = 0, *, device="cuda", stream=None):
    """ssm_calib_issue: returns (stamps [waves, 8] int64 on the device, sink); run on `stream`."""
    lib = load()
    dev = torch.device(device)
    stamps = torch.zeros(workgroups * 4, CALIB_STAMP_WORDS, dtype=torch.int64, device=dev)
    sink = torch.empty(workgroups * CALIB_THREADS, dtype=torch.float32, device=dev)
    st = lib.ssm_calib_issue(kind, workgroups, iters, split, _ptr(stamps), _ptr(sink), stream_handle(stream, dev))
    if st != 0:
        raise SsmError("ssm_calib_issue", st, lib.ssm_status_str(st).decode())
    return stamps, sink


def calib_copy(src, dst, *, stream=None):
    """ssm_calib_copy of src's bytes into dst (same byte count, both contiguous on the GPU)."""
    lib = load()
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_cuda and dst.is_cuda and src.is_contiguous()
                                                     and dst.is_contiguous()):
        raise ValueError("calib_copy: contiguous GPU tensors of the same byte count expected")
    st = lib.ssm_calib_copy(_ptr(src), _ptr(dst), n, stream_handle(stream, src.device))
    if st != 0:
        raise SsmError("ssm_calib_copy", st, lib.ssm_status_str(st).decode())


def calib_read(src, sink=None, *, stream=None):
    """ssm_calib_read of src's bytes; returns the sink tensor."""
    lib = load()
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("calib_read: a contiguous GPU tensor expected")
    nsink = int(lib.ssm_calib_read_sink_floats())
    sink = torch.empty(nsink, dtype=torch.float32, device=src.device) if sink is None else sink
    if sink.numel() < nsink or sink.dtype != torch.float32:
        raise ValueError(f"calib_read: sink must hold {nsink} float32")
    st = lib.ssm_calib_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), stream_handle(stream, src.device))
    if st != 0:
        raise SsmError("ssm_calib_read", st, lib.ssm_status_str(st).decode())
    return sink
