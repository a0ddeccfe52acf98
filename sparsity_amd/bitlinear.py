"""ctypes binding of libbitlinear (argument marshalling only; every step runs in HIP kernels).

Names mirror the C ABI: ``bitlinear_packed_bytes``, ``bitlinear_pack``, ``bitlinear_pack_noalloc``,
``act_quant_i8``,
``bitlinear_fwd``, ``bitlinear_group_table_bytes``, ``bitlinear_group_build``,
``bitlinear_fwd_group``, ``bitlinear_group_fused_table_bytes``, ``bitlinear_group_fused_build``,
``bitlinear_fwd_group_fused``, ``bitlinear_bwd_workspace_bytes``, ``bitlinear_bwd``,
``bitlinear_bwd_group_plan``, ``bitlinear_bwd_group_build``, ``bitlinear_bwd_group``,
``bitlinear_pack_group_plan``, ``bitlinear_pack_group_build``, ``bitlinear_pack_group``,
``bitlinear_transcode6``, the chain and prefill-group calls.
``pack`` / ``PackGroup`` / ``act_quant`` / ``fwd`` / ``transcode6`` / ``FwdGroup`` / ``FusedGroup``
/ ``bwd`` / ``BwdGroup`` are convenience
wrappers that allocate the output tensors with torch on the input's device and enqueue on torch's
current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

BL_OK = 0
BL_LAYOUT_SPARSE = 0
BL_LAYOUT_DENSE2 = 1
BL_LAYOUT_SPARSE6 = 2
BL_DTYPE_F32 = 0
BL_DTYPE_BF16 = 1
BL_BWD_ACCUM_DX = 1
BL_BWD_ACCUM_DW = 2



class BlFwdDesc(ctypes.Structure):
    """bl_fwd_desc: the arguments of one bitlinear_fwd call inside a group."""
    _fields_ = [("xq", ctypes.c_void_p), ("x_scale", ctypes.c_void_p), ("T", ctypes.c_int64),
                ("K", ctypes.c_int64), ("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("gamma", ctypes.c_void_p), ("n", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("acc_opt", ctypes.c_void_p)]


class BlFwdXDesc(ctypes.Structure):
    """bl_fwd_x_desc: one projection of a fused group (bf16 activations, quantized in-kernel)."""
    _fields_ = [("x", ctypes.c_void_p), ("T", ctypes.c_int64), ("K", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("y", ctypes.c_void_p), ("acc_opt", ctypes.c_void_p)]


class BlBwdDesc(ctypes.Structure):
    """bl_bwd_desc: the arguments of one bitlinear_bwd call inside a grouped backward."""
    _fields_ = [("dy", ctypes.c_void_p), ("xq", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("K", ctypes.c_int64), ("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("gamma", ctypes.c_void_p), ("n", ctypes.c_int64), ("dx", ctypes.c_void_p),
                ("dw", ctypes.c_void_p), ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class BlBwdGroupPlan(ctypes.Structure):
    """bl_bwd_group_plan: table and workspace sizes and the two launch grids of a group."""
    _fields_ = [("table_bytes", ctypes.c_size_t), ("ws_bytes", ctypes.c_size_t),
                ("prep_blocks", ctypes.c_int64), ("jobs", ctypes.c_int64),
                ("N", ctypes.c_int32), ("M", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class BlPackDesc(ctypes.Structure):
    """bl_pack_desc: the arguments of one bitlinear_pack call inside a grouped pack."""
    _fields_ = [("W", ctypes.c_void_p), ("n", ctypes.c_int64), ("K", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("gamma", ctypes.c_void_p)]


class BlPackGroupPlan(ctypes.Structure):
    """bl_pack_group_plan: table and workspace sizes and the pack launch's grid."""
    _fields_ = [("table_bytes", ctypes.c_size_t), ("ws_bytes", ctypes.c_size_t),
                ("count", ctypes.c_int64), ("pack_blocks", ctypes.c_int64),
                ("N", ctypes.c_int32), ("M", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class BlQuantDesc(ctypes.Structure):
    """bl_quant_desc: the arguments of one act_quant_i8 call inside a grouped quantization."""
    _fields_ = [("x", ctypes.c_void_p), ("T", ctypes.c_int64), ("K", ctypes.c_int64),
                ("xq", ctypes.c_void_p), ("x_scale", ctypes.c_void_p)]


class BlGemmGroupPlan(ctypes.Structure):
    """bl_gemm_group_plan: table size and the grid of a grouped prefill forward."""
    _fields_ = [("table_bytes", ctypes.c_size_t), ("jobs", ctypes.c_int64),
                ("N", ctypes.c_int32), ("M", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class BlChainLayer(ctypes.Structure):
    """bl_chain_layer: one layer of a fused decode chain (its input is the previous layer's y)."""
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("K", ctypes.c_int64), ("y", ctypes.c_void_p),
                ("acc_opt", ctypes.c_void_p)]


class BlChainPlan(ctypes.Structure):
    """bl_chain_plan: table and workspace sizes and the launch's LDS bytes of a chain."""
    _fields_ = [("table_bytes", ctypes.c_size_t), ("ws_bytes", ctypes.c_size_t),
                ("L", ctypes.c_int64), ("T", ctypes.c_int64), ("smem", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")
_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = lib().bitlinear_strerror(status).decode()
        super().__init__(f"{call} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libbitlinear.so (built by ``sparsity_amd.build``); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparsity_amd.build` "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.bitlinear_packed_bytes.argtypes = [i64, i64, i32, i32, i32, ctypes.POINTER(sz),
                                             ctypes.POINTER(sz), ctypes.POINTER(i64), ctypes.POINTER(sz)]
        L.bitlinear_pack.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.bitlinear_pack_noalloc.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
        L.act_quant_i8.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp]
        L.act_quant_i8_group.argtypes = [ctypes.POINTER(BlQuantDesc), i64, i32, i32, vp]
        L.bitlinear_fwd.argtypes = [vp, vp, i64, i64, vp, vp, vp, i32, i32, i32, i64, vp, vp, vp]
        L.bitlinear_transcode6.argtypes = [vp, vp, i64, i64, vp, vp]
        dp = ctypes.POINTER(BlFwdDesc)
        L.bitlinear_group_table_bytes.argtypes = [dp, i64, i32, i32, i32, ctypes.POINTER(sz),
                                                  ctypes.POINTER(i64)]
        L.bitlinear_group_build.argtypes = [dp, i64, i32, i32, i32, vp, sz, vp]
        L.bitlinear_fwd_group.argtypes = [vp, i64, i32, i32, i32, vp]
        xp = ctypes.POINTER(BlFwdXDesc)
        L.bitlinear_group_fused_table_bytes.argtypes = [xp, i64, i32, i32, i32,
                                                        ctypes.POINTER(sz), ctypes.POINTER(i64)]
        L.bitlinear_group_fused_build.argtypes = [xp, i64, i32, i32, i32, vp, sz, vp]
        L.bitlinear_fwd_group_fused.argtypes = [vp, i64, i32, i32, i32, vp]
        L.bitlinear_bwd_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
        L.bitlinear_bwd.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp, vp, i32, i32, i32, vp, vp,
                                    i32, vp, sz, vp]
        bp = ctypes.POINTER(BlBwdDesc)
        pp = ctypes.POINTER(BlBwdGroupPlan)
        L.bitlinear_bwd_group_plan.argtypes = [bp, i64, i64, i32, i32, i32, pp]
        L.bitlinear_bwd_group_build.argtypes = [bp, i64, i64, i32, i32, i32, vp, sz, vp, sz, vp]
        L.bitlinear_bwd_group.argtypes = [vp, pp, vp]
        kp = ctypes.POINTER(BlPackDesc)
        kpp = ctypes.POINTER(BlPackGroupPlan)
        L.bitlinear_pack_group_plan.argtypes = [kp, i64, i32, i32, i32, kpp]
        L.bitlinear_pack_group_build.argtypes = [kp, i64, i32, i32, i32, vp, sz, vp, sz, vp]
        L.bitlinear_pack_group.argtypes = [vp, kpp, vp]
        gp = ctypes.POINTER(BlGemmGroupPlan)
        L.bitlinear_gemm_group_plan.argtypes = [dp, i64, i32, i32, i32, gp]
        L.bitlinear_gemm_group_build.argtypes = [dp, i64, i32, i32, i32, vp, sz, vp]
        L.bitlinear_gemm_group.argtypes = [vp, gp, vp]
        cl = ctypes.POINTER(BlChainLayer)
        cpp = ctypes.POINTER(BlChainPlan)
        L.bitlinear_chain_plan.argtypes = [cl, i64, i64, i32, i32, i32, cpp]
        L.bitlinear_chain_build.argtypes = [cl, i64, i64, i32, i32, i32, vp, sz, vp]
        L.bitlinear_fwd_chain.argtypes = [vp, cpp, vp, i32, vp, sz, i64, vp]
        L.bitlinear_strerror.argtypes = [i32]
        L.bitlinear_strerror.restype = ctypes.c_char_p
        L.bitlinear_layout_version.argtypes = []
        for f in (L.bitlinear_packed_bytes, L.bitlinear_pack, L.bitlinear_pack_noalloc,
                  L.act_quant_i8, L.bitlinear_fwd,
                  L.bitlinear_layout_version, L.bitlinear_group_table_bytes,
                  L.bitlinear_group_build, L.bitlinear_fwd_group,
                  L.bitlinear_bwd_workspace_bytes, L.bitlinear_bwd,
                  L.bitlinear_group_fused_table_bytes, L.bitlinear_group_fused_build,
                  L.bitlinear_fwd_group_fused, L.bitlinear_bwd_group_plan,
                  L.bitlinear_bwd_group_build, L.bitlinear_bwd_group,
                  L.bitlinear_pack_group_plan, L.bitlinear_pack_group_build,
                  L.bitlinear_pack_group, L.bitlinear_gemm_group_plan,
                  L.bitlinear_gemm_group_build, L.bitlinear_gemm_group,
                  L.act_quant_i8_group, L.bitlinear_chain_plan, L.bitlinear_chain_build,
                  L.bitlinear_fwd_chain):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, call: str) -> None:
    if status != BL_OK:
        raise BitLinearError(status, call)


# ---------------------------------------------------------------------------------------------
# raw C ABI (integers and pointers)
# ---------------------------------------------------------------------------------------------

def bitlinear_packed_bytes(n: int, K: int, N: int, M: int, layout: int):
    """Returns (status, codes_bytes, meta_bytes, K_eff, ws_bytes)."""
    cb, mb, ws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    ke = ctypes.c_int64()
    st = lib().bitlinear_packed_bytes(n, K, N, M, layout, ctypes.byref(cb), ctypes.byref(mb),
                                      ctypes.byref(ke), ctypes.byref(ws))
    return st, cb.value, mb.value, ke.value, ws.value


def bitlinear_pack(W, n, K, N, M, layout, codes, meta, gamma, ws, ws_bytes, stream) -> int:
    return lib().bitlinear_pack(W, n, K, N, M, layout, codes, meta, gamma, ws, ws_bytes, stream)


def bitlinear_pack_noalloc(W, n, K, N, M, layout, codes, meta, gamma, stream) -> int:
    return lib().bitlinear_pack_noalloc(W, n, K, N, M, layout, codes, meta, gamma, stream)


def act_quant_i8(x, x_dtype, T, K, lift_M, xq, x_scale, stream) -> int:
    return lib().act_quant_i8(x, x_dtype, T, K, lift_M, xq, x_scale, stream)


def act_quant_i8_group(descs, x_dtype, lift_M, stream) -> int:
    """descs: a ctypes array of BlQuantDesc."""
    return lib().act_quant_i8_group(descs, len(descs), x_dtype, lift_M, stream)


def bitlinear_fwd(xq, x_scale, T, K, codes, meta, gamma, N, M, layout, n, y, acc, stream) -> int:
    return lib().bitlinear_fwd(xq, x_scale, T, K, codes, meta, gamma, N, M, layout, n, y, acc, stream)


def bitlinear_transcode6(codes, meta, n, K, out, stream) -> int:
    return lib().bitlinear_transcode6(codes, meta, n, K, out, stream)


def bitlinear_group_table_bytes(descs, N, M, layout):
    """descs: a ctypes array of BlFwdDesc.  Returns (status, table_bytes, work_items)."""
    tb, wi = ctypes.c_size_t(), ctypes.c_int64()
    st = lib().bitlinear_group_table_bytes(descs, len(descs), N, M, layout, ctypes.byref(tb),
                                           ctypes.byref(wi))
    return st, tb.value, wi.value


def bitlinear_group_build(descs, N, M, layout, table, table_bytes, stream) -> int:
    return lib().bitlinear_group_build(descs, len(descs), N, M, layout, table, table_bytes, stream)


def bitlinear_fwd_group(table, work_items, N, M, layout, stream) -> int:
    return lib().bitlinear_fwd_group(table, work_items, N, M, layout, stream)


def bitlinear_group_fused_table_bytes(descs, N, M, layout):
    """descs: a ctypes array of BlFwdXDesc.  Returns (status, table_bytes, work_items)."""
    tb, wi = ctypes.c_size_t(), ctypes.c_int64()
    st = lib().bitlinear_group_fused_table_bytes(descs, len(descs), N, M, layout,
                                                 ctypes.byref(tb), ctypes.byref(wi))
    return st, tb.value, wi.value


def bitlinear_group_fused_build(descs, N, M, layout, table, table_bytes, stream) -> int:
    return lib().bitlinear_group_fused_build(descs, len(descs), N, M, layout, table, table_bytes,
                                             stream)


def bitlinear_fwd_group_fused(table, work_items, N, M, layout, stream) -> int:
    return lib().bitlinear_fwd_group_fused(table, work_items, N, M, layout, stream)


def bitlinear_bwd_workspace_bytes(T, n, K):
    """Returns (status, ws_bytes)."""
    ws = ctypes.c_size_t()
    st = lib().bitlinear_bwd_workspace_bytes(T, n, K, ctypes.byref(ws))
    return st, ws.value


def bitlinear_bwd(dy, T, n, xq, x_scale, K, codes, meta, gamma, N, M, layout, dx, dw, flags, ws,
                  ws_bytes, stream) -> int:
    return lib().bitlinear_bwd(dy, T, n, xq, x_scale, K, codes, meta, gamma, N, M, layout, dx, dw,
                               flags, ws, ws_bytes, stream)


def bitlinear_pack_group_plan(descs, N, M, layout):
    """Returns (status, BlPackGroupPlan)."""
    plan = BlPackGroupPlan()
    st = lib().bitlinear_pack_group_plan(descs, len(descs), N, M, layout, ctypes.byref(plan))
    return st, plan


def bitlinear_pack_group_build(descs, N, M, layout, ws, ws_bytes, table, table_bytes, stream) -> int:
    return lib().bitlinear_pack_group_build(descs, len(descs), N, M, layout, ws, ws_bytes, table,
                                            table_bytes, stream)


def bitlinear_pack_group(table, plan, stream) -> int:
    return lib().bitlinear_pack_group(table, ctypes.byref(plan) if plan is not None else None,
                                      stream)


def bitlinear_bwd_group_plan(descs, T, N, M, layout):
    """Returns (status, BlBwdGroupPlan)."""
    plan = BlBwdGroupPlan()
    st = lib().bitlinear_bwd_group_plan(descs, len(descs), T, N, M, layout, ctypes.byref(plan))
    return st, plan


def bitlinear_bwd_group_build(descs, T, N, M, layout, ws, ws_bytes, table, table_bytes,
                              stream) -> int:
    return lib().bitlinear_bwd_group_build(descs, len(descs), T, N, M, layout, ws, ws_bytes, table,
                                           table_bytes, stream)


def bitlinear_bwd_group(table, plan, stream) -> int:
    return lib().bitlinear_bwd_group(table, ctypes.byref(plan) if plan is not None else None,
                                     stream)


def bitlinear_gemm_group_plan(descs, N, M, layout):
    """Returns (status, BlGemmGroupPlan)."""
    plan = BlGemmGroupPlan()
    st = lib().bitlinear_gemm_group_plan(descs, len(descs), N, M, layout, ctypes.byref(plan))
    return st, plan


def bitlinear_gemm_group_build(descs, N, M, layout, table, table_bytes, stream) -> int:
    return lib().bitlinear_gemm_group_build(descs, len(descs), N, M, layout, table, table_bytes,
                                            stream)


def bitlinear_gemm_group(table, plan, stream) -> int:
    return lib().bitlinear_gemm_group(table, ctypes.byref(plan) if plan is not None else None,
                                      stream)


def bitlinear_chain_plan(layers, T, N, M, layout):
    """layers: a ctypes array of BlChainLayer.  Returns (status, BlChainPlan)."""
    plan = BlChainPlan()
    st = lib().bitlinear_chain_plan(layers, len(layers), T, N, M, layout, ctypes.byref(plan))
    return st, plan


def bitlinear_chain_build(layers, T, N, M, layout, table, table_bytes, stream) -> int:
    return lib().bitlinear_chain_build(layers, len(layers), T, N, M, layout, table, table_bytes,
                                       stream)


def bitlinear_fwd_chain(table, plan, x0, x_dtype, ws, ws_bytes, spin_limit, stream) -> int:
    return lib().bitlinear_fwd_chain(table, ctypes.byref(plan) if plan is not None else None, x0,
                                     x_dtype, ws, ws_bytes, spin_limit, stream)


# ---------------------------------------------------------------------------------------------
# torch convenience wrappers
# ---------------------------------------------------------------------------------------------

def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, dtype, numel: int, device, name: str) -> None:
    """Raise unless t is a contiguous CUDA tensor of `dtype` on `device` with at least `numel`
    elements: the C ABI receives bare pointers and cannot check sizes, so a short or foreign
    buffer would be read or written out of bounds by the kernels."""
    if t is None:
        raise ValueError(f"{name}: buffer missing")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name}: must be a CUDA tensor on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, got {t.numel()}")


def packed_bytes(n: int, K: int, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE):
    st, cb, mb, ke, ws = bitlinear_packed_bytes(n, K, N, M, layout)
    _check(st, "bitlinear_packed_bytes")
    return cb, mb, ke, ws


def pack(W, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE, out=None, ws=None):
    """Mask + ternarize + pack a contiguous fp32 CUDA tensor W[n][K].

    Returns (codes uint8, meta uint8 or None, gamma fp32[1]) on W's device.  ``out`` may supply
    preallocated (codes, meta, gamma); ``ws`` a uint8 workspace.
    """
    import torch
    assert W.is_cuda and W.dtype == torch.float32 and W.is_contiguous() and W.dim() == 2
    n, K = W.shape
    cb, mb, _, wsb = packed_bytes(n, K, N, M, layout)
    if out is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=W.device)
        meta = torch.empty(mb, dtype=torch.uint8, device=W.device) if mb else None
        gamma = torch.empty(4, dtype=torch.float32, device=W.device)[:1]
    else:
        codes, meta, gamma = out
    if ws is None:
        ws = torch.empty(wsb, dtype=torch.uint8, device=W.device)
    _need(codes, torch.uint8, cb, W.device, "codes")
    if mb:
        _need(meta, torch.uint8, mb, W.device, "meta")
    elif meta is not None:
        raise ValueError("meta: must be None for the dense 2-bit layout")
    _need(gamma, torch.float32, 1, W.device, "gamma")
    _need(ws, torch.uint8, wsb, W.device, "ws")
    _check(bitlinear_pack(W.data_ptr(), n, K, N, M, layout, codes.data_ptr(), _ptr(meta),
                          gamma.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "bitlinear_pack")
    return codes, meta, gamma


def act_quant(x, lift_M: int = 0, out=None):
    """Per-token int8 quantization of a contiguous fp32/bf16 CUDA tensor x[T][K].

    Returns (xq int8 [T][K_eff], scale fp32 [T]).
    """
    import torch
    assert x.is_cuda and x.is_contiguous() and x.dim() == 2
    T, K = x.shape
    dt = {torch.float32: BL_DTYPE_F32, torch.bfloat16: BL_DTYPE_BF16}[x.dtype]
    ke = K // lift_M * (2 * lift_M - 4) if lift_M else K
    if out is None:
        xq = torch.empty((T, ke), dtype=torch.int8, device=x.device)
        scale = torch.empty(max(T, 4), dtype=torch.float32, device=x.device)[:T]
    else:
        xq, scale = out
    _need(xq, torch.int8, T * ke, x.device, "xq")
    _need(scale, torch.float32, T, x.device, "scale")
    _check(act_quant_i8(x.data_ptr(), dt, T, K, lift_M, xq.data_ptr(), scale.data_ptr(), _stream()),
           "act_quant_i8")
    return xq, scale


def act_quant_group(xs, lift_M: int = 0, outs=None):
    """act_quant of several contiguous CUDA tensors x[T][K] (one dtype) in one launch.

    Returns a list of (xq, scale), equal to ``act_quant`` per tensor bit for bit; ``outs``, if
    given, is a list of (xq, scale) buffers to write.
    """
    import torch
    dts = {torch.float32: BL_DTYPE_F32, torch.bfloat16: BL_DTYPE_BF16}
    dt = dts[xs[0].dtype]
    arr = (BlQuantDesc * len(xs))()
    res = []
    for i, x in enumerate(xs):
        assert x.is_cuda and x.is_contiguous() and x.dim() == 2 and dts[x.dtype] == dt
        T, K = x.shape
        ke = K // lift_M * (2 * lift_M - 4) if lift_M else K
        if outs is None:
            xq = torch.empty((T, ke), dtype=torch.int8, device=x.device)
            scale = torch.empty(max(T, 4), dtype=torch.float32, device=x.device)[:T]
        else:
            xq, scale = outs[i]
            _need(xq, torch.int8, T * ke, x.device, f"outs[{i}] xq")
            _need(scale, torch.float32, T, x.device, f"outs[{i}] scale")
        res.append((xq, scale))
        arr[i] = BlQuantDesc(_ptr(x), T, K, _ptr(xq), _ptr(scale))
    _check(act_quant_i8_group(arr, dt, lift_M, _stream()), "act_quant_i8_group")
    return res


def fwd(xq, scale, K: int, codes, meta, gamma, n: int, N: int = 2, M: int = 4,
        layout: int = BL_LAYOUT_SPARSE, want_acc: bool = False, out=None):
    """y[T][n] fp32 from int8 activations and packed weights; optionally also int32 acc."""
    import torch
    T = xq.shape[0]
    cb, mb, ke, _ = packed_bytes(n, K, N, M, layout)
    dev = xq.device
    if xq.dim() != 2 or xq.shape[1] != ke:
        raise ValueError(f"xq: must be [T][{ke}] (the packed K axis of K = {K}), got {tuple(xq.shape)}")
    _need(xq, torch.int8, T * ke, dev, "xq")
    _need(scale, torch.float32, T, dev, "scale")
    _need(codes, torch.uint8, cb, dev, "codes")
    if mb:
        _need(meta, torch.uint8, mb, dev, "meta")
    elif meta is not None:
        raise ValueError("meta: must be None for a layout without index dwords")
    _need(gamma, torch.float32, 1, dev, "gamma")
    if out is None:
        y = torch.empty((T, n), dtype=torch.float32, device=dev)
        acc = torch.empty((T, n), dtype=torch.int32, device=dev) if want_acc else None
    else:
        y, acc = out
    _need(y, torch.float32, T * n, dev, "y")
    if acc is not None:
        _need(acc, torch.int32, T * n, dev, "acc")
    _check(bitlinear_fwd(xq.data_ptr(), scale.data_ptr(), T, K, codes.data_ptr(), _ptr(meta),
                         gamma.data_ptr(), N, M, layout, n, y.data_ptr(), _ptr(acc), _stream()),
           "bitlinear_fwd")
    return (y, acc) if want_acc else y


def transcode6(codes, meta, n: int, K: int, out=None):
    """Re-encode the 2:4 SPARSE packed buffers (codes, meta) of an n x K master into the SPARSE6
    stream (uint8); the master's gamma is unchanged.  ``out`` may supply the stream buffer."""
    import torch
    cb, mb, _, _ = packed_bytes(n, K, 2, 4, BL_LAYOUT_SPARSE)
    sb, _, _, _ = packed_bytes(n, K, 2, 4, BL_LAYOUT_SPARSE6)
    dev = codes.device
    _need(codes, torch.uint8, cb, dev, "codes")
    _need(meta, torch.uint8, mb, dev, "meta")
    if out is None:
        out = torch.empty(sb, dtype=torch.uint8, device=dev)
    _need(out, torch.uint8, sb, dev, "out")
    _check(bitlinear_transcode6(codes.data_ptr(), meta.data_ptr(), n, K, out.data_ptr(), _stream()),
           "bitlinear_transcode6")
    return out


class PackGroup:
    """A built grouped pack: ``PackGroup(masters)`` then ``group()`` re-packs every master.

    ``masters`` is a list of dicts with keys W (contiguous fp32 CUDA tensor [n][K]) and optionally
    out = (codes, meta, gamma); outputs are allocated when not given and exposed as
    ``group.outputs`` (a list of (codes, meta, gamma)).  Results equal ``pack`` per master, bit
    for bit.  Tensors are referenced, not copied; the masters are read at each launch.
    """

    def __init__(self, masters, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE, ws=None):
        import torch
        self._keep = list(masters)
        arr = (BlPackDesc * len(masters))()
        self.outputs = []
        for i, m in enumerate(masters):
            W = m["W"]
            assert W.is_cuda and W.dtype == torch.float32 and W.is_contiguous() and W.dim() == 2
            n, K = W.shape
            if m.get("out") is None:
                cb, mb, _, _ = packed_bytes(n, K, N, M, layout)
                out = (torch.empty(cb, dtype=torch.uint8, device=W.device),
                       torch.empty(mb, dtype=torch.uint8, device=W.device) if mb else None,
                       torch.empty(4, dtype=torch.float32, device=W.device)[:1])
            else:
                out = m["out"]
            self.outputs.append(out)
            arr[i] = BlPackDesc(W.data_ptr(), n, K, out[0].data_ptr(), _ptr(out[1]),
                                out[2].data_ptr())
        self.descs = arr
        st, plan = bitlinear_pack_group_plan(arr, N, M, layout)
        _check(st, "bitlinear_pack_group_plan")
        self.plan = plan
        dev = masters[0]["W"].device
        self.table = torch.empty(max(plan.table_bytes, 16), dtype=torch.uint8, device=dev)
        if ws is None:
            ws = torch.empty(max(plan.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.ws = ws
        _check(bitlinear_pack_group_build(arr, N, M, layout, ws.data_ptr(), ws.numel(),
                                          self.table.data_ptr(), self.table.numel(), _stream()),
               "bitlinear_pack_group_build")

    def __call__(self):
        _check(bitlinear_pack_group(self.table.data_ptr(), self.plan, _stream()),
               "bitlinear_pack_group")


class FwdGroup:
    """A built group of independent projections: ``FwdGroup(projs)`` then ``group()`` launches.

    ``projs`` is a list of dicts with keys xq, scale, K, codes, meta, gamma, n, y and optionally
    acc (torch CUDA tensors / ints), all sharing (N, M, layout).  The tensors are referenced, not
    copied: keep them alive while the group is used; their contents are read at each launch.
    """

    def __init__(self, projs, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE):
        import torch
        self.N, self.M, self.layout = N, M, layout
        self._keep = list(projs)
        arr = (BlFwdDesc * len(projs))()
        for i, p in enumerate(projs):
            arr[i] = BlFwdDesc(_ptr(p["xq"]), _ptr(p["scale"]), p["xq"].shape[0], p["K"],
                               _ptr(p["codes"]), _ptr(p.get("meta")), _ptr(p["gamma"]), p["n"],
                               _ptr(p["y"]), _ptr(p.get("acc")))
        self.descs = arr
        st, tb, wi = bitlinear_group_table_bytes(arr, N, M, layout)
        _check(st, "bitlinear_group_table_bytes")
        dev = projs[0]["codes"].device
        self.table = torch.empty(max(tb, 16), dtype=torch.uint8, device=dev)
        self.work_items = wi
        _check(bitlinear_group_build(arr, N, M, layout, self.table.data_ptr(), self.table.numel(),
                                     _stream()), "bitlinear_group_build")

    def __call__(self):
        _check(bitlinear_fwd_group(self.table.data_ptr(), self.work_items, self.N, self.M,
                                   self.layout, _stream()), "bitlinear_fwd_group")


class GemmGroup:
    """A built grouped prefill forward: ``GemmGroup(projs)`` then ``group()`` launches.

    ``projs`` as for FwdGroup (T > 128 tokens each).  y (and acc) equal ``fwd`` per projection,
    bit for bit.  The tensors are referenced, not copied; their contents are read at each launch.
    """

    def __init__(self, projs, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE):
        import torch
        self._keep = list(projs)
        arr = (BlFwdDesc * len(projs))()
        for i, p in enumerate(projs):
            arr[i] = BlFwdDesc(_ptr(p["xq"]), _ptr(p["scale"]), p["xq"].shape[0], p["K"],
                               _ptr(p["codes"]), _ptr(p.get("meta")), _ptr(p["gamma"]), p["n"],
                               _ptr(p["y"]), _ptr(p.get("acc")))
        self.descs = arr
        st, plan = bitlinear_gemm_group_plan(arr, N, M, layout)
        _check(st, "bitlinear_gemm_group_plan")
        self.plan = plan
        dev = projs[0]["codes"].device
        self.table = torch.empty(max(plan.table_bytes, 16), dtype=torch.uint8, device=dev)
        _check(bitlinear_gemm_group_build(arr, N, M, layout, self.table.data_ptr(),
                                          self.table.numel(), _stream()),
               "bitlinear_gemm_group_build")

    def __call__(self):
        _check(bitlinear_gemm_group(self.table.data_ptr(), self.plan, _stream()),
               "bitlinear_gemm_group")


class FusedGroup:
    """A built fused group: ``FusedGroup(projs)`` then ``group()`` quantizes and multiplies.

    ``projs`` is a list of dicts with keys x (bf16 CUDA tensor [T][K]), K, codes, meta, gamma, n,
    y and optionally acc, all sharing (N, M, layout) with no activation lifting (2:4 SPARSE or
    DENSE2).  Tensors are referenced, not copied; their contents are read at each launch.
    """

    def __init__(self, projs, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE):
        import torch
        self.N, self.M, self.layout = N, M, layout
        self._keep = list(projs)
        arr = (BlFwdXDesc * len(projs))()
        for i, p in enumerate(projs):
            arr[i] = BlFwdXDesc(_ptr(p["x"]), p["x"].shape[0], p["K"], _ptr(p["codes"]),
                                _ptr(p.get("meta")), _ptr(p["gamma"]), p["n"], _ptr(p["y"]),
                                _ptr(p.get("acc")))
        self.descs = arr
        st, tb, wi = bitlinear_group_fused_table_bytes(arr, N, M, layout)
        _check(st, "bitlinear_group_fused_table_bytes")
        dev = projs[0]["codes"].device
        self.table = torch.empty(max(tb, 16), dtype=torch.uint8, device=dev)
        self.work_items = wi
        _check(bitlinear_group_fused_build(arr, N, M, layout, self.table.data_ptr(),
                                           self.table.numel(), _stream()),
               "bitlinear_group_fused_build")

    def __call__(self):
        _check(bitlinear_fwd_group_fused(self.table.data_ptr(), self.work_items, self.N, self.M,
                                         self.layout, _stream()), "bitlinear_fwd_group_fused")


def bwd_workspace_bytes(T: int, n: int, K: int) -> int:
    st, ws = bitlinear_bwd_workspace_bytes(T, n, K)
    _check(st, "bitlinear_bwd_workspace_bytes")
    return ws


def bwd(dy, xq, scale, K: int, codes, meta, gamma, n: int, N: int = 2, M: int = 4,
        layout: int = BL_LAYOUT_SPARSE, want_dx: bool = True, want_dw: bool = True,
        out=None, accumulate: Tuple[bool, bool] = (False, False), ws=None):
    """Straight-through gradients (dx fp32 [T][K], dw fp32 [n][K]) of one BitLinear.

    dy: bf16 [T][n]; xq / scale: the plain (unlifted) int8 activations and token scales; codes /
    meta / gamma: the packed weights.  ``out`` may supply (dx, dw) (either may be None when not
    wanted); ``accumulate`` adds into them.  ``ws`` may supply a uint8 workspace.
    """
    import torch
    T = dy.shape[0]
    dev = dy.device
    if out is None:
        dx = torch.empty((T, K), dtype=torch.float32, device=dev) if want_dx else None
        dw = torch.empty((n, K), dtype=torch.float32, device=dev) if want_dw else None
    else:
        dx, dw = out
    if ws is None:
        ws = torch.empty(max(bwd_workspace_bytes(T, n, K), 256), dtype=torch.uint8, device=dev)
    flags = (BL_BWD_ACCUM_DX if accumulate[0] else 0) | (BL_BWD_ACCUM_DW if accumulate[1] else 0)
    _check(bitlinear_bwd(_ptr(dy), T, n, _ptr(xq), _ptr(scale), K, _ptr(codes), _ptr(meta),
                         _ptr(gamma), N, M, layout, _ptr(dx), _ptr(dw), flags, _ptr(ws), ws.numel(),
                         _stream()), "bitlinear_bwd")
    return dx, dw


class BwdGroup:
    """A built grouped backward: ``BwdGroup(projs, T)`` then ``group()`` computes every gradient.

    ``projs`` is a list of dicts with keys dy (bf16 [T][n]), xq, scale, K, codes, meta, gamma, n,
    dx, dw (fp32 tensors or None) and optionally accumulate = (dx?, dw?), all sharing T and
    (N, M, layout).  The result is that of ``bwd`` called for each projection in list order;
    projections that name the same dx tensor sum into it (with accumulate[0] set on the later
    ones).  Tensors are referenced, not copied; their contents are read at each launch.  ``ws``
    may supply the uint8 workspace.
    """

    def __init__(self, projs, T: int, N: int = 2, M: int = 4, layout: int = BL_LAYOUT_SPARSE,
                 ws=None):
        import torch
        self._keep = list(projs)
        arr = (BlBwdDesc * len(projs))()
        for i, p in enumerate(projs):
            acc = p.get("accumulate", (False, False))
            flags = (BL_BWD_ACCUM_DX if acc[0] else 0) | (BL_BWD_ACCUM_DW if acc[1] else 0)
            arr[i] = BlBwdDesc(_ptr(p["dy"]), _ptr(p["xq"]), _ptr(p["scale"]), p["K"],
                               _ptr(p["codes"]), _ptr(p.get("meta")), _ptr(p["gamma"]), p["n"],
                               _ptr(p.get("dx")), _ptr(p.get("dw")), flags, 0)
        self.descs = arr
        st, plan = bitlinear_bwd_group_plan(arr, T, N, M, layout)
        _check(st, "bitlinear_bwd_group_plan")
        self.plan = plan
        dev = projs[0]["codes"].device
        self.table = torch.empty(max(plan.table_bytes, 16), dtype=torch.uint8, device=dev)
        if ws is None:
            ws = torch.empty(max(plan.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.ws = ws
        _check(bitlinear_bwd_group_build(arr, T, N, M, layout, ws.data_ptr(), ws.numel(),
                                         self.table.data_ptr(), self.table.numel(), _stream()),
               "bitlinear_bwd_group_build")

    def __call__(self):
        _check(bitlinear_bwd_group(self.table.data_ptr(), self.plan, _stream()),
               "bitlinear_bwd_group")


class Chain:
    """A built fused decode chain: ``Chain(layers, T)`` then ``chain(x0)`` runs every layer.

    ``layers`` is a list of dicts with keys codes, meta, gamma, n, K and optionally y and acc
    (2:4 packed weights; K of each layer == n of the previous one).  y (fp32 [T][n]) is
    allocated when not given; ``chain.ys`` / ``chain.accs`` list the outputs.  ``chain(x0)``
    (bf16 or fp32 CUDA tensor [T][K0]) enqueues the whole chain; ``chain.error()`` (a host sync)
    is nonzero if a bounded wait gave up, in which case the outputs are invalid.
    """

    def __init__(self, layers, T: int, ws=None):
        import torch
        self._keep = list(layers)
        self.T = T
        arr = (BlChainLayer * len(layers))()
        self.ys, self.accs = [], []
        dev = layers[0]["codes"].device
        for i, ly in enumerate(layers):
            y = ly.get("y")
            if y is None:
                y = torch.empty((T, ly["n"]), dtype=torch.float32, device=dev)
            _need(y, torch.float32, T * ly["n"], dev, f"layers[{i}] y")
            acc = ly.get("acc")
            if acc is not None:
                _need(acc, torch.int32, T * ly["n"], dev, f"layers[{i}] acc")
            cb, mb, _, _ = packed_bytes(ly["n"], ly["K"])
            _need(ly["codes"], torch.uint8, cb, dev, f"layers[{i}] codes")
            _need(ly["meta"], torch.uint8, mb, dev, f"layers[{i}] meta")
            _need(ly["gamma"], torch.float32, 1, dev, f"layers[{i}] gamma")
            self.ys.append(y)
            self.accs.append(acc)
            arr[i] = BlChainLayer(_ptr(ly["codes"]), _ptr(ly["meta"]), _ptr(ly["gamma"]), ly["n"],
                                  ly["K"], _ptr(y), _ptr(acc))
        self.layers = arr
        st, plan = bitlinear_chain_plan(arr, T, 2, 4, BL_LAYOUT_SPARSE)
        _check(st, "bitlinear_chain_plan")
        self.plan = plan
        self.table = torch.empty(max(plan.table_bytes, 16), dtype=torch.uint8, device=dev)
        if ws is None:
            ws = torch.empty(max(plan.ws_bytes, 256), dtype=torch.uint8, device=dev)
        _need(ws, torch.uint8, plan.ws_bytes, dev, "ws")
        self.ws = ws
        self.K0 = layers[0]["K"]
        _check(bitlinear_chain_build(arr, T, 2, 4, BL_LAYOUT_SPARSE, self.table.data_ptr(),
                                     self.table.numel(), _stream()), "bitlinear_chain_build")

    def __call__(self, x0, spin_limit: int = 0):
        import torch
        dts = {torch.float32: BL_DTYPE_F32, torch.bfloat16: BL_DTYPE_BF16}
        assert x0.is_cuda and x0.is_contiguous() and tuple(x0.shape) == (self.T, self.K0)
        _check(bitlinear_fwd_chain(self.table.data_ptr(), self.plan, x0.data_ptr(), dts[x0.dtype],
                                   self.ws.data_ptr(), self.ws.numel(), spin_limit, _stream()),
               "bitlinear_fwd_chain")

    def error(self) -> int:
        """The workspace's error word (after the launch completes; synchronizes the device)."""
        import torch
        torch.cuda.synchronize()
        return int(self.ws[4:8].cpu().view(torch.int32)[0])
