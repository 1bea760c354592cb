"""ctypes binding of libmoe.so: argument marshalling only.

Each function has the name of the C entry point it calls, takes torch
tensors resident on the GPU (PyTorch provides device memory and the stream)
and forwards raw pointers, sizes and strides.  Output tensors may be passed
in; otherwise they are allocated with ``torch.empty`` on the input's device.
All arithmetic happens in the HIP kernels.  If the shared library is
missing, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_BIAS_LOGIT, MOE_BIAS_SELECT = 0, 1
MOE_DERR_EXPERT_ID, MOE_DERR_GROUP_SIZES, MOE_DERR_ROWS = 1, 2, 4
MOE_FP8_E4M3, MOE_FP8_E5M2 = 0, 1
ABI_VERSION = 12  # moe_abi_version() of the library these signatures describe

# Entry points (name -> (restype, argtypes)); must match include/moe.h.
_P, _I, _L, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_F = ctypes.c_float
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_abi_version": (_I, []),
    "moe_route": (_I, [_P, _P, _I, _I, _I, _L, _I, _I, _I, _I, _P, _P, _P]),
    "moe_route_bwd": (_I, [_P, _P, _I, _P, _P, _L, _I, _I, _I, _I, _P, _I, _P]),
    "moe_aux_loss_workspace": (_S, [_L, _I]),
    "moe_aux_loss": (_I, [_P, _P, _L, _I, _I, _I, _F, _P, _P, _P, _P, _S, _P]),
    "moe_aux_loss_bwd": (_I, [_P, _P, _L, _I, _I, _I, _F, _P, _I, _I, _P]),
    "moe_rows_bound": (_L, [_L, _I, _I, _I, _I, _I]),
    "moe_permute_workspace": (_S, [_L, _I, _I]),
    "moe_permute": (_I, [_P, _I, _L, _L, _P, _I, _I, _I, _I, _I, _P, _L, _P, _P, _P, _P, _P,
                         _P, _S, _P, _P]),
    "moe_permute_noalloc": (_I, [_P, _I, _L, _L, _P, _I, _I, _I, _I, _I, _P, _L, _P, _P, _P, _P,
                                 _P, _P, _P]),
    "moe_permute_bwd": (_I, [_P, _I, _L, _L, _I, _L, _P, _P, _I, _P]),
    "moe_gmm": (_I, [_P, _L, _L, _P, _L, _L, _I, _P, _P, _I, _L, _L, _I, _P, _P, _L, _L, _I, _I,
                     _P, _P]),
    "moe_gmm_swiglu": (_I, [_P, _L, _L, _P, _L, _L, _P, _P, _I, _L, _L, _I, _P, _P, _L, _P, _L, _L,
                            _P, _P]),
    "moe_gmm_swiglu_bwd": (_I, [_P, _L, _L, _P, _L, _L, _P, _P, _I, _L, _L, _I, _P, _P, _L, _P, _P,
                                _L, _L, _P, _P]),
    "moe_tgmm": (_I, [_P, _L, _P, _L, _P, _P, _I, _L, _L, _L, _I, _P, _L, _L, _I, _I, _P, _P]),
    "moe_group_sum_workspace": (_S, [_L, _I, _L]),
    "moe_router_bwd_workspace": (_S, [_L, _L, _I]),
    "moe_router_bwd": (_I, [_P, _P, _P, _L, _L, _I, _P, _P, _I, _I, _P, _S, _P, _P]),
    "moe_group_sum": (_I, [_P, _L, _I, _P, _P, _I, _L, _L, _P, _I, _I, _P, _S, _P, _P]),
    "moe_fp8_scale_workspace": (_S, [_L, _L, _I]),
    "moe_fp8_amax_scale": (_I, [_P, _L, _I, _L, _L, _I, _I, _P, _P, _S, _P]),
    "moe_fp8_padded_rows": (_L, [_L, _I]),
    "moe_fp8_quantize": (_I, [_P, _L, _I, _L, _L, _P, _I, _P, _I, _I, _P, _L, _P, _L, _L, _P, _P]),
    "moe_gmm_fp8": (_I, [_P, _L, _L, _I, _P, _P, _L, _L, _I, _I, _P, _P, _P, _I, _L, _L, _P, _P,
                         _L, _L, _I, _I, _P, _P]),
    "moe_tgmm_fp8": (_I, [_P, _L, _I, _P, _P, _L, _I, _P, _P, _P, _I, _L, _L, _L, _P, _L, _L, _I,
                          _I, _P, _P]),
    "moe_swiglu": (_I, [_P, _P, _I, _L, _L, _L, _P, _I, _P]),
    "moe_swiglu_bwd": (_I, [_P, _P, _I, _L, _P, _L, _L, _P, _P, _L, _I, _P]),
    "moe_combine": (_I, [_P, _I, _L, _L, _I, _L, _P, _P, _P, _P]),
    "moe_combine_bwd": (_I, [_P, _P, _I, _L, _L, _I, _L, _P, _P, _P, _P, _P, _P]),
}

_lib = None


class MoeError(RuntimeError):
    pass


def load():
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_grouped_top_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.moe_abi_version() != ABI_VERSION:
            raise MoeError(f"{LIB_PATH} reports ABI version {lib.moe_abi_version()}, the binding "
                           f"expects {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load().moe_status_string(rc).decode()
        raise MoeError(f"{what} failed with status {rc}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError("tensor must be on the GPU")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoeError(f"unsupported dtype {t.dtype}")


def _torch_dtype(code: int):
    return torch.bfloat16 if code == MOE_BF16 else torch.float32


def _score(score) -> int:
    if score in ("softmax", MOE_SOFTMAX):
        return MOE_SOFTMAX
    if score in ("sigmoid", MOE_SIGMOID):
        return MOE_SIGMOID
    raise MoeError(f"unknown score function {score!r}")


def _rowmajor(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise MoeError(f"{name} must be a 2-D view with unit column stride")
    return t.stride(0)


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")


def _i32vec(t: Optional[torch.Tensor], n: int, name: str, optional: bool = False):
    """A contiguous int32 vector of n entries (group sizes, valid rows)."""
    if t is None:
        if optional:
            return
        raise MoeError(f"{name} is required")
    if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1 or t.numel() != n:
        raise MoeError(f"{name} must be a contiguous int32 vector of {n} entries "
                       f"(got {t.dtype}, shape {tuple(t.shape)})")


# ----------------------------------------------------------------- routing

def _bias_mode(mode) -> int:
    if mode in ("logit", MOE_BIAS_LOGIT):
        return MOE_BIAS_LOGIT
    if mode in ("select", MOE_BIAS_SELECT):
        return MOE_BIAS_SELECT
    raise MoeError(f"unknown bias mode {mode!r}")


def moe_route(logits, K: int, score="softmax", renorm: bool = True, bias=None,
              topk_ids=None, topk_w=None, stream=None, bias_mode="logit", n_groups: int = 0,
              topk_groups: int = 0):
    T, E = logits.shape
    _contig(logits, "logits")
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    _check(load().moe_route(_ptr(logits), _ptr(bias), _bias_mode(bias_mode), int(n_groups),
                            int(topk_groups), T, E, K, _score(score), int(bool(renorm)),
                            _ptr(topk_ids), _ptr(topk_w), _stream(stream)), "moe_route")
    return topk_ids, topk_w


def moe_route_bwd(logits, topk_ids, d_topk_w, score="softmax", renorm: bool = True, bias=None,
                  d_logits=None, dtype=torch.float32, stream=None, bias_mode="logit"):
    T, E = logits.shape
    K = topk_ids.shape[1]
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=dtype, device=logits.device)
    _check(load().moe_route_bwd(_ptr(logits), _ptr(bias), _bias_mode(bias_mode), _ptr(topk_ids),
                                _ptr(d_topk_w), T, E, K, _score(score), int(bool(renorm)),
                                _ptr(d_logits), _dtype_code(d_logits), _stream(stream)),
           "moe_route_bwd")
    return d_logits


def moe_aux_loss_workspace(T: int, E: int) -> int:
    return load().moe_aux_loss_workspace(T, E)


def moe_aux_loss(logits, topk_ids, alpha: float, score="softmax", loss=None, counts=None,
                 probs=None, workspace=None, stream=None):
    """Returns (loss [1] float32, counts [E] int32, probs [E] float32)."""
    T, E = logits.shape
    K = topk_ids.shape[1]
    _contig(logits, "logits")
    dev = logits.device
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if probs is None:
        probs = torch.empty(E, dtype=torch.float32, device=dev)
    ws_bytes = moe_aux_loss_workspace(T, E)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(load().moe_aux_loss(_ptr(logits), _ptr(topk_ids), T, E, K, _score(score), float(alpha),
                               _ptr(loss), _ptr(counts), _ptr(probs), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_aux_loss")
    return loss, counts, probs


def moe_aux_loss_bwd(logits, counts, K: int, alpha: float, score="softmax", d_logits=None,
                     dtype=torch.float32, accumulate: bool = False, stream=None):
    T, E = logits.shape
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=dtype, device=logits.device)
    _check(load().moe_aux_loss_bwd(_ptr(logits), _ptr(counts), T, E, K, _score(score),
                                   float(alpha), _ptr(d_logits), _dtype_code(d_logits),
                                   int(bool(accumulate)), _stream(stream)), "moe_aux_loss_bwd")
    return d_logits


# ------------------------------------------------------------- permutation

def moe_rows_bound(T: int, K: int, E: int, align: int = 0, capacity: int = 0,
                   capacity_layout: bool = False) -> int:
    r = load().moe_rows_bound(T, K, E, align, capacity, int(bool(capacity_layout)))
    if r < 0:
        raise MoeError("moe_rows_bound: invalid arguments")
    return r


def moe_permute_workspace(T: int, K: int, E: int) -> int:
    return load().moe_permute_workspace(T, K, E)


def moe_permute(x, topk_ids, E: int, align: int = 0, capacity: int = 0,
                capacity_layout: bool = False, rows: Optional[int] = None, x_sorted=None,
                with_rows: bool = True, err=None, workspace=None, out=None, stream=None,
                noalloc: bool = False):
    """Returns dict(x_sorted, counts, group_sizes, group_offsets, row_of_slot,
    slot_of_row).  ``rows`` defaults to moe_rows_bound(...); ``out`` may hold
    preallocated index tensors under the same keys.  ``noalloc`` calls
    moe_permute_noalloc (the library's static scratch, no workspace)."""
    T, K = topk_ids.shape
    dev = topk_ids.device
    if rows is None:
        rows = moe_rows_bound(T, K, E, align, capacity, capacity_layout)
    out = dict(out or {})
    i32 = dict(dtype=torch.int32, device=dev)
    counts = out.get("counts") if out.get("counts") is not None else torch.empty(E, **i32)
    gsz = out.get("group_sizes") if out.get("group_sizes") is not None else torch.empty(E, **i32)
    goff = out.get("group_offsets") if out.get("group_offsets") is not None else torch.empty(E + 1, **i32)
    ros = out.get("row_of_slot") if out.get("row_of_slot") is not None else torch.empty(T * K, **i32)
    sor = out.get("slot_of_row") if out.get("slot_of_row") is not None else torch.empty(rows, **i32)
    D = 0
    dt = MOE_BF16
    if x is not None and with_rows:
        T2, D = x.shape
        assert T2 == T
        _contig(x, "x")
        dt = _dtype_code(x)
        if x_sorted is None:
            x_sorted = torch.empty((rows, D), dtype=x.dtype, device=dev)
        _contig(x_sorted, "x_sorted")
        assert x_sorted.shape[0] == rows and x_sorted.shape[1] == D
    else:
        x_sorted = None
    if noalloc:
        _check(load().moe_permute_noalloc(_ptr(x) if x_sorted is not None else None, dt, T, D,
                                          _ptr(topk_ids), K, E, align, capacity,
                                          int(bool(capacity_layout)), _ptr(x_sorted), rows,
                                          _ptr(counts), _ptr(gsz), _ptr(goff), _ptr(ros),
                                          _ptr(sor), _ptr(err), _stream(stream)),
               "moe_permute_noalloc")
        return dict(x_sorted=x_sorted, counts=counts, group_sizes=gsz, group_offsets=goff,
                    row_of_slot=ros, slot_of_row=sor)
    ws_bytes = moe_permute_workspace(T, K, E)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(load().moe_permute(_ptr(x) if x_sorted is not None else None, dt, T, D, _ptr(topk_ids),
                              K, E, align, capacity, int(bool(capacity_layout)), _ptr(x_sorted),
                              rows, _ptr(counts), _ptr(gsz), _ptr(goff), _ptr(ros), _ptr(sor),
                              _ptr(workspace), workspace.numel(), _ptr(err), _stream(stream)),
           "moe_permute")
    return dict(x_sorted=x_sorted, counts=counts, group_sizes=gsz, group_offsets=goff,
                row_of_slot=ros, slot_of_row=sor)


def moe_permute_bwd(d_x_sorted, row_of_slot, T: int, K: int, d_x=None, accumulate: bool = False,
                    stream=None):
    rows, D = d_x_sorted.shape
    _contig(d_x_sorted, "d_x_sorted")
    if d_x is None:
        d_x = torch.empty((T, D), dtype=d_x_sorted.dtype, device=d_x_sorted.device)
    _contig(d_x, "d_x")
    _check(load().moe_permute_bwd(_ptr(d_x_sorted), _dtype_code(d_x_sorted), T, D, K, rows,
                                  _ptr(row_of_slot), _ptr(d_x), int(bool(accumulate)),
                                  _stream(stream)), "moe_permute_bwd")
    return d_x


# ----------------------------------------------------------- grouped GEMMs

def moe_gmm(lhs, rhs, group_sizes, trans_rhs: bool = False, out=None, rows_out: Optional[int] = None,
            out_dtype=None, accumulate: bool = False, err=None, stream=None, bias=None,
            valid_rows=None):
    """out[rows of g] (+)= lhs[rows of g] . rhs[g] (+ bias[g]) (rhs[g]: [K, N],
    or [N, K] used transposed; bias: optional contiguous [G, N] in lhs's
    dtype).  lhs and out may be strided 2-D views (unit column stride); rhs
    a 3-D view with unit last stride.  valid_rows ([G] int32, optional): lhs
    rows past valid_rows[g] in each group are zero and are not read."""
    M_lhs, Kd = lhs.shape
    ld_lhs = _rowmajor(lhs, "lhs")
    if rhs.dim() != 3 or rhs.stride(2) != 1:
        raise MoeError("rhs must be a 3-D view with unit last stride")
    G = rhs.shape[0]
    N = rhs.shape[1] if trans_rhs else rhs.shape[2]
    if (rhs.shape[2] if trans_rhs else rhs.shape[1]) != Kd:
        raise MoeError("contracting dimensions differ")
    _i32vec(group_sizes, G, "group_sizes")
    _i32vec(valid_rows, G, "valid_rows", optional=True)
    if lhs.dtype != rhs.dtype:
        raise MoeError("lhs and rhs dtypes differ")
    if bias is not None:
        _contig(bias, "bias")
        if tuple(bias.shape) != (G, N) or bias.dtype != lhs.dtype:
            raise MoeError("bias must be [G, N] in the dtype of lhs")
    if out is None:
        M_out = M_lhs if rows_out is None else rows_out
        odt = lhs.dtype if out_dtype is None else out_dtype
        out = torch.empty((M_out, N), dtype=odt, device=lhs.device)
    if out.dim() != 2 or out.shape[1] != N:
        raise MoeError(f"out must be [rows, {N}] (got {tuple(out.shape)})")
    if out_dtype is not None and out.dtype != out_dtype:
        raise MoeError("out does not have out_dtype")
    M_out = out.shape[0]
    ld_out = _rowmajor(out, "out")
    _check(load().moe_gmm(_ptr(lhs), M_lhs, ld_lhs, _ptr(rhs), rhs.stride(1), rhs.stride(0),
                          int(bool(trans_rhs)), _ptr(group_sizes), _ptr(valid_rows), G, Kd, N,
                          _dtype_code(lhs),
                          _ptr(bias), _ptr(out), M_out, ld_out, _dtype_code(out), int(bool(accumulate)),
                          _ptr(err), _stream(stream)), "moe_gmm")
    return out


def moe_gmm_swiglu(lhs, wi, group_sizes, act=None, h=None, rows_out: Optional[int] = None,
                   bias=None, valid_rows=None, write_h: bool = True, err=None, stream=None):
    """Fused up-projection with SwiGLU: h[rows of g] = lhs[rows of g] . wi[g]
    (+ bias[g]) with wi [G, K, 2F] = [wi_0 | wi_1] (3-D view, unit last
    stride), and act = silu(h[:, :F]) * h[:, F:] from the bf16-rounded h.
    Returns (h, act); h is allocated only when write_h and h is None."""
    M_lhs, Kd = lhs.shape
    ld_lhs = _rowmajor(lhs, "lhs")
    if wi.dim() != 3 or wi.stride(2) != 1:
        raise MoeError("wi must be a 3-D view with unit last stride")
    G, K2, F2 = wi.shape
    if K2 != Kd:
        raise MoeError("contracting dimensions differ")
    if F2 % 2:
        raise MoeError("wi must have 2F columns")
    F = F2 // 2
    _i32vec(group_sizes, G, "group_sizes")
    _i32vec(valid_rows, G, "valid_rows", optional=True)
    if lhs.dtype != wi.dtype:
        raise MoeError("lhs and wi dtypes differ")
    if bias is not None:
        _contig(bias, "bias")
        if tuple(bias.shape) != (G, F2) or bias.dtype != lhs.dtype:
            raise MoeError("bias must be [G, 2F] in the dtype of lhs")
    M_out = M_lhs if rows_out is None else rows_out
    if act is None:
        act = torch.empty((M_out, F), dtype=lhs.dtype, device=lhs.device)
    if h is None and write_h:
        h = torch.empty((M_out, F2), dtype=lhs.dtype, device=lhs.device)
    if act.dim() != 2 or act.shape[0] != M_out or act.shape[1] != F:
        raise MoeError("act must be [rows_out, F]")
    if h is not None and (h.dim() != 2 or h.shape[0] != M_out or h.shape[1] != F2):
        raise MoeError("h must be [rows_out, 2F]")
    if act.dtype != torch.bfloat16 or (h is not None and h.dtype != torch.bfloat16):
        raise MoeError("h and act must be bfloat16")
    ld_act = _rowmajor(act, "act")
    ld_h = _rowmajor(h, "h") if h is not None else 0
    _check(load().moe_gmm_swiglu(_ptr(lhs), M_lhs, ld_lhs, _ptr(wi), wi.stride(1), wi.stride(0),
                                 _ptr(group_sizes), _ptr(valid_rows), G, Kd, F, _dtype_code(lhs),
                                 _ptr(bias), _ptr(h), ld_h, _ptr(act), ld_act, M_out, _ptr(err),
                                 _stream(stream)), "moe_gmm_swiglu")
    return h, act


def moe_gmm_swiglu_bwd(d_y, wo, group_sizes, h0, h1, d_h0=None, d_h1=None,
                       rows_out: Optional[int] = None, valid_rows=None, err=None, stream=None):
    """d_act[rows of g] = d_y[rows of g] . wo[g]^T (wo [G, F, K], 3-D view with
    unit last stride), rounded to bf16, then the SwiGLU backward with the
    forward's h0, h1 ([M, F] 2-D views sharing one row stride) into d_h0,
    d_h1 ([M, F] views sharing one row stride).  Returns (d_h0, d_h1)."""
    M_lhs, Kd = d_y.shape
    ld_lhs = _rowmajor(d_y, "d_y")
    if wo.dim() != 3 or wo.stride(2) != 1:
        raise MoeError("wo must be a 3-D view with unit last stride")
    G, F, K2 = wo.shape
    if K2 != Kd:
        raise MoeError("contracting dimensions differ")
    _i32vec(group_sizes, G, "group_sizes")
    _i32vec(valid_rows, G, "valid_rows", optional=True)
    if d_y.dtype != wo.dtype:
        raise MoeError("d_y and wo dtypes differ")
    M_out = M_lhs if rows_out is None else rows_out
    if d_h0 is None:
        d_h0 = torch.empty((M_out, F), dtype=d_y.dtype, device=d_y.device)
    if d_h1 is None:
        d_h1 = torch.empty((M_out, F), dtype=d_y.dtype, device=d_y.device)
    for t, n in ((h0, "h0"), (h1, "h1"), (d_h0, "d_h0"), (d_h1, "d_h1")):
        if t.dim() != 2 or t.shape[0] < M_out or t.shape[1] != F:
            raise MoeError(f"{n} must be [rows_out, F]")
        if t.dtype != torch.bfloat16:
            raise MoeError(f"{n} must be bfloat16")
    ld_h, ld_dh = _rowmajor(h0, "h0"), _rowmajor(d_h0, "d_h0")
    if _rowmajor(h1, "h1") != ld_h or _rowmajor(d_h1, "d_h1") != ld_dh:
        raise MoeError("h0/h1 and d_h0/d_h1 must share their row strides")
    _check(load().moe_gmm_swiglu_bwd(_ptr(d_y), M_lhs, ld_lhs, _ptr(wo), wo.stride(1), wo.stride(0),
                                     _ptr(group_sizes), _ptr(valid_rows), G, Kd, F,
                                     _dtype_code(d_y), _ptr(h0), _ptr(h1), ld_h, _ptr(d_h0),
                                     _ptr(d_h1), ld_dh, M_out, _ptr(err), _stream(stream)),
           "moe_gmm_swiglu_bwd")
    return d_h0, d_h1


def moe_tgmm(lhs, rhs, group_sizes, out=None, out_dtype=None, accumulate: bool = False, err=None,
             stream=None, valid_rows=None):
    """out[g] (+)= lhs[rows of g]^T . rhs[rows of g] -> [G, K, N].  valid_rows
    ([G] int32, optional): rows past valid_rows[g] in each group are zero in
    lhs or rhs and are skipped."""
    M, Kd = lhs.shape
    M2, N = rhs.shape
    if M2 != M:
        raise MoeError("lhs and rhs row counts differ")
    if lhs.dtype != rhs.dtype:
        raise MoeError("lhs and rhs dtypes differ")
    G = group_sizes.numel()
    _i32vec(group_sizes, G, "group_sizes")
    _i32vec(valid_rows, G, "valid_rows", optional=True)
    if out is None:
        odt = lhs.dtype if out_dtype is None else out_dtype
        out = torch.empty((G, Kd, N), dtype=odt, device=lhs.device)
    if out.dim() != 3 or out.stride(2) != 1 or tuple(out.shape) != (G, Kd, N):
        raise MoeError(f"out must be [{G}, {Kd}, {N}] with unit last stride "
                       f"(got {tuple(out.shape)})")
    if out_dtype is not None and out.dtype != out_dtype:
        raise MoeError("out does not have out_dtype")
    _check(load().moe_tgmm(_ptr(lhs), _rowmajor(lhs, "lhs"), _ptr(rhs), _rowmajor(rhs, "rhs"),
                           _ptr(group_sizes), _ptr(valid_rows), G, M, Kd, N, _dtype_code(lhs),
                           _ptr(out),
                           out.stride(1), out.stride(0), _dtype_code(out), int(bool(accumulate)),
                           _ptr(err), _stream(stream)), "moe_tgmm")
    return out


def moe_router_bwd_workspace(T: int, D: int, E: int) -> int:
    return load().moe_router_bwd_workspace(T, D, E)


def moe_router_bwd(x, Wg, d_logits, d_Wg=None, dx=None, accumulate_dx: bool = False,
                   dx_dtype=None, workspace=None, err=None, stream=None):
    """Router-GEMM backward: d_Wg = x^T . d_logits [D, E] float32 and
    dx (+)= d_logits . Wg^T [T, D] (x [T, D], Wg [D, E] bf16; d_logits
    [T, E] float32; all contiguous).  Returns (d_Wg, dx)."""
    T, D = x.shape
    D2, E = Wg.shape
    if D2 != D or tuple(d_logits.shape) != (T, E):
        raise MoeError("x [T, D], Wg [D, E] and d_logits [T, E] do not match")
    if x.dtype != torch.bfloat16 or Wg.dtype != torch.bfloat16:
        raise MoeError("x and Wg must be bfloat16")
    if d_logits.dtype != torch.float32:
        raise MoeError("d_logits must be float32")
    for t, n in ((x, "x"), (Wg, "Wg"), (d_logits, "d_logits")):
        _contig(t, n)
    if d_Wg is None:
        d_Wg = torch.empty((D, E), dtype=torch.float32, device=x.device)
    if tuple(d_Wg.shape) != (D, E) or d_Wg.dtype != torch.float32:
        raise MoeError("d_Wg must be [D, E] float32")
    _contig(d_Wg, "d_Wg")
    if dx is None:
        if accumulate_dx:
            raise MoeError("accumulate_dx needs dx")
        dx = torch.empty((T, D), dtype=x.dtype if dx_dtype is None else dx_dtype, device=x.device)
    if tuple(dx.shape) != (T, D):
        raise MoeError("dx must be [T, D]")
    _contig(dx, "dx")
    ws_bytes = moe_router_bwd_workspace(T, D, E)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    _check(load().moe_router_bwd(_ptr(x), _ptr(Wg), _ptr(d_logits), T, D, E, _ptr(d_Wg),
                                 _ptr(dx), _dtype_code(dx), int(bool(accumulate_dx)),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _ptr(err), _stream(stream)), "moe_router_bwd")
    return d_Wg, dx


def moe_group_sum_workspace(M: int, G: int, N: int) -> int:
    return load().moe_group_sum_workspace(M, G, N)


def moe_group_sum(x, group_sizes, out=None, out_dtype=torch.float32, accumulate: bool = False,
                  valid_rows=None, workspace=None, err=None, stream=None):
    """out[g] (+)= sum of the rows of group g of x [M, N] -> [G, N] (the
    gradient of a per-group bias).  x may be a strided 2-D view."""
    M, N = x.shape
    G = group_sizes.numel()
    if out is None:
        out = torch.empty((G, N), dtype=out_dtype, device=x.device)
    _contig(out, "out")
    if tuple(out.shape) != (G, N):
        raise MoeError("out must be [G, N]")
    _i32vec(group_sizes, G, "group_sizes")
    _i32vec(valid_rows, G, "valid_rows", optional=True)
    ws_bytes = moe_group_sum_workspace(M, G, N)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    _check(load().moe_group_sum(_ptr(x), _rowmajor(x, "x"), _dtype_code(x), _ptr(group_sizes),
                                _ptr(valid_rows), G, M, N, _ptr(out), _dtype_code(out),
                                int(bool(accumulate)), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _ptr(err),
                                _stream(stream)), "moe_group_sum")
    return out


# --------------------------------------------------------------------- FP8

def _fmt(f) -> int:
    if f in ("e4m3", MOE_FP8_E4M3):
        return MOE_FP8_E4M3
    if f in ("e5m2", MOE_FP8_E5M2):
        return MOE_FP8_E5M2
    raise MoeError(f"unknown FP8 format {f!r}")


def moe_fp8_scale_workspace(rows: int, cols: int, G: int = 1) -> int:
    return load().moe_fp8_scale_workspace(rows, cols, G)


def moe_fp8_padded_rows(rows: int, G: int) -> int:
    return load().moe_fp8_padded_rows(rows, G)


def moe_fp8_amax_scale(x, fmt, G: int = 1, scales=None, workspace=None, stream=None):
    """Current scaling of x [rows, cols] (G equal row blocks): returns the
    float32 [3, G] tensor (amax, scale, scale_inv)."""
    rows, cols = x.shape
    if scales is None:
        scales = torch.empty((3, G), dtype=torch.float32, device=x.device)
    _contig(scales, "scales")
    ws_bytes = moe_fp8_scale_workspace(rows, cols, G)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    _check(load().moe_fp8_amax_scale(_ptr(x), _rowmajor(x, "x"), _dtype_code(x), rows, cols, G,
                                     _fmt(fmt), _ptr(scales), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream)), "moe_fp8_amax_scale")
    return scales


def moe_fp8_quantize(x, group_sizes, scale, fmt, per_group: bool = False, q=None, qt=None,
                     qt_group_stride: int = 0, ld_qt: Optional[int] = None, err=None, stream=None):
    """FP8 codes of x [rows, cols] times scale (device float32: scale[g] per
    group, or scale[0]).  q: row-wise uint8 copy [rows, cols] (2-D view) or
    None; qt: transposed copy (uint8 buffer; padded [cols, P] layout when
    qt_group_stride is 0, else per group [cols, n_g] blocks) or None."""
    rows, cols = x.shape
    G = group_sizes.numel()
    ld_q = _rowmajor(q, "q") if q is not None else 0
    if qt is not None and ld_qt is None:
        ld_qt = qt.stride(0) if qt.dim() == 2 else qt.stride(-2)
    _check(load().moe_fp8_quantize(_ptr(x), _rowmajor(x, "x"), _dtype_code(x), rows, cols,
                                   _ptr(group_sizes), G, _ptr(scale), int(bool(per_group)),
                                   _fmt(fmt), _ptr(q), ld_q, _ptr(qt), int(ld_qt or 0),
                                   int(qt_group_stride), _ptr(err), _stream(stream)),
           "moe_fp8_quantize")
    return q, qt


def moe_gmm_fp8(lhs, lhs_fmt, lhs_scale_inv, rhs, rhs_fmt, rhs_scale_inv, group_sizes, out=None,
                rows_out: Optional[int] = None, out_dtype=torch.bfloat16, accumulate: bool = False,
                bias=None, err=None, stream=None, valid_rows=None, trans_rhs: bool = True):
    """out[rows of g] (+)= sa sb[g] lhs[rows of g] . B_g (+ bias[g]); lhs
    uint8 [M, K] (2-D view); rhs uint8 3-D view with unit last stride:
    [G, N, K] holding B_g^T (trans_rhs) or [G, K, N] holding B_g; scale_inv
    tensors float32 on the device."""
    M_lhs, Kd = lhs.shape
    if rhs.dim() != 3 or rhs.stride(2) != 1 or rhs.shape[2 if trans_rhs else 1] != Kd:
        raise MoeError("rhs must be a [G, N, K] (trans_rhs) or [G, K, N] view with unit last "
                       "stride")
    G, N = rhs.shape[0], rhs.shape[1 if trans_rhs else 2]
    if out is None:
        out = torch.empty((M_lhs if rows_out is None else rows_out, N), dtype=out_dtype,
                          device=lhs.device)
    if bias is not None:
        _contig(bias, "bias")
    _check(load().moe_gmm_fp8(_ptr(lhs), M_lhs, _rowmajor(lhs, "lhs"), _fmt(lhs_fmt),
                              _ptr(lhs_scale_inv), _ptr(rhs), rhs.stride(1), rhs.stride(0),
                              int(bool(trans_rhs)), _fmt(rhs_fmt), _ptr(rhs_scale_inv),
                              _ptr(group_sizes),
                              _ptr(valid_rows), G, Kd, N,
                              _ptr(bias), _ptr(out), out.shape[0], _rowmajor(out, "out"),
                              _dtype_code(out), int(bool(accumulate)), _ptr(err),
                              _stream(stream)), "moe_gmm_fp8")
    return out


def moe_tgmm_fp8(lhs_t, lhs_fmt, lhs_scale_inv, rhs_t, rhs_fmt, rhs_scale_inv, group_sizes,
                 M: int, out=None, out_dtype=torch.bfloat16, accumulate: bool = False,
                 valid_rows=None, err=None, stream=None):
    """out[g] (+)= sa sb lhs_t[:, cols of g] . rhs_t[:, cols of g]^T ->
    [G, Kd, N]; lhs_t [Kd, P], rhs_t [N, P] uint8 in the padded transposed
    layout of moe_fp8_quantize for M grouped rows."""
    Kd, N = lhs_t.shape[0], rhs_t.shape[0]
    G = group_sizes.numel()
    if out is None:
        out = torch.empty((G, Kd, N), dtype=out_dtype, device=lhs_t.device)
    if out.dim() != 3 or out.stride(2) != 1:
        raise MoeError("out must be [G, K, N] with unit last stride")
    _check(load().moe_tgmm_fp8(_ptr(lhs_t), _rowmajor(lhs_t, "lhs_t"), _fmt(lhs_fmt),
                               _ptr(lhs_scale_inv), _ptr(rhs_t), _rowmajor(rhs_t, "rhs_t"),
                               _fmt(rhs_fmt), _ptr(rhs_scale_inv), _ptr(group_sizes),
                               _ptr(valid_rows), G, M, Kd, N, _ptr(out), out.stride(1),
                               out.stride(0), _dtype_code(out), int(bool(accumulate)), _ptr(err),
                               _stream(stream)), "moe_tgmm_fp8")
    return out


# ------------------------------------------------------------------ SwiGLU

def _halves(h0, h1, name):
    """h0, h1: [rows, F] views with unit column stride and one common row
    stride (contiguous tensors, or the two halves of a [rows, 2F] tensor)."""
    if h0.shape != h1.shape or h0.dim() != 2:
        raise MoeError(f"{name}: both halves must be [rows, F]")
    if h0.stride(1) != 1 or h1.stride(1) != 1 or h0.stride(0) != h1.stride(0):
        raise MoeError(f"{name}: halves need unit column stride and a common row stride")
    if h0.dtype != h1.dtype:
        raise MoeError(f"{name}: halves differ in dtype")
    return h0.stride(0) if h0.shape[0] > 1 else h0.shape[1]


def moe_swiglu(h0, h1, act=None, act_dtype=None, stream=None):
    ld = _halves(h0, h1, "h")
    rows, F = h0.shape
    if act is None:
        act = torch.empty((rows, F), dtype=h0.dtype if act_dtype is None else act_dtype,
                          device=h0.device)
    _contig(act, "act")
    _check(load().moe_swiglu(_ptr(h0), _ptr(h1), _dtype_code(h0), rows, F, ld, _ptr(act),
                             _dtype_code(act), _stream(stream)), "moe_swiglu")
    return act


def moe_swiglu_bwd(h0, h1, d_act, d_h0=None, d_h1=None, stream=None):
    ld = _halves(h0, h1, "h")
    rows, F = h0.shape
    _contig(d_act, "d_act")
    if d_h0 is None:
        d_h0 = torch.empty_like(d_act)
    if d_h1 is None:
        d_h1 = torch.empty_like(d_act)
    ldd = _halves(d_h0, d_h1, "d_h")
    if d_h0.dtype != d_act.dtype:
        raise MoeError("d_h0/d_h1 must have the dtype of d_act")
    _check(load().moe_swiglu_bwd(_ptr(h0), _ptr(h1), _dtype_code(h0), ld, _ptr(d_act), rows, F,
                                 _ptr(d_h0), _ptr(d_h1), ldd, _dtype_code(d_act), _stream(stream)),
           "moe_swiglu_bwd")
    return d_h0, d_h1


# ----------------------------------------------------------------- combine

def moe_combine(y_sorted, row_of_slot, topk_w, y=None, stream=None):
    rows, D = y_sorted.shape
    T, K = topk_w.shape
    _contig(y_sorted, "y_sorted")
    if y is None:
        y = torch.empty((T, D), dtype=y_sorted.dtype, device=y_sorted.device)
    _check(load().moe_combine(_ptr(y_sorted), _dtype_code(y_sorted), T, D, K, rows,
                              _ptr(row_of_slot), _ptr(topk_w), _ptr(y), _stream(stream)),
           "moe_combine")
    return y


def moe_combine_bwd(d_y, y_sorted, row_of_slot, slot_of_row, topk_w, d_y_sorted=None,
                    d_topk_w=None, stream=None):
    rows, D = y_sorted.shape
    T, K = topk_w.shape
    _contig(d_y, "d_y")
    _contig(y_sorted, "y_sorted")
    if d_y_sorted is None:
        d_y_sorted = torch.empty_like(y_sorted)
    if d_topk_w is None:
        d_topk_w = torch.empty((T, K), dtype=torch.float32, device=d_y.device)
    _check(load().moe_combine_bwd(_ptr(d_y), _ptr(y_sorted), _dtype_code(y_sorted), T, D, K, rows,
                                  _ptr(row_of_slot), _ptr(slot_of_row), _ptr(topk_w),
                                  _ptr(d_y_sorted), _ptr(d_topk_w), _stream(stream)),
           "moe_combine_bwd")
    return d_y_sorted, d_topk_w
