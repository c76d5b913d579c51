"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the path runs in the HIP kernels.
PyTorch supplies device memory and the stream; each call passes
``tensor.data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``.  The
binding checks what the C ABI cannot see -- that every tensor is a
contiguous device tensor of the dtype and size the call implies -- and
raises :class:`MoeError` on any non-zero status.  There is no fallback: if
libmoe.so is missing, importing this module's functions fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB points the binding at another build of the same library (the host
# sanitizer run of the CPU tests uses one); default: the in-tree build.
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_HERE, "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_MISALIGNED", 4: "MOE_ERR_WORKSPACE_TOO_SMALL", 5: "MOE_ERR_HIP"}

EXPORTS = ("moe_status_string", "moe_route_workspace_size", "moe_route",
           "moe_dispatch_workspace_size", "moe_dispatch", "moe_route_dispatch_workspace_size",
           "moe_route_dispatch", "moe_route_dispatch_noalloc", "moe_route_pack_gate",
           "moe_route_prepacked", "moe_route_dispatch_prepacked",
           "moe_ep_dispatch_workspace_size", "moe_ep_dispatch",
           "moe_combine", "moe_aggregate", "moe_grouped_linear", "moe_combine_backward",
           "moe_dispatch_backward",
           "moe_route_backward_workspace_size", "moe_route_backward")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} "
                         f"({library().moe_status_string(status).decode()})")


_lib = None


def library() -> ctypes.CDLL:
    """Load libmoe.so (built by ``python -m moe_token_routing_router_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m moe_token_routing_router_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_route_workspace_size.argtypes = [i32, i32, ctypes.c_int]
        lib.moe_route_workspace_size.restype = sz
        lib.moe_route.argtypes = [P, P, P, i64, i32, i32, i32, ctypes.c_int, P, P, P, P, sz, P]
        lib.moe_route.restype = ctypes.c_int
        lib.moe_dispatch_workspace_size.argtypes = [i64, i32, i32]
        lib.moe_dispatch_workspace_size.restype = sz
        lib.moe_dispatch.argtypes = [P, P, i64, i32, i32, i32, ctypes.c_int, P, P, P, P, P, P,
                                     sz, P]
        lib.moe_dispatch.restype = ctypes.c_int
        lib.moe_route_dispatch_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.c_int]
        lib.moe_route_dispatch_workspace_size.restype = sz
        lib.moe_route_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, ctypes.c_int, P, P, P, P,
                                           P, P, P, P, sz, P]
        lib.moe_route_dispatch.restype = ctypes.c_int
        lib.moe_route_dispatch_noalloc.argtypes = [P, P, P, i64, i32, i32, i32, ctypes.c_int, P,
                                                   P, P, P, P, P, P, P]
        lib.moe_route_dispatch_noalloc.restype = ctypes.c_int
        lib.moe_route_pack_gate.argtypes = [P, i32, i32, ctypes.c_int, P, sz, P]
        lib.moe_route_pack_gate.restype = ctypes.c_int
        lib.moe_route_prepacked.argtypes = [P, P, sz, P, i64, i32, i32, i32, ctypes.c_int, P, P,
                                            P, P]
        lib.moe_route_prepacked.restype = ctypes.c_int
        lib.moe_route_dispatch_prepacked.argtypes = [P, P, sz, P, i64, i32, i32, i32,
                                                     ctypes.c_int, P, P, P, P, P, P, P, P, sz, P]
        lib.moe_route_dispatch_prepacked.restype = ctypes.c_int
        lib.moe_ep_dispatch_workspace_size.argtypes = [i64, i32, i32, i32]
        lib.moe_ep_dispatch_workspace_size.restype = sz
        lib.moe_ep_dispatch.argtypes = [P, P, i64, i32, i32, i32, i32, ctypes.c_int, P, P, P, P,
                                        P, P, P, P, P, P, P, sz, P]
        lib.moe_ep_dispatch.restype = ctypes.c_int
        lib.moe_combine.argtypes = [P, P, P, i64, i32, i32, ctypes.c_int, P, P]
        lib.moe_combine.restype = ctypes.c_int
        lib.moe_grouped_linear.argtypes = [P, P, P, i64, i32, i32, i32, ctypes.c_int, P, P]
        lib.moe_grouped_linear.restype = ctypes.c_int
        lib.moe_aggregate.argtypes = [P, P, P, P, i64, i32, i32, ctypes.c_int, P, P]
        lib.moe_aggregate.restype = ctypes.c_int
        lib.moe_combine_backward.argtypes = [P, P, P, P, i64, i32, i32, ctypes.c_int, P, P, P]
        lib.moe_combine_backward.restype = ctypes.c_int
        lib.moe_dispatch_backward.argtypes = [P, P, i64, i32, i32, ctypes.c_int, P, P]
        lib.moe_dispatch_backward.restype = ctypes.c_int
        lib.moe_route_backward_workspace_size.argtypes = [i64, i32, i32, i32, ctypes.c_int]
        lib.moe_route_backward_workspace_size.restype = sz
        lib.moe_route_backward.argtypes = [P, P, P, P, P, P, P, P, P, i64, i32, i32, i32,
                                           ctypes.c_int, P, P, P, P, sz, P]
        lib.moe_route_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


# ------------------------------------------------------------------ helpers

def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MOE_BF16
    if dt == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {dt}; expected bfloat16 or float32")


def _dev(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int,
         device: Optional[torch.device] = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


# ------------------------------------------------------------------ sizes

def moe_route_workspace_size(H: int, E: int, dtype: torch.dtype) -> int:
    return int(library().moe_route_workspace_size(H, E, _dtype_code(dtype)))


def moe_dispatch_workspace_size(N: int, E: int, K: int) -> int:
    return int(library().moe_dispatch_workspace_size(N, E, K))


def moe_route_dispatch_workspace_size(N: int, H: int, E: int, K: int, dtype: torch.dtype) -> int:
    return int(library().moe_route_dispatch_workspace_size(N, H, E, K, _dtype_code(dtype)))


def moe_ep_dispatch_workspace_size(N: int, E: int, K: int, ep_size: int) -> int:
    return int(library().moe_ep_dispatch_workspace_size(N, E, K, ep_size))


def moe_route_backward_workspace_size(N: int, H: int, E: int, K: int, dtype: torch.dtype) -> int:
    return int(library().moe_route_backward_workspace_size(N, H, E, K, _dtype_code(dtype)))


# ------------------------------------------------------------------ calls

def moe_route(x: torch.Tensor, gate_w: torch.Tensor, bias: Optional[torch.Tensor], K: int,
              topk_ids: torch.Tensor, topk_w: torch.Tensor,
              counts: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> None:
    """Router: x [N,H] @ gate_w [H,E] (+ bias [E] fp32) -> topk_ids [N,K]
    int32, topk_w [N,K] fp32, optional counts [E] int32.  workspace is a
    uint8 device tensor of at least moe_route_workspace_size(H, E, dtype)
    bytes (None when that size is 0)."""
    N, H = x.shape
    E = gate_w.shape[1]
    if gate_w.shape[0] != H:
        raise ValueError("gate_w must be [H, E]")
    dev = x.device
    dt = _dtype_code(x.dtype)
    ws = None
    ws_bytes = 0
    if workspace is not None:
        ws = _dev(workspace, "workspace", torch.uint8, workspace.numel(), dev)
        ws_bytes = workspace.numel()
    args = (_dev(x, "x", x.dtype, N * H, dev), _dev(gate_w, "gate_w", x.dtype, H * E, dev),
            _dev(bias, "bias", torch.float32, E, dev), N, H, E, K, dt,
            _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
            _dev(topk_w, "topk_w", torch.float32, N * K, dev),
            _dev(counts, "counts", torch.int32, E, dev), ws, ws_bytes, _stream(dev))
    _check("moe_route", library().moe_route(*args))


def moe_dispatch(topk_ids: torch.Tensor, x: Optional[torch.Tensor], E: int,
                 counts: torch.Tensor, offsets: torch.Tensor, perm: torch.Tensor,
                 inv: torch.Tensor, x_perm: Optional[torch.Tensor],
                 workspace: torch.Tensor, H: Optional[int] = None,
                 dtype: Optional[torch.dtype] = None) -> None:
    """Counting-sort dispatch of topk_ids [N,K]: counts [E], offsets [E+1],
    perm/inv [N*K] (int32) and, if x_perm is given, x_perm [N*K,H] rows of x.
    With x and x_perm both None, pass H and dtype explicitly."""
    N, K = topk_ids.shape
    dev = topk_ids.device
    if x is not None:
        H = x.shape[1]
        dtype = x.dtype
    if H is None or dtype is None:
        raise ValueError("H and dtype are needed when x is None")
    _check("moe_dispatch", library().moe_dispatch(
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(x, "x", dtype, N * H, dev), N, H, E, K, _dtype_code(dtype),
        _dev(counts, "counts", torch.int32, E, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev),
        _dev(perm, "perm", torch.int32, N * K, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(x_perm, "x_perm", dtype, N * K * H, dev),
        _dev(workspace, "workspace", torch.uint8, workspace.numel(), dev), workspace.numel(),
        _stream(dev)))


def moe_route_dispatch(x: torch.Tensor, gate_w: torch.Tensor, bias: Optional[torch.Tensor],
                       K: int, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                       counts: torch.Tensor, offsets: torch.Tensor, perm: torch.Tensor,
                       inv: torch.Tensor, x_perm: Optional[torch.Tensor],
                       workspace: torch.Tensor) -> None:
    """moe_route then moe_dispatch of its ids, fused (see include/moe.h)."""
    N, H = x.shape
    E = gate_w.shape[1]
    if gate_w.shape[0] != H:
        raise ValueError("gate_w must be [H, E]")
    dev = x.device
    _check("moe_route_dispatch", library().moe_route_dispatch(
        _dev(x, "x", x.dtype, N * H, dev), _dev(gate_w, "gate_w", x.dtype, H * E, dev),
        _dev(bias, "bias", torch.float32, E, dev), N, H, E, K, _dtype_code(x.dtype),
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev),
        _dev(counts, "counts", torch.int32, E, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev),
        _dev(perm, "perm", torch.int32, N * K, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(x_perm, "x_perm", x.dtype, N * K * H, dev),
        _dev(workspace, "workspace", torch.uint8, workspace.numel(), dev), workspace.numel(),
        _stream(dev)))


def moe_route_dispatch_noalloc(x: torch.Tensor, gate_w: torch.Tensor,
                               bias: Optional[torch.Tensor], K: int, topk_ids: torch.Tensor,
                               topk_w: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor,
                               perm: torch.Tensor, inv: torch.Tensor,
                               x_perm: Optional[torch.Tensor]) -> None:
    """moe_route_dispatch with the library's built-in per-GPU workspace
    (no workspace argument, no allocation; see include/moe.h).  Calls that
    may overlap on one GPU race on that workspace."""
    N, H = x.shape
    E = gate_w.shape[1]
    if gate_w.shape[0] != H:
        raise ValueError("gate_w must be [H, E]")
    dev = x.device
    if torch.cuda.current_device() != dev.index:
        raise ValueError(f"the current device ({torch.cuda.current_device()}) is not {dev}")
    _check("moe_route_dispatch_noalloc", library().moe_route_dispatch_noalloc(
        _dev(x, "x", x.dtype, N * H, dev), _dev(gate_w, "gate_w", x.dtype, H * E, dev),
        _dev(bias, "bias", torch.float32, E, dev), N, H, E, K, _dtype_code(x.dtype),
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev),
        _dev(counts, "counts", torch.int32, E, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev),
        _dev(perm, "perm", torch.int32, N * K, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(x_perm, "x_perm", x.dtype, N * K * H, dev), _stream(dev)))


def moe_ep_dispatch(topk_ids: torch.Tensor, x: Optional[torch.Tensor], E: int, ep_size: int,
                    counts: torch.Tensor, offsets: torch.Tensor, perm: torch.Tensor,
                    inv: torch.Tensor, send_counts: torch.Tensor, send_offsets: torch.Tensor,
                    send_tok: torch.Tensor, send_row: torch.Tensor, expand_idx: torch.Tensor,
                    x_send: Optional[torch.Tensor], workspace: torch.Tensor,
                    H: Optional[int] = None, dtype: Optional[torch.dtype] = None) -> None:
    """Expert-parallel send metadata of topk_ids [N,K] for ep_size ranks
    (see include/moe.h); x_send [N*min(K,ep_size), H] rows of x if given."""
    N, K = topk_ids.shape
    dev = topk_ids.device
    if x is not None:
        H = x.shape[1]
        dtype = x.dtype
    if H is None or dtype is None:
        raise ValueError("H and dtype are needed when x is None")
    cap = N * min(K, ep_size)
    _check("moe_ep_dispatch", library().moe_ep_dispatch(
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(x, "x", dtype, N * H, dev), N, H, E, K, ep_size, _dtype_code(dtype),
        _dev(counts, "counts", torch.int32, E, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev),
        _dev(perm, "perm", torch.int32, N * K, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(send_counts, "send_counts", torch.int32, ep_size, dev),
        _dev(send_offsets, "send_offsets", torch.int32, ep_size + 1, dev),
        _dev(send_tok, "send_tok", torch.int32, cap, dev),
        _dev(send_row, "send_row", torch.int32, N * K, dev),
        _dev(expand_idx, "expand_idx", torch.int32, N * K, dev),
        _dev(x_send, "x_send", dtype, cap * H, dev),
        _dev(workspace, "workspace", torch.uint8, workspace.numel(), dev), workspace.numel(),
        _stream(dev)))


def moe_combine(y: torch.Tensor, inv: torch.Tensor, topk_w: torch.Tensor,
                out: torch.Tensor) -> None:
    """Weighted combine: out [N,H] = sum_k topk_w[n,k] * y[inv[n*K+k]], with
    y [N*K,H] in dispatched order."""
    N, K = topk_w.shape
    H = y.shape[1]
    dev = y.device
    _check("moe_combine", library().moe_combine(
        _dev(y, "y", y.dtype, N * K * H, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev), N, H, K, _dtype_code(y.dtype),
        _dev(out, "out", y.dtype, N * H, dev), _stream(dev)))


def moe_aggregate(y: torch.Tensor, inv: torch.Tensor, topk_w: torch.Tensor,
                  residual: torch.Tensor, out: torch.Tensor) -> None:
    """forward_aggregate: out [N,H] = sum_k topk_w[n,k] * y[inv[n*K+k]] + residual."""
    N, K = topk_w.shape
    H = y.shape[1]
    dev = y.device
    _check("moe_aggregate", library().moe_aggregate(
        _dev(y, "y", y.dtype, N * K * H, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev),
        _dev(residual, "residual", y.dtype, N * H, dev), N, H, K, _dtype_code(y.dtype),
        _dev(out, "out", y.dtype, N * H, dev), _stream(dev)))


def moe_grouped_linear(x_perm: torch.Tensor, weight: torch.Tensor, offsets: torch.Tensor,
                       y: torch.Tensor) -> None:
    """Expert layer: y[p] = weight[e] @ x_perm[p] for the rows of expert e's
    segment (offsets); weight [E,F,H]."""
    T, H = x_perm.shape
    E, F, H2 = weight.shape
    if H2 != H:
        raise ValueError("weight must be [E, F, H]")
    dev = x_perm.device
    dt = x_perm.dtype
    _check("moe_grouped_linear", library().moe_grouped_linear(
        _dev(x_perm, "x_perm", dt, T * H, dev), _dev(weight, "weight", dt, E * F * H, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev), T, H, E, F, _dtype_code(dt),
        _dev(y, "y", dt, T * F, dev), _stream(dev)))


def moe_combine_backward(dout: torch.Tensor, y: torch.Tensor, inv: torch.Tensor,
                         topk_w: torch.Tensor, dy: torch.Tensor, dtopk_w: torch.Tensor) -> None:
    """Gradient of moe_combine: dy [N*K,H] (dispatched order), dtopk_w [N,K]."""
    N, K = topk_w.shape
    H = dout.shape[1]
    dev = dout.device
    _check("moe_combine_backward", library().moe_combine_backward(
        _dev(dout, "dout", dout.dtype, N * H, dev), _dev(y, "y", dout.dtype, N * K * H, dev),
        _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev), N, H, K, _dtype_code(dout.dtype),
        _dev(dy, "dy", dout.dtype, N * K * H, dev),
        _dev(dtopk_w, "dtopk_w", torch.float32, N * K, dev), _stream(dev)))


def moe_dispatch_backward(dx_perm: torch.Tensor, inv: torch.Tensor, dx: torch.Tensor) -> None:
    """Gradient of the dispatch row copy: dx [N,H] = sum_k dx_perm[inv[n*K+k]]."""
    N, H = dx.shape
    T = inv.numel()
    if N and T % N:
        raise ValueError("inv must hold N*K entries")
    K = T // N if N else 1
    dev = dx.device
    _check("moe_dispatch_backward", library().moe_dispatch_backward(
        _dev(dx_perm, "dx_perm", dx.dtype, T * H, dev), _dev(inv, "inv", torch.int32, T, dev),
        N, H, K, _dtype_code(dx.dtype), _dev(dx, "dx", dx.dtype, N * H, dev), _stream(dev)))


def moe_route_backward(x_perm: torch.Tensor, gate_w: torch.Tensor, topk_ids: torch.Tensor,
                       topk_w: torch.Tensor, dtopk_w: torch.Tensor, perm: torch.Tensor,
                       offsets: torch.Tensor, inv: Optional[torch.Tensor],
                       dx_perm: Optional[torch.Tensor], dgate_w: torch.Tensor,
                       dbias: Optional[torch.Tensor], dx: torch.Tensor,
                       workspace: torch.Tensor) -> None:
    """Gradient of moe_route's weights (ids fixed) with respect to gate_w,
    bias and x, plus the dispatch backward of dx_perm (see include/moe.h)."""
    N, K = topk_ids.shape
    H, E = gate_w.shape
    dev = gate_w.device
    dt = gate_w.dtype
    _check("moe_route_backward", library().moe_route_backward(
        _dev(x_perm, "x_perm", dt, N * K * H, dev), _dev(gate_w, "gate_w", dt, H * E, dev),
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev),
        _dev(dtopk_w, "dtopk_w", torch.float32, N * K, dev),
        _dev(perm, "perm", torch.int32, N * K, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev),
        _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(dx_perm, "dx_perm", dt, N * K * H, dev), N, H, E, K, _dtype_code(dt),
        _dev(dgate_w, "dgate_w", torch.float32, H * E, dev),
        _dev(dbias, "dbias", torch.float32, E, dev), _dev(dx, "dx", dt, N * H, dev),
        _dev(workspace, "workspace", torch.uint8, workspace.numel(), dev), workspace.numel(),
        _stream(dev)))


def _packed_gate(packed_gate: torch.Tensor, H: int, E: int, dtype: torch.dtype,
                 dev: torch.device):
    """The packed gate of moe_route_pack_gate: uint8 of the packed size, or
    gate_w itself ([H, E] of the tokens' dtype) when that size is 0."""
    n = moe_route_workspace_size(H, E, dtype)
    if n:
        return _dev(packed_gate, "packed_gate", torch.uint8, n, dev)
    return _dev(packed_gate, "packed_gate (gate_w itself at this size)", dtype, H * E, dev)


def moe_route_pack_gate(gate_w: torch.Tensor, packed: Optional[torch.Tensor]) -> None:
    """Re-lay gate_w [H,E] out once for the prepacked router calls into
    packed (uint8, moe_route_workspace_size(H, E, dtype) bytes; None when
    that size is 0: then the packed gate is gate_w itself)."""
    H, E = gate_w.shape
    dev = gate_w.device
    n = moe_route_workspace_size(H, E, gate_w.dtype)
    _check("moe_route_pack_gate", library().moe_route_pack_gate(
        _dev(gate_w, "gate_w", gate_w.dtype, H * E, dev), H, E, _dtype_code(gate_w.dtype),
        _dev(packed, "packed", torch.uint8, n, dev) if n else None, n, _stream(dev)))


def moe_route_prepacked(x: torch.Tensor, packed_gate: torch.Tensor, E: int,
                        bias: Optional[torch.Tensor], K: int, topk_ids: torch.Tensor,
                        topk_w: torch.Tensor, counts: Optional[torch.Tensor] = None) -> None:
    """moe_route with the gate packed by moe_route_pack_gate (no workspace)."""
    N, H = x.shape
    dev = x.device
    _check("moe_route_prepacked", library().moe_route_prepacked(
        _dev(x, "x", x.dtype, N * H, dev), _packed_gate(packed_gate, H, E, x.dtype, dev),
        packed_gate.numel() * packed_gate.element_size(), _dev(bias, "bias", torch.float32, E, dev), N, H, E, K, _dtype_code(x.dtype),
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev),
        _dev(counts, "counts", torch.int32, E, dev), _stream(dev)))


def moe_route_dispatch_prepacked(x: torch.Tensor, packed_gate: torch.Tensor, E: int,
                                 bias: Optional[torch.Tensor], K: int, topk_ids: torch.Tensor,
                                 topk_w: torch.Tensor, counts: torch.Tensor,
                                 offsets: torch.Tensor, perm: torch.Tensor, inv: torch.Tensor,
                                 x_perm: Optional[torch.Tensor], workspace: torch.Tensor) -> None:
    """moe_route_dispatch with the gate packed by moe_route_pack_gate."""
    N, H = x.shape
    dev = x.device
    _check("moe_route_dispatch_prepacked", library().moe_route_dispatch_prepacked(
        _dev(x, "x", x.dtype, N * H, dev), _packed_gate(packed_gate, H, E, x.dtype, dev),
        packed_gate.numel() * packed_gate.element_size(), _dev(bias, "bias", torch.float32, E, dev), N, H, E, K, _dtype_code(x.dtype),
        _dev(topk_ids, "topk_ids", torch.int32, N * K, dev),
        _dev(topk_w, "topk_w", torch.float32, N * K, dev),
        _dev(counts, "counts", torch.int32, E, dev),
        _dev(offsets, "offsets", torch.int32, E + 1, dev),
        _dev(perm, "perm", torch.int32, N * K, dev), _dev(inv, "inv", torch.int32, N * K, dev),
        _dev(x_perm, "x_perm", x.dtype, N * K * H, dev),
        _dev(workspace, "workspace", torch.uint8, workspace.numel(), dev), workspace.numel(),
        _stream(dev)))


# ------------------------------------------------------- allocating forms

def pack_gate(gate_w: torch.Tensor) -> torch.Tensor:
    """The packed gate for the prepacked router calls (a new uint8 tensor,
    or gate_w itself where the router reads the gate as it is)."""
    H, E = gate_w.shape
    n = moe_route_workspace_size(H, E, gate_w.dtype)
    if not n:
        moe_route_pack_gate(gate_w, None)
        return gate_w
    packed = torch.empty((n,), dtype=torch.uint8, device=gate_w.device)
    moe_route_pack_gate(gate_w, packed)
    return packed


def route_prepacked(x: torch.Tensor, packed_gate: torch.Tensor, E: int, K: int,
                    bias: Optional[torch.Tensor] = None, with_counts: bool = False):
    """Allocate outputs and run moe_route_prepacked; returns (ids, w, counts-or-None)."""
    N = x.shape[0]
    ids = torch.empty((N, K), dtype=torch.int32, device=x.device)
    w = torch.empty((N, K), dtype=torch.float32, device=x.device)
    counts = torch.empty((E,), dtype=torch.int32, device=x.device) if with_counts else None
    moe_route_prepacked(x, packed_gate, E, bias, K, ids, w, counts)
    return ids, w, counts


def route_dispatch_prepacked(x: torch.Tensor, packed_gate: torch.Tensor, E: int, K: int,
                             bias: Optional[torch.Tensor] = None, with_rows: bool = True):
    """Allocate outputs and run moe_route_dispatch_prepacked; returns
    (ids, w, counts, offsets, perm, inv, x_perm-or-None)."""
    N, H = x.shape
    dev = x.device
    ids = torch.empty((N, K), dtype=torch.int32, device=dev)
    w = torch.empty((N, K), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((N * K,), dtype=torch.int32, device=dev)
    inv = torch.empty((N * K,), dtype=torch.int32, device=dev)
    x_perm = torch.empty((N * K, H), dtype=x.dtype, device=dev) if with_rows else None
    ws = torch.empty((max(1, moe_route_dispatch_workspace_size(N, H, E, K, x.dtype)),),
                     dtype=torch.uint8, device=dev)
    moe_route_dispatch_prepacked(x, packed_gate, E, bias, K, ids, w, counts, offsets, perm, inv,
                                 x_perm, ws)
    return ids, w, counts, offsets, perm, inv, x_perm


def route(x: torch.Tensor, gate_w: torch.Tensor, K: int, bias: Optional[torch.Tensor] = None,
          with_counts: bool = False):
    """Allocate outputs and run moe_route; returns (ids, w, counts-or-None)."""
    N, H = x.shape
    E = gate_w.shape[1]
    ids = torch.empty((N, K), dtype=torch.int32, device=x.device)
    w = torch.empty((N, K), dtype=torch.float32, device=x.device)
    counts = torch.empty((E,), dtype=torch.int32, device=x.device) if with_counts else None
    nws = moe_route_workspace_size(H, E, x.dtype)
    ws = torch.empty((nws,), dtype=torch.uint8, device=x.device) if nws else None
    moe_route(x, gate_w, bias, K, ids, w, counts, ws)
    return ids, w, counts


def dispatch(topk_ids: torch.Tensor, x: Optional[torch.Tensor], E: int, with_rows: bool = True):
    """Allocate outputs and run moe_dispatch; returns
    (counts, offsets, perm, inv, x_perm-or-None)."""
    N, K = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((N * K,), dtype=torch.int32, device=dev)
    inv = torch.empty((N * K,), dtype=torch.int32, device=dev)
    x_perm = None
    if with_rows:
        x_perm = torch.empty((N * K, x.shape[1]), dtype=x.dtype, device=dev)
    ws = torch.empty((moe_dispatch_workspace_size(N, E, K),), dtype=torch.uint8, device=dev)
    moe_dispatch(topk_ids, x, E, counts, offsets, perm, inv, x_perm, ws,
                 H=None if x is not None else 8, dtype=None if x is not None else torch.bfloat16)
    return counts, offsets, perm, inv, x_perm


def route_dispatch(x: torch.Tensor, gate_w: torch.Tensor, K: int,
                   bias: Optional[torch.Tensor] = None, with_rows: bool = True):
    """Allocate outputs and run moe_route_dispatch; returns
    (ids, w, counts, offsets, perm, inv, x_perm-or-None)."""
    N, H = x.shape
    E = gate_w.shape[1]
    dev = x.device
    ids = torch.empty((N, K), dtype=torch.int32, device=dev)
    w = torch.empty((N, K), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((N * K,), dtype=torch.int32, device=dev)
    inv = torch.empty((N * K,), dtype=torch.int32, device=dev)
    x_perm = torch.empty((N * K, H), dtype=x.dtype, device=dev) if with_rows else None
    ws = torch.empty((max(1, moe_route_dispatch_workspace_size(N, H, E, K, x.dtype)),),
                     dtype=torch.uint8, device=dev)
    moe_route_dispatch(x, gate_w, bias, K, ids, w, counts, offsets, perm, inv, x_perm, ws)
    return ids, w, counts, offsets, perm, inv, x_perm


def ep_dispatch(topk_ids: torch.Tensor, x: Optional[torch.Tensor], E: int, ep_size: int,
                with_rows: bool = True):
    """Allocate outputs and run moe_ep_dispatch; returns (counts, offsets,
    perm, inv, send_counts, send_offsets, send_tok, send_row, expand_idx,
    x_send-or-None); send_tok and x_send have N*min(K, ep_size) rows, of
    which the first send_offsets[ep_size] are written."""
    N, K = topk_ids.shape
    dev = topk_ids.device
    cap = N * min(K, ep_size)
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.empty((E,), **i32), torch.empty((E + 1,), **i32)
    perm, inv = torch.empty((N * K,), **i32), torch.empty((N * K,), **i32)
    send_counts, send_offsets = torch.empty((ep_size,), **i32), torch.empty((ep_size + 1,), **i32)
    send_tok = torch.empty((cap,), **i32)
    send_row, expand_idx = torch.empty((N * K,), **i32), torch.empty((N * K,), **i32)
    x_send = torch.empty((cap, x.shape[1]), dtype=x.dtype, device=dev) if with_rows else None
    ws = torch.empty((max(1, moe_ep_dispatch_workspace_size(N, E, K, ep_size)),),
                     dtype=torch.uint8, device=dev)
    moe_ep_dispatch(topk_ids, x if with_rows else None, E, ep_size, counts, offsets, perm, inv,
                    send_counts, send_offsets, send_tok, send_row, expand_idx, x_send, ws,
                    H=None if with_rows else 8, dtype=None if with_rows else torch.bfloat16)
    return (counts, offsets, perm, inv, send_counts, send_offsets, send_tok, send_row,
            expand_idx, x_send)


def combine(y: torch.Tensor, inv: torch.Tensor, topk_w: torch.Tensor) -> torch.Tensor:
    """Allocate the output and run moe_combine."""
    N = topk_w.shape[0]
    out = torch.empty((N, y.shape[1]), dtype=y.dtype, device=y.device)
    moe_combine(y, inv, topk_w, out)
    return out


def combine_backward(dout: torch.Tensor, y: torch.Tensor, inv: torch.Tensor,
                     topk_w: torch.Tensor):
    """Allocate and run moe_combine_backward; returns (dy, dtopk_w)."""
    dy = torch.empty_like(y)
    dw = torch.empty_like(topk_w)
    moe_combine_backward(dout, y, inv, topk_w, dy, dw)
    return dy, dw


def dispatch_backward(dx_perm: torch.Tensor, inv: torch.Tensor, N: int) -> torch.Tensor:
    """Allocate and run moe_dispatch_backward; returns dx [N,H]."""
    dx = torch.empty((N, dx_perm.shape[1]), dtype=dx_perm.dtype, device=dx_perm.device)
    moe_dispatch_backward(dx_perm, inv, dx)
    return dx


def route_backward(x_perm: torch.Tensor, gate_w: torch.Tensor, topk_ids: torch.Tensor,
                   topk_w: torch.Tensor, dtopk_w: torch.Tensor, perm: torch.Tensor,
                   offsets: torch.Tensor, inv: Optional[torch.Tensor] = None,
                   dx_perm: Optional[torch.Tensor] = None, with_bias: bool = True):
    """Allocate and run moe_route_backward; returns (dgate_w, dbias-or-None, dx)."""
    N, K = topk_ids.shape
    H, E = gate_w.shape
    dev = gate_w.device
    dgate_w = torch.empty((H, E), dtype=torch.float32, device=dev)
    dbias = torch.empty((E,), dtype=torch.float32, device=dev) if with_bias else None
    dx = torch.empty((N, H), dtype=gate_w.dtype, device=dev)
    ws = torch.empty((max(1, moe_route_backward_workspace_size(N, H, E, K, gate_w.dtype)),),
                     dtype=torch.uint8, device=dev)
    moe_route_backward(x_perm, gate_w, topk_ids, topk_w, dtopk_w, perm, offsets, inv, dx_perm,
                       dgate_w, dbias, dx, ws)
    return dgate_w, dbias, dx


def aggregate(y: torch.Tensor, inv: torch.Tensor, topk_w: torch.Tensor,
              residual: torch.Tensor) -> torch.Tensor:
    """Allocate the output and run moe_aggregate."""
    out = torch.empty_like(residual)
    moe_aggregate(y, inv, topk_w, residual, out)
    return out


def grouped_linear(x_perm: torch.Tensor, weight: torch.Tensor,
                   offsets: torch.Tensor) -> torch.Tensor:
    """Allocate y [T,F] (zero-filled: rows past offsets[E] are not written)
    and run moe_grouped_linear."""
    y = torch.zeros((x_perm.shape[0], weight.shape[1]), dtype=x_perm.dtype, device=x_perm.device)
    moe_grouped_linear(x_perm, weight, offsets, y)
    return y
