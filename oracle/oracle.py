"""numpy front end of the C oracle (test infrastructure only).

Arrays are passed to oracle.c by pointer; all arithmetic happens there, in
IEEE double.  bf16 tensors travel as their raw uint16 bit patterns, fp32 as
float32.  See oracle.c for the definitions and the pages they follow:
  route    - moe-engine page, "Fused Triton routing kernel" section
  dispatch - PithTrain page, section 8.2 (counting sort instead of argsort)
  ep_dispatch - the same section: per-rank counts, send metadata, dedup
  *_backward - the gradients of route, dispatch and combine (training runs
               the stages backward; PithTrain page, section 6.2)
  aggregate - forward_aggregate: weighted expert output + residual (6.1)
  grouped_linear - one linear map per expert over the dispatched rows (the
               expert layer between dispatch and combine, 6.1 forward_mlp)
  combine  - PithTrain page, section 6.1 (forward_aggregate)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB lets the mutation test load a deliberately broken build of
# oracle.c to show that the pins catch it.
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPES = {"f32": 0, "bf16": 1}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_route.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_dispatch.argtypes = [P, i64, i32, i32, P, P, P, P]
        lib.oracle_dispatch.restype = ctypes.c_int
        lib.oracle_ep_dispatch.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P]
        lib.oracle_ep_dispatch.restype = ctypes.c_int
        lib.oracle_permute_rows.argtypes = [P, i64, i32, i64, P, P]
        lib.oracle_permute_rows.restype = ctypes.c_int
        lib.oracle_combine.argtypes = [P, P, P, i64, i32, i32, i32, P]
        lib.oracle_combine.restype = ctypes.c_int
        lib.oracle_combine_backward.argtypes = [P, P, P, P, i64, i32, i32, i32, P, P]
        lib.oracle_combine_backward.restype = ctypes.c_int
        lib.oracle_dispatch_backward.argtypes = [P, P, i64, i32, i32, i32, P]
        lib.oracle_dispatch_backward.restype = ctypes.c_int
        lib.oracle_route_backward.argtypes = [P, P, P, P, P, P, P, i64, i32, i32, i32, i32,
                                              P, P, P, P]
        lib.oracle_route_backward.restype = ctypes.c_int
        lib.oracle_aggregate.argtypes = [P, P, P, P, i64, i32, i32, i32, P]
        lib.oracle_aggregate.restype = ctypes.c_int
        lib.oracle_grouped_linear.argtypes = [P, P, P, i32, i32, i32, i32, P, i64, P]
        lib.oracle_grouped_linear.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_set_threads.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [dbl]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = dbl
        _lib = lib
    return _lib



def set_threads(n):
    """Threads for the token loops of route and combine (default 1).  Tokens
    are independent and each is computed the same way, so results do not
    depend on n; only the CPU baseline's timing uses more than one."""
    return int(_load().oracle_set_threads(int(n)))

def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(a, dtype):
    want = np.uint16 if dtype == "bf16" else np.float32
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be passed as {want.__name__}, got {a.dtype}")
    return a


def route(x, gate_w, bias, K, dtype):
    """Router: logits, top-K ids, renormalised weights, K-th/(K+1)-th margin.

    x [N,H], gate_w [H,E] in `dtype` storage; bias [E] float32 or None.
    Returns (ids int32 [N,K], w float32 [N,K], logits float64 [N,E],
    margin float64 [N]).
    """
    x = _storage(x, dtype)
    gate_w = _storage(gate_w, dtype)
    N, H = x.shape
    H2, E = gate_w.shape
    if H2 != H:
        raise ValueError("gate_w must be [H, E]")
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (E,):
            raise ValueError("bias must be [E]")
    ids = np.empty((N, K), np.int32)
    w = np.empty((N, K), np.float32)
    logits = np.empty((N, E), np.float64)
    margin = np.empty((N,), np.float64)
    rc = _load().oracle_route(_ptr(x), _ptr(gate_w), _ptr(bias), N, H, E, K,
                              DTYPES[dtype], _ptr(ids), _ptr(w), _ptr(logits),
                              _ptr(margin))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    return ids, w, logits, margin


def dispatch(ids, E):
    """Counting-sort dispatch metadata.

    ids int32 [N,K].  Returns (counts [E], offsets [E+1], perm [N*K],
    inv [N*K]), all int32; perm maps dispatched row -> flat slot n*K+k and
    inv maps slot -> row.
    """
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, K = ids.shape
    counts = np.empty((E,), np.int32)
    offsets = np.empty((E + 1,), np.int32)
    perm = np.empty((N * K,), np.int32)
    inv = np.empty((N * K,), np.int32)
    rc = _load().oracle_dispatch(_ptr(ids), N, K, E, _ptr(counts), _ptr(offsets),
                                 _ptr(perm), _ptr(inv))
    if rc != 0:
        raise ValueError("oracle_dispatch rejected its arguments")
    return counts, offsets, perm, inv


def ep_dispatch(ids, E, R):
    """Expert-parallel send metadata with per-(token, rank) deduplication.

    ids int32 [N,K]; R ranks of E/R experts each.  Returns (send_counts [R],
    send_offsets [R+1], send_tok [S], send_row [N*K], expand_idx [N*K]), all
    int32, S = send_offsets[R] (see oracle_ep_dispatch for the definitions).
    """
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    N, K = ids.shape
    T = N * K
    send_counts = np.empty((R,), np.int32)
    send_offsets = np.empty((R + 1,), np.int32)
    send_tok = np.empty((max(T, 1),), np.int32)
    send_row = np.empty((T,), np.int32)
    expand_idx = np.empty((T,), np.int32)
    rc = _load().oracle_ep_dispatch(_ptr(ids), N, K, E, R, _ptr(send_counts),
                                    _ptr(send_offsets), _ptr(send_tok), _ptr(send_row),
                                    _ptr(expand_idx))
    if rc != 0:
        raise ValueError("oracle_ep_dispatch rejected its arguments")
    return send_counts, send_offsets, send_tok[:send_offsets[R]].copy(), send_row, expand_idx


def permute_rows(x, perm, K):
    """x_perm[r] = x[perm[r] // K], a byte copy; x is any 2-D array."""
    x = np.ascontiguousarray(x)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    N = x.shape[0]
    out = np.empty((perm.shape[0],) + x.shape[1:], x.dtype)
    rc = _load().oracle_permute_rows(_ptr(x), N, K, x[0:1].nbytes if N else 1,
                                     _ptr(perm), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_permute_rows rejected its arguments")
    return out


def combine(y, inv, w, dtype):
    """Weighted combine: out[n] = sum_k w[n,k] * y[inv[n*K+k]], rounded once.

    y [N*K, H] in `dtype` storage, inv int32 [N*K], w float32 [N,K].
    Returns out [N,H] in `dtype` storage.
    """
    y = _storage(y, dtype)
    w = np.ascontiguousarray(w, dtype=np.float32)
    inv = np.ascontiguousarray(inv, dtype=np.int32)
    N, K = w.shape
    H = y.shape[1]
    if y.shape[0] != N * K or inv.shape != (N * K,):
        raise ValueError("y must be [N*K, H] and inv [N*K]")
    out = np.empty((N, H), y.dtype)
    rc = _load().oracle_combine(_ptr(y), _ptr(inv), _ptr(w), N, H, K,
                                DTYPES[dtype], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_combine rejected its arguments")
    return out


def round_bf16(v):
    """One-step nearest-even rounding of a Python float to bf16 bits."""
    return int(_load().oracle_round_bf16(float(v)))


def decode_bf16(bits):
    """bf16 bit pattern -> float (exact)."""
    return float(_load().oracle_decode_bf16(int(bits)))


def combine_backward(dout, y, inv, w, dtype):
    """Gradient of the combine: (dy [N*K,H] in `dtype` storage, rows in
    dispatched order; dw [N,K] float32)."""
    dout = _storage(dout, dtype)
    y = _storage(y, dtype)
    inv = np.ascontiguousarray(inv, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    H = dout.shape[1]
    dy = np.empty((N * K, H), dout.dtype)
    dw = np.empty((N, K), np.float32)
    rc = _load().oracle_combine_backward(_ptr(dout), _ptr(y), _ptr(inv), _ptr(w), N, H, K,
                                         DTYPES[dtype], _ptr(dy), _ptr(dw))
    if rc != 0:
        raise ValueError("oracle_combine_backward rejected its arguments")
    return dy, dw


def dispatch_backward(dx_perm, inv, K, dtype):
    """Gradient of the row dispatch: dx [N,H] = sum_k dx_perm[inv[n*K+k]]."""
    dx_perm = _storage(dx_perm, dtype)
    inv = np.ascontiguousarray(inv, dtype=np.int32)
    N = inv.shape[0] // K
    H = dx_perm.shape[1]
    dx = np.empty((N, H), dx_perm.dtype)
    rc = _load().oracle_dispatch_backward(_ptr(dx_perm), _ptr(inv), N, H, K, DTYPES[dtype],
                                          _ptr(dx))
    if rc != 0:
        raise ValueError("oracle_dispatch_backward rejected its arguments")
    return dx


def route_backward(x, gate_w, bias, ids, dw, dx_perm, inv, dtype):
    """Gradient of the router weights (fixed selection ids) with respect to
    gate_w, bias and x, plus the dispatch backward of dx_perm (or None).
    Returns (dlogits [N,E] float64, dgate_w [H,E] float32, dbias [E]
    float32, dx [N,H] in `dtype` storage)."""
    x = _storage(x, dtype)
    gate_w = _storage(gate_w, dtype)
    N, H = x.shape
    E = gate_w.shape[1]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    K = ids.shape[1]
    dw = np.ascontiguousarray(dw, dtype=np.float32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    if dx_perm is not None:
        dx_perm = _storage(dx_perm, dtype)
        inv = np.ascontiguousarray(inv, dtype=np.int32)
    dlogits = np.empty((N, E), np.float64)
    dgate_w = np.empty((H, E), np.float32)
    dbias = np.empty((E,), np.float32)
    dx = np.empty((N, H), x.dtype)
    rc = _load().oracle_route_backward(_ptr(x), _ptr(gate_w), _ptr(bias), _ptr(ids), _ptr(dw),
                                       _ptr(dx_perm), _ptr(inv if dx_perm is not None else None),
                                       N, H, E, K, DTYPES[dtype], _ptr(dlogits),
                                       _ptr(dgate_w), _ptr(dbias), _ptr(dx))
    if rc != 0:
        raise ValueError("oracle_route_backward rejected its arguments")
    return dlogits, dgate_w, dbias, dx


def aggregate(y, inv, w, residual, dtype):
    """forward_aggregate: the weighted expert output plus the residual [N,H]."""
    y = _storage(y, dtype)
    residual = _storage(residual, dtype)
    inv = np.ascontiguousarray(inv, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    H = y.shape[1]
    out = np.empty((N, H), y.dtype)
    rc = _load().oracle_aggregate(_ptr(y), _ptr(inv), _ptr(w), _ptr(residual), N, H, K,
                                  DTYPES[dtype], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_aggregate rejected its arguments")
    return out


def grouped_linear(x_perm, weight, offsets, dtype, rows=None):
    """One linear map per expert over its dispatched rows: y[p] =
    weight[e] @ x_perm[p] for offsets[e] <= p < offsets[e+1]; weight
    [E,F,H].  With rows given, only those rows are computed (y [len(rows),F])."""
    x_perm = _storage(x_perm, dtype)
    weight = _storage(weight, dtype)
    E, F, H = weight.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
    n = len(rows) if rows is not None else int(offsets[E])
    y = np.empty((n, F), x_perm.dtype)
    rc = _load().oracle_grouped_linear(_ptr(x_perm), _ptr(weight), _ptr(offsets), E, H, F,
                                       DTYPES[dtype], _ptr(rows), n, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_grouped_linear rejected its arguments")
    return y
