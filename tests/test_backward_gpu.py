"""Backward of the path, HIP vs the CPU oracle, through the C ABI, on the GPU.

The forward's routing (ids, weights) and dispatch metadata come from the
oracle, so every call is compared on the same selection.  Upstream gradients
are seeded synthetic arrays of the workload's shapes.

Rules:
  * dy of the combine backward: bit for bit (w * dout rounded once, exactly);
  * dtopk_w: |gpu - ref| <= 1e-5 * S + 1e-6 with S[n,k] = sum_h |dout * y|
    (fp32 accumulation over H products);
  * dx (dispatch and router backward): the combine rule, 1e-2 * |ref| + 1e-4
    for bf16 (one bf16 rounding), 1e-5 * |ref| + 1e-6 for fp32;
  * dgate_w, dbias: |gpu - ref| <= 1e-4 * S + 1e-7 with S the same sums over
    absolute values (fp32 accumulation in chunks, then over the chunks).
"""
import numpy as np
import pytest
import torch

from moe_token_routing_router_amd import _lib as L
from moe_token_routing_router_amd import inputs as I
from oracle import oracle as O
from tests.parity import (check_combine, check_sum_tight, decode, from_dev, sum_of_abs_terms,
                          to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.library()


def _case(d):
    """Oracle forward (ids, w, dispatch) and seeded upstream gradients."""
    N, H, E, K, dt = d["N"], d["H"], d["E"], d["K"], d["dtype"]
    ids, w, _, _ = O.route(d["x"], d["gate_w"], d["bias"], K, dt)
    counts, offsets, perm, inv = O.dispatch(ids, E)
    rng = np.random.default_rng(1000 + N + H)
    dout = d["y"][:N] if len(d["y"]) >= N else d["x"]
    dw = rng.standard_normal((N, K)).astype(np.float32)
    return dict(ids=ids, w=w, offsets=offsets, perm=perm, inv=inv, dout=dout, dw=dw)


def _abs_dot(a, b_rows, dtype, chunk=2048):
    """sum_h |a[n,h] * b[n,k,h]| for the tolerance scale, in row chunks."""
    N = a.shape[0]
    out = []
    for s in range(0, N, chunk):
        aa = np.abs(decode(a[s:s + chunk], dtype))
        bb = np.abs(decode(b_rows[s:s + chunk], dtype))
        out.append(np.einsum("nh,nkh->nk", aa, bb))
    return np.concatenate(out) if out else np.zeros((0, b_rows.shape[1]))


def _check_combine_backward(d, c):
    N, H, K, dt = d["N"], d["H"], d["K"], d["dtype"]
    dy, dwt = L.combine_backward(to_dev(c["dout"], dt), to_dev(d["y"], dt),
                                 torch.from_numpy(c["inv"]).cuda(), torch.from_numpy(c["w"]).cuda())
    torch.cuda.synchronize()
    rdy, rdw = O.combine_backward(c["dout"], d["y"], c["inv"], c["w"], dt)
    np.testing.assert_array_equal(from_dev(dy), rdy)
    S = _abs_dot(c["dout"], d["y"][c["inv"].reshape(N, K)], dt)
    err = np.abs(from_dev(dwt).astype(np.float64) - rdw)
    assert (err <= 1e-5 * S + 1e-6).all(), f"dtopk_w error {err.max()}"


def _check_route_backward(d, c, with_dx_perm=True):
    N, H, E, K, dt = d["N"], d["H"], d["E"], d["K"], d["dtype"]
    x_perm = O.permute_rows(d["x"], c["perm"], K)
    dx_perm = d["y"] if with_dx_perm else None
    dg, db, dx = L.route_backward(
        to_dev(x_perm, dt), to_dev(d["gate_w"], dt), torch.from_numpy(c["ids"]).cuda(),
        torch.from_numpy(c["w"]).cuda(), torch.from_numpy(c["dw"]).cuda(),
        torch.from_numpy(c["perm"]).cuda(), torch.from_numpy(c["offsets"]).cuda(),
        torch.from_numpy(c["inv"]).cuda(), to_dev(dx_perm, dt))
    torch.cuda.synchronize()
    rdl, rdg, rdb, rdx = O.route_backward(d["x"], d["gate_w"], d["bias"], c["ids"], c["dw"],
                                          dx_perm, c["inv"], dt)
    xa = np.abs(decode(d["x"], dt))
    S = xa.T @ np.abs(rdl)
    err = np.abs(from_dev(dg).astype(np.float64) - rdg)
    assert (err <= 1e-4 * S + 1e-7).all(), f"dgate_w error {err.max()} (scale {S.max()})"
    Sb = np.abs(rdl).sum(axis=0)
    errb = np.abs(from_dev(db).astype(np.float64) - rdb)
    assert (errb <= 1e-4 * Sb + 1e-7).all(), f"dbias error {errb.max()}"
    check_combine(from_dev(dx), rdx, dt)
    return from_dev(dg), from_dev(dx)


WORKLOADS = list(I.WORKLOADS)


@pytest.mark.parametrize("name", WORKLOADS)
def test_combine_backward_full_size(name):
    print(f"[combine_backward] {name}", flush=True)
    d = I.make_inputs(name)
    _check_combine_backward(d, _case(d))


@pytest.mark.parametrize("name", WORKLOADS)
def test_dispatch_backward_full_size(name):
    print(f"[dispatch_backward] {name}", flush=True)
    d = I.make_inputs(name)
    ids = I.random_ids(7, d["N"], d["E"], d["K"])
    _, _, _, inv = O.dispatch(ids, d["E"])
    dx = L.dispatch_backward(to_dev(d["y"], d["dtype"]), torch.from_numpy(inv).cuda(), d["N"])
    torch.cuda.synchronize()
    ref = O.dispatch_backward(d["y"], inv, d["K"], d["dtype"])
    check_combine(from_dev(dx), ref, d["dtype"])
    S = sum_of_abs_terms(d["y"], inv, d["K"], d["dtype"])
    check_sum_tight(from_dev(dx), ref, S, d["K"], d["dtype"])


@pytest.mark.parametrize("name", WORKLOADS)
def test_route_backward_full_size(name):
    print(f"[route_backward] {name}", flush=True)
    d = I.make_inputs(name)
    _check_route_backward(d, _case(d))


BWD_EDGE = [
    # (N, H, E, K, dtype, bias)
    (1, 256, 16, 2, "bf16", False),
    (17, 128, 16, 2, "bf16", True),
    (65, 72, 20, 3, "bf16", True),        # H not a multiple of 64, E not a power of 2
    (100, 8, 4, 4, "bf16", False),        # K == E: the full softmax
    (37, 4, 5, 1, "f32", True),           # K = 1: no router gradient
    (129, 520, 256, 16, "bf16", True),    # E and K at their limits (generic-K kernels)
    (203, 96, 128, 8, "bf16", True),
    (1000, 264, 32, 3, "f32", False),     # generic K, fp32
    (5000, 128, 64, 6, "bf16", True),
    (600, 8192, 64, 2, "bf16", False),    # rows wider than one pass of the row loops
    # from 4096 tokens on, E <= 64 and K in {1, 2, 4, 8}: dx with the gate's
    # column slices in LDS
    (4096, 264, 64, 8, "bf16", True),     # K = 8; 33 vectors: one ragged slice
    (5000, 520, 16, 1, "f32", True),      # K = 1 (dx = the dispatch term), fp32
    (4500, 72, 33, 2, "bf16", False),     # 9 vectors per row: 55 idle lanes per wave
    (4100, 4104, 64, 4, "bf16", True),    # 513 vectors: a last slice of one vector
]


@pytest.mark.parametrize("N,H,E,K,dtype,bias", BWD_EDGE)
def test_backward_edge_cases(N, H, E, K, dtype, bias):
    print(f"[backward edge] N={N} H={H} E={E} K={K} {dtype} bias={bias}", flush=True)
    d = I.random_case(N * 13 + H, N, H, E, K, dtype, bias=bias)
    c = _case(d)
    _check_combine_backward(d, c)
    dg, dx = _check_route_backward(d, c)
    if K == 1:
        assert (dg == 0).all()
    # without dx_perm: the router part alone
    _check_route_backward(d, c, with_dx_perm=False)


def test_route_backward_skewed_with_empty_experts():
    # 48 experts, many without tokens: their gate columns get exactly zero
    N, H, E, K = 3001, 64, 48, 4
    print("[route_backward skewed]", flush=True)
    d = I.random_case(77, N, H, E, K, "bf16", bias=True)
    # a bias that favours six experts: most of the others get no token
    d["bias"] = np.where(np.arange(E) < 6, 4.0, -4.0).astype(np.float32)
    c = _case(d)
    counts = np.diff(c["offsets"])
    assert (counts == 0).sum() > E // 2
    dg, _ = _check_route_backward(d, c)
    assert (dg[:, counts == 0] == 0).all()


def test_backward_empty():
    dev = torch.device("cuda")
    H, E, K = 64, 16, 2
    z32 = torch.empty((0, K), dtype=torch.float32, device=dev)
    zi = torch.empty((0, K), dtype=torch.int32, device=dev)
    gw = torch.ones((H, E), dtype=torch.bfloat16, device=dev)
    dg, db, dx = L.route_backward(torch.empty((0, H), dtype=torch.bfloat16, device=dev), gw, zi,
                                  z32, z32, torch.empty((0,), dtype=torch.int32, device=dev),
                                  torch.zeros((E + 1,), dtype=torch.int32, device=dev))
    dy, dw = L.combine_backward(torch.empty((0, H), dtype=torch.bfloat16, device=dev),
                                torch.empty((0, H), dtype=torch.bfloat16, device=dev),
                                torch.empty((0,), dtype=torch.int32, device=dev), z32)
    torch.cuda.synchronize()
    assert (dg == 0).all() and (db == 0).all() and dx.shape == (0, H) and dw.shape == (0, K)


def test_backward_bitwise_deterministic():
    d = I.make_inputs("small-bf16")
    c = _case(d)
    K, dt = d["K"], d["dtype"]
    x_perm = to_dev(O.permute_rows(d["x"], c["perm"], K), dt)
    args = (x_perm, to_dev(d["gate_w"], dt), torch.from_numpy(c["ids"]).cuda(),
            torch.from_numpy(c["w"]).cuda(), torch.from_numpy(c["dw"]).cuda(),
            torch.from_numpy(c["perm"]).cuda(), torch.from_numpy(c["offsets"]).cuda(),
            torch.from_numpy(c["inv"]).cuda(), to_dev(d["y"], dt))
    a = L.route_backward(*args)
    b = L.route_backward(*args)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)
