"""Seeded random shapes through the whole path on the GPU against the oracle.

Forward: the router (ids where the logit gaps are clear, weights), the fused
route+dispatch and the two-call sequence (bit for bit against each other and
against the oracle's counting sort of the GPU's ids), the standalone dispatch
of the oracle's ids, and the combine.  Backward and the widened calls, on the
oracle's routing of the same inputs: the combine backward, the dispatch
backward, the router backward with and without dx_perm, the aggregate with
its residual, and the expert-parallel send metadata over a random number of
ranks.

The 30 shapes are drawn once from a fixed seed: token counts from 1 to about
40000 (so the dispatch takes each of its forms: the small histogram summed
by the scatter, the block-prefix scatter and the scan kernel), hidden sizes
that are and are not multiples of 64, expert counts from 1 to 256 and K from
1 to min(E, 8).  Each case prints its shape before it runs."""
import numpy as np
import pytest
import torch

from moe_token_routing_router_amd import _lib as L
from moe_token_routing_router_amd import inputs as I
from oracle import oracle as O
from tests.parity import check_combine, check_route, check_sum_tight, from_dev, \
    sum_of_abs_terms, to_dev
from tests.test_backward_gpu import _case, _check_combine_backward, _check_route_backward
from tests.test_parity_gpu import _ep_check, _fused_and_check, gpu_dispatch, gpu_route

pytestmark = pytest.mark.gpu


def _shapes(n_cases=30, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        E = int(rng.choice([1, 2, 5, 16, 24, 48, 64, 64, 96, 128, 200, 256]))
        K = int(rng.integers(1, min(E, 8) + 1))
        N = int(np.exp(rng.uniform(0, np.log(40000))))
        dtype = "f32" if i % 6 == 5 else "bf16"
        step = 8 if dtype == "bf16" else 4
        H = int(rng.choice([step, 64, 72, 136, 256, 264]))
        H = max(step, H - H % step)
        out.append((N, H, E, K, dtype, bool(rng.integers(0, 2))))
    return out


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.library()


# and the shapes at the library's switch points, one on each side
THRESHOLD_SHAPES = [
    # the gathers' workgroup cap: from 16384 tokens, 4 KiB rows, 24 KiB per
    # workgroup (bf16 H = 2048 and 4096, fp32 H = 1024)
    (16383, 2048, 64, 2, "bf16", False), (16384, 2048, 64, 4, "bf16", True),
    (16385, 4096, 64, 2, "bf16", False), (16384, 1024, 32, 2, "f32", True),
    # router kernel switches: experts split from 8192 tokens at 129..256
    # experts, 16-token workgroups up to 4096 tokens, 128-token ones from 32768
    (8191, 64, 200, 4, "bf16", True), (8192, 64, 256, 8, "bf16", False),
    (4096, 128, 64, 4, "bf16", True), (4097, 128, 64, 5, "bf16", False),
    (32767, 64, 128, 2, "bf16", False), (32768, 64, 100, 8, "bf16", True),
    # the scatter's own block sums: at most 512 blocks and K <= 4 (the
    # standalone dispatch) or K <= 8 (the fused call)
    (32768, 72, 64, 4, "bf16", False), (32769, 72, 64, 4, "bf16", True),
    (2048, 264, 64, 5, "bf16", False), (2048, 264, 64, 8, "bf16", True),
    (2048, 264, 64, 9, "bf16", False),
    # the row-major gate at exactly 64 experts, packed at 65; fp32 H split
    # four ways from H = 128
    (3000, 128, 65, 3, "bf16", True), (3000, 128, 64, 3, "bf16", True),
    (1000, 124, 16, 2, "f32", False), (1000, 128, 16, 2, "f32", True),
]


@pytest.mark.parametrize("N,H,E,K,dtype,bias", _shapes() + THRESHOLD_SHAPES)
def test_random_shape_forward(N, H, E, K, dtype, bias):
    print(f"[random] N={N} H={H} E={E} K={K} {dtype} bias={bias}", flush=True)
    d = I.random_case(N * 31 + H * 7 + E, N, H, E, K, dtype, bias=bias)
    ids_o, w_o, logits_o, _ = O.route(d["x"], d["gate_w"], d["bias"], K, dtype)
    ids, w, counts = gpu_route(d)
    check_route(ids, w, ids_o, w_o, logits_o, K, dtype, H=H)
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    # fused call == two calls == the oracle's counting sort of the GPU's ids
    _fused_and_check(d, K, E, dtype)
    # standalone dispatch of the oracle's ids
    oc, oo, op, oi = O.dispatch(ids_o, E)
    gc, go, gp, gi, gx = gpu_dispatch(ids_o, d["x"], E, dtype)
    for a, b in ((gc, oc), (go, oo), (gp, op), (gi, oi)):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(gx.view(np.uint8), O.permute_rows(d["x"], op, K).view(np.uint8))
    # combine of expert outputs in the oracle's dispatched order
    out = L.combine(to_dev(d["y"], dtype), torch.from_numpy(oi).cuda(),
                    torch.from_numpy(w_o).cuda())
    torch.cuda.synchronize()
    ref = O.combine(d["y"], oi, w_o, dtype)
    check_combine(from_dev(out), ref, dtype)
    check_sum_tight(from_dev(out), ref, sum_of_abs_terms(d["y"], oi, K, dtype, w=w_o), K, dtype)


@pytest.mark.parametrize("N,H,E,K,dtype,bias", _shapes() + THRESHOLD_SHAPES)
def test_random_shape_backward_aggregate_ep(N, H, E, K, dtype, bias):
    print(f"[random bwd] N={N} H={H} E={E} K={K} {dtype} bias={bias}", flush=True)
    d = I.random_case(N * 31 + H * 7 + E, N, H, E, K, dtype, bias=bias)
    c = _case(d)
    _check_combine_backward(d, c)
    _check_route_backward(d, c)
    _check_route_backward(d, c, with_dx_perm=False)
    # dispatch backward (unit weights) and aggregate (weights + residual)
    inv_d = torch.from_numpy(c["inv"]).cuda()
    dx = L.dispatch_backward(to_dev(d["y"], dtype), inv_d, N)
    out = L.aggregate(to_dev(d["y"], dtype), inv_d, torch.from_numpy(c["w"]).cuda(),
                      to_dev(d["x"], dtype))
    torch.cuda.synchronize()
    ref = O.dispatch_backward(d["y"], c["inv"], K, dtype)
    check_combine(from_dev(dx), ref, dtype)
    check_sum_tight(from_dev(dx), ref, sum_of_abs_terms(d["y"], c["inv"], K, dtype), K, dtype)
    ref = O.aggregate(d["y"], c["inv"], c["w"], d["x"], dtype)
    check_combine(from_dev(out), ref, dtype)
    S = sum_of_abs_terms(d["y"], c["inv"], K, dtype, w=c["w"], residual=d["x"])
    check_sum_tight(from_dev(out), ref, S, K + 1, dtype)
    # expert-parallel metadata: a rank count that divides E
    divisors = [r for r in range(1, E + 1) if E % r == 0]
    R = int(np.random.default_rng(N + E).choice(divisors))
    print(f"[random ep] ep_size={R}", flush=True)
    _ep_check(c["ids"], d["x"], E, R, dtype)
