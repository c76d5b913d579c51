"""Grouped expert linear layer, HIP vs the CPU oracle, through the C ABI.

Rule: |gpu - ref| <= 1e-2 * |ref| + 2e-5 * S + 1e-6 for bf16 outputs (one bf16
rounding on each side, fp32 accumulation on the GPU) and 2e-5 * S + 1e-6 for
fp32, with S[p, f] = sum_h |x_perm[p, h] * weight[e][f][h]| (numpy, float64).
Small and ragged shapes, and the 256 x 256 ring-tile path at small H with
over a thousand tiles, are compared on every output; the headline shape
(N*K = 32768 dispatched rows, H = F = 4096, 64 experts) on sampled rows that
the oracle computes one by one, in the launch configuration the benchmark
times.  Rows past offsets[E] must stay untouched.
"""
import numpy as np
import pytest
import torch

from moe_token_routing_router_amd import _lib as L
from moe_token_routing_router_amd import inputs as I
from oracle import oracle as O
from tests.parity import decode, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.library()


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _check(got, ref, x, W, off, rows, dtype):
    seg = np.searchsorted(off, rows, side="right") - 1
    Wa = np.abs(decode(W, dtype))
    S = np.empty((len(rows), W.shape[1]))
    for e in np.unique(seg):  # S = |x| @ |W[e]|^T, one product per expert's rows
        sel = np.nonzero(seg == e)[0]
        S[sel] = np.abs(decode(x[rows[sel]], dtype)) @ Wa[e].T
    g = decode(got, dtype)
    r = decode(ref, dtype)
    rel = 1e-2 if dtype == "bf16" else 0.0
    err = np.abs(g - r)
    bad = err > rel * np.abs(r) + 2e-5 * S + 1e-6
    assert not bad.any(), f"{bad.sum()} outputs off, max error {err.max()}"


def _run(x, W, off, T, dtype):
    y = L.grouped_linear(to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    return from_dev(y)


CASES = [
    # (counts per expert, H, F, dtype)
    ([130, 0, 1, 257, 64], 256, 128, "bf16"),        # ragged tiles, an empty expert
    ([7, 300, 0, 0, 45, 128, 129], 72, 136, "bf16"),  # H, F not multiples of 64/128
    ([1], 8, 8, "bf16"),                              # the smallest rows
    ([512] * 3, 1024, 1024, "bf16"),                  # several full tiles each way
    ([33, 0, 97], 520, 264, "f32"),
    ([0] * 255 + [70], 128, 64, "bf16"),              # 256 experts, one with rows
]


@pytest.mark.parametrize("counts,H,F,dtype", CASES)
def test_grouped_linear_every_output(counts, H, F, dtype):
    print(f"[grouped] counts={counts[:8]} H={H} F={F} {dtype}", flush=True)
    E = len(counts)
    off = _offsets(counts)
    T = int(off[-1]) + 5  # rows past offsets[E] must stay untouched
    x = I.random_case(T + H, T, H, 4, 1, dtype, with_y=False)["x"]
    W = I.expert_weights(H + F, E, F, H, dtype)
    got = _run(x, W, off, T, dtype)
    ref = O.grouped_linear(x, W, off, dtype)
    n = int(off[-1])
    _check(got[:n], ref, x, W, off, np.arange(n), dtype)
    assert (got[n:] == 0).all()


def test_grouped_linear_headline_shape_sampled_rows():
    # the dispatched rows of the headline routing shape: 64 experts, N*K =
    # 32768 rows of H = 4096, F = 4096 outputs; counts from the routed ids
    N, H, E, K, F = 16384, 4096, 64, 2, 4096
    print("[grouped] headline shape, sampled rows", flush=True)
    ids = I.random_ids(5, N, E, K, skew=0.3)
    counts = np.bincount(ids.ravel(), minlength=E)
    off = _offsets(counts)
    T = N * K
    x = I.random_case(5, T, H, 4, 1, "bf16", with_y=False)["x"]
    W = I.expert_weights(6, E, F, H, "bf16")
    got = _run(x, W, off, T, "bf16")
    rng = np.random.default_rng(7)
    # first and last row of every expert's segment (tile edges) plus random rows
    edges = np.concatenate([off[:-1][counts > 0], off[1:][counts > 0] - 1])
    rows = np.unique(np.concatenate([edges, rng.integers(0, T, 64)])).astype(np.int32)
    ref = O.grouped_linear(x, W, off, "bf16", rows=rows)
    _check(got[rows], ref, x, W, off, rows, "bf16")


@pytest.mark.parametrize("H,F", [(96, 1000), (32, 1024), (64, 1000), (192, 1024)])
def test_grouped_linear_large_tiles_ragged_every_output(H, F):
    # enough tiles for the 256 x 256 path (about 1200 tiles of 256 x 256),
    # with 32-wide K steps (H = 96: three steps, H = 32: one) and 64-wide
    # ones (H = 64: one, H = 192: three), a ragged last n-tile (F = 1000) and
    # experts of every size including empty ones; every output against the
    # oracle (small H keeps the oracle's 2-13 G multiply-adds to seconds)
    N, E, K = 33000, 40, 2
    print(f"[grouped] large tiles H={H} F={F}, every output", flush=True)
    ids = I.random_ids(H + F, N, E, K, skew=0.8)
    counts = np.bincount(ids.ravel(), minlength=E)
    counts[[3, 17]] = 0
    off = _offsets(counts)
    T = int(off[-1]) + 3
    x = I.random_case(H, T, H, 4, 1, "bf16", with_y=False)["x"]
    W = I.expert_weights(F, E, F, H, "bf16")
    got = _run(x, W, off, T, "bf16")
    n = int(off[-1])
    tiles = sum(-(-int(c) // 256) for c in counts) * -(-F // 256)
    assert tiles >= 1024, tiles
    ref = O.grouped_linear(x, W, off, "bf16")
    _check(got[:n], ref, x, W, off, np.arange(n), "bf16")
    assert (got[n:] == 0).all()
