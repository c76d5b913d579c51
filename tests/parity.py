"""Comparison rules between the HIP path and the CPU oracle.

Integer outputs must match bit for bit.  Router ids are compared where the
answer is unique: a row whose K-th and (K+1)-th oracle logits differ by more
than 1e-3 must select the same set of experts, and the same order where every
adjacent gap among the top K+1 logits exceeds 1e-3; rows inside the margin
must pick valid experts (each within 1e-3 of the K-th logit).  Weights are
matched by (token, expert): within 2e-3 for bf16 inputs, 1e-5 for fp32.
Combine outputs: |gpu - ref| <= 1e-2*|ref| + 1e-4 for bf16 and
1e-5*|ref| + 1e-6 for fp32.

Beside those contract rules, the arithmetic the kernels claim is checked
tightly (check_sum_tight): a sum of n terms accumulated in fp32 and rounded
once differs from the oracle's exactly rounded sum by at most one unit in the
last place of the output format plus the fp32 accumulation error
n * 2^-24 * sum|terms|, and for bf16 outputs all but a few elements in 10^4
are bit-identical (they differ only where the fp32 error straddles a bf16
rounding point; in outputs too small for that rate, at most three elements).  A kernel that accumulated in bf16, rounded a product or a
partial sum to bf16, or truncated instead of rounding fails it.
"""
import numpy as np
import torch

from moe_token_routing_router_amd import inputs as I

MARGIN = 1e-3
U32 = 2.0 ** -24           # unit roundoff of fp32
MIN_EXACT = {"bf16": 0.9995}
MIN_MISMATCHES = 3          # ... but always this many allowed
W_TOL = {"bf16": 2e-3, "f32": 1e-5}
# what fp32 accumulation of the logits (exact bf16 products, or fp32 FMAs)
# and an fp32 softmax leave in the weights: logit errors of about 1e-6 for
# rows of up to W_TIGHT_H terms, and |dw| <= max|dl| / 2.  Rounding errors of
# a longer sum grow like the square root of its length on these random
# inputs, so beyond W_TIGHT_H terms the bound is scaled by
# sqrt(H / W_TIGHT_H).
W_TIGHT = {"bf16": 1e-5, "f32": 1e-6}
W_TIGHT_H = {"bf16": 4096, "f32": 1024}
C_REL = {"bf16": 1e-2, "f32": 1e-5}
C_ABS = {"bf16": 1e-4, "f32": 1e-6}


def to_dev(a, dtype):
    """numpy storage (uint16 bf16 bits or float32) -> device tensor."""
    if a is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def from_dev(t):
    """device tensor -> numpy storage (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode(a, dtype):
    if dtype == "bf16":
        return I.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def check_route(ids_g, w_g, ids_o, w_o, logits_o, K, dtype, H=None):
    """Assert router parity; returns the number of rows exempt by the margin.
    H, if given, is the logits' sum length (it widens the tight weight bound
    beyond W_TIGHT_H terms)."""
    N, E = logits_o.shape
    w_tight = W_TIGHT[dtype] * (max(1.0, H / W_TIGHT_H[dtype]) ** 0.5 if H else 1.0)
    assert ids_g.shape == (N, K) and w_g.shape == (N, K)
    assert ids_g.min() >= 0 and ids_g.max() < E, "router id out of range"
    srt = -np.sort(-logits_o, axis=1)
    if K < E:
        margin = srt[:, K - 1] - srt[:, K]
        gaps = srt[:, :K] - srt[:, 1:K + 1]
    else:
        margin = np.full(N, np.inf)
        gaps = np.concatenate([srt[:, :K - 1] - srt[:, 1:K], np.full((N, 1), np.inf)], 1)
    sure = margin > MARGIN
    ordered = sure & (gaps.min(axis=1) > MARGIN)
    # distinct ids per row
    s = np.sort(ids_g, axis=1)
    assert (np.diff(s, axis=1) > 0).all() if K > 1 else True, "duplicate expert in a row"
    # same set on rows with a clear margin, same order where gaps are clear
    so = np.sort(ids_o, axis=1)
    bad = sure & (s != so).any(axis=1)
    assert not bad.any(), f"{bad.sum()} rows choose a different expert set, e.g. row " \
                          f"{np.nonzero(bad)[0][:3]}"
    bad = ordered & (ids_g != ids_o).any(axis=1)
    assert not bad.any(), f"{bad.sum()} rows order their experts differently"
    # weights matched by (row, expert) on rows with the same set
    tol = W_TOL[dtype]
    rows = np.nonzero(sure)[0]
    og = np.argsort(ids_g[rows], axis=1, kind="stable")
    oo = np.argsort(ids_o[rows], axis=1, kind="stable")
    wg = np.take_along_axis(w_g[rows], og, 1).astype(np.float64)
    wo = np.take_along_axis(w_o[rows], oo, 1).astype(np.float64)
    err = np.abs(wg - wo).max() if len(rows) else 0.0
    assert err <= tol, f"router weight error {err} > {tol}"
    print(f"    router weight error {err:.3g} (tight bound {w_tight:g})", flush=True)
    assert err <= w_tight, f"router weight error {err} > {w_tight}"
    # rows inside the margin: valid picks, weights = softmax of the chosen
    # oracle logits, summing to one
    ex = np.nonzero(~sure)[0]
    if len(ex):
        lk = srt[ex, K - 1]
        chosen = np.take_along_axis(logits_o[ex], ids_g[ex].astype(np.int64), 1)
        assert (chosen >= lk[:, None] - MARGIN).all(), "invalid pick inside the margin"
        ref = np.exp(chosen - chosen.max(1, keepdims=True))
        ref /= ref.sum(1, keepdims=True)
        assert np.abs(ref - w_g[ex]).max() <= tol
        assert np.abs(ref - w_g[ex]).max() <= w_tight
    assert np.abs(w_g.astype(np.float64).sum(1) - 1).max() <= 1e-5
    return int((~sure).sum())


def check_combine(out_g, out_o, dtype):
    g = decode(out_g, dtype)
    o = decode(out_o, dtype)
    lim = C_REL[dtype] * np.abs(o) + C_ABS[dtype]
    err = np.abs(g - o)
    bad = err > lim
    assert not bad.any(), f"{bad.sum()} combine elements out of tolerance, worst " \
                          f"{(err - lim).max()} at {np.unravel_index(np.argmax(err - lim), err.shape)}"
    return float((err / (np.abs(o) + C_ABS[dtype])).max())


def sum_of_abs_terms(y, inv, K, dtype, w=None, residual=None, chunk=1024):
    """S[n, :] = sum_k |w[n,k]| * |y[inv[n*K+k], :]| (+ |residual[n, :]|) in
    float64, by chunks of tokens; w None means unit weights."""
    inv = np.asarray(inv, dtype=np.int64)
    N = inv.shape[0] // K
    H = y.shape[1]
    S = np.zeros((N, H))
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        acc = np.zeros((n1 - n0, H))
        for k in range(K):
            rows = np.abs(decode(y[inv[n0 * K + k:n1 * K:K]], dtype))
            if w is not None:
                rows *= np.abs(w[n0:n1, k].astype(np.float64))[:, None]
            acc += rows
        if residual is not None:
            acc += np.abs(decode(residual[n0:n1], dtype))
        S[n0:n1] = acc
    return S


def ulp(v, dtype):
    """Spacing of the format at |v| (normal range; the smallest normal
    spacing below it)."""
    p = 7 if dtype == "bf16" else 23
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - p)


def check_sum_tight(out_g, out_o, S, nterms, dtype):
    """Assert |g - o| <= max(ulp(g), ulp(o)) + nterms * 2^-24 * S on every
    element (see the module docstring) and, for bf16, that at least
    MIN_EXACT of the elements are bit-identical.  Returns the bit-identical
    fraction."""
    g = decode(out_g, dtype)
    o = decode(out_o, dtype)
    lim = np.maximum(ulp(g, dtype), ulp(o, dtype)) + nterms * U32 * S
    err = np.abs(g - o)
    bad = err > lim
    assert not bad.any(), f"{bad.sum()} elements beyond one ulp plus the fp32 accumulation " \
                          f"error, worst {(err - lim).max()} at " \
                          f"{np.unravel_index(np.argmax(err - lim), err.shape)}"
    size = np.asarray(out_g).size
    mism = int((np.asarray(out_g) != np.asarray(out_o)).sum())
    exact = 1.0 - mism / size if size else 1.0
    print(f"    bit-identical fraction {exact:.6f}", flush=True)
    if dtype in MIN_EXACT:
        # a rate: a handful of boundary cases in a tiny output is not one
        allowed = max(MIN_MISMATCHES, int((1.0 - MIN_EXACT[dtype]) * size))
        assert mism <= allowed, f"only {exact} of the outputs are bit-identical ({mism} differ)"
    return exact
