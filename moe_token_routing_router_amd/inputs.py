"""Seeded synthetic inputs for the MoE routing path.

This module holds no arithmetic of the method: it only draws random data of
the shapes and distributions of the five workloads and stores it as fp32 or
as bf16 bit patterns.  Both the HIP path and the CPU oracle are fed from
here.  Everything is drawn with numpy's PCG64 (``default_rng(seed)``) in a
fixed order -- x, gate_w, bias, then y -- so that asking for fewer arrays
never changes the ones that are drawn.

Workloads (tokens N, hidden H, experts E, top-K):
  tiny-fp32     N=512   H=256  E=16  K=2  fp32, no bias
  small-bf16    N=2048  H=1024 E=64  K=2  bf16, no bias
  biased-bf16   N=4096  H=2048 E=64  K=4  bf16, bias ~ N(0, variance 0.5)
  h4096-bf16    N=16384 H=4096 E=64  K=2  bf16, no bias (8 sequences x 2048)
  zipf128-bf16  N=32768 H=2048 E=128 K=8  bf16, bias = -1.1*ln(rank) over a
                seeded rank permutation, plus 4 experts forced dead (-1e4)

x ~ N(0,1) [N,H];  gate_w ~ N(0, 1/H) [H,E];  y ~ N(0,1) [N*K,H] (expert
outputs in dispatched order).  bf16 values are the round-to-nearest-even
image of the fp32 draw, rounded once; the same bits go to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    E: int
    K: int
    dtype: str            # "f32" or "bf16"
    bias: str             # "none", "normal", "zipf"
    seed: int
    bias_var: float = 0.0
    zipf_s: float = 0.0
    dead: int = 0

    @property
    def T(self) -> int:
        return self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def describe(self) -> str:
        return (f"route+dispatch+combine N={self.N} H={self.H} E={self.E} "
                f"K={self.K} {self.dtype}")


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-fp32", 512, 256, 16, 2, "f32", "none", seed=1),
        Workload("small-bf16", 2048, 1024, 64, 2, "bf16", "none", seed=2),
        Workload("biased-bf16", 4096, 2048, 64, 4, "bf16", "normal", seed=3,
                 bias_var=0.5),
        Workload("h4096-bf16", 16384, 4096, 64, 2, "bf16", "none", seed=4),
        Workload("zipf128-bf16", 32768, 2048, 128, 8, "bf16", "zipf", seed=5,
                 zipf_s=1.1, dead=4),
    ]
}

HEADLINE = "h4096-bf16"

_CHUNK_ROWS = 4096


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even) and return
    the uint16 bit patterns.  Inputs here are always finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _normal_rows(rng, rows: int, cols: int, dtype: str, scale: float = 1.0):
    """Draw a [rows, cols] standard-normal matrix in chunks of rows, scaled,
    stored as float32 or as bf16 bits."""
    out = np.empty((rows, cols), np.float32 if dtype == "f32" else np.uint16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        out[r0:r1] = blk if dtype == "f32" else f32_to_bf16_bits(blk)
    return out


def _bias(rng, w: Workload) -> Optional[np.ndarray]:
    if w.bias == "none":
        return None
    if w.bias == "normal":
        return rng.normal(0.0, math.sqrt(w.bias_var), w.E).astype(np.float32)
    if w.bias == "zipf":
        # rank r_e = 1 + pi(e) for a seeded permutation pi; the logit bias is
        # the log of the Zipf(s) weight r^-s, so a softmax over the bias alone
        # reproduces the Zipf distribution.  The `dead` experts with the
        # largest ranks get a bias far below every logit, so they receive no
        # tokens.
        pi = rng.permutation(w.E)
        rank = 1 + pi
        b = (-w.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
        b[rank > w.E - w.dead] = np.float32(-1.0e4)
        return b
    raise ValueError(f"unknown bias kind {w.bias}")


def make_inputs(w: Workload | str, with_y: bool = True, n_tokens: Optional[int] = None):
    """Return a dict with x, gate_w, bias (or None) and, if asked, y.

    ``n_tokens`` overrides N (the draw is then a different, smaller problem of
    the same distribution; the shapes of gate_w and bias do not change).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    N = w.N if n_tokens is None else int(n_tokens)
    rng = np.random.default_rng(w.seed)
    x = _normal_rows(rng, N, w.H, w.dtype)
    gate_w = _normal_rows(rng, w.H, w.E, w.dtype, scale=1.0 / math.sqrt(w.H))
    bias = _bias(rng, w)
    d = {"x": x, "gate_w": gate_w, "bias": bias, "N": N, "H": w.H, "E": w.E,
         "K": w.K, "dtype": w.dtype}
    if with_y:
        d["y"] = _normal_rows(rng, N * w.K, w.H, w.dtype)
    return d


def random_case(seed: int, N: int, H: int, E: int, K: int, dtype: str,
                bias: bool = False, with_y: bool = True):
    """A small random case of any shape (for edge-case tests)."""
    rng = np.random.default_rng(seed)
    x = _normal_rows(rng, N, H, dtype)
    gate_w = _normal_rows(rng, H, E, dtype, scale=1.0 / math.sqrt(H))
    b = rng.normal(0.0, 1.0, E).astype(np.float32) if bias else None
    d = {"x": x, "gate_w": gate_w, "bias": b, "N": N, "H": H, "E": E, "K": K,
         "dtype": dtype}
    if with_y:
        d["y"] = _normal_rows(rng, N * K, H, dtype)
    return d


def expert_weights(seed: int, E: int, F: int, H: int, dtype: str) -> np.ndarray:
    """Synthetic expert-layer weights [E,F,H] ~ N(0, 1/H) (random init of the
    expert layer; no checkpoint), drawn expert by expert."""
    rng = np.random.default_rng(seed)
    out = np.empty((E, F, H), np.float32 if dtype == "f32" else np.uint16)
    for e in range(E):
        out[e] = _normal_rows(rng, F, H, dtype, scale=1.0 / math.sqrt(H))
    return out


def random_ids(seed: int, N: int, E: int, K: int, skew: float = 0.0) -> np.ndarray:
    """Distinct expert ids per token, [N,K] int32; with skew > 0 the experts
    are drawn with Zipf-like weights so some segments are large and some
    empty."""
    rng = np.random.default_rng(seed)
    logw = -skew * np.log1p(np.arange(E, dtype=np.float64))
    # K distinct draws without replacement, weights exp(logw): the K largest
    # of logw + Gumbel noise (the Gumbel-top-k construction).
    g = rng.gumbel(size=(N, E)) + logw[None, :]
    return np.argsort(-g, axis=1, kind="stable")[:, :K].astype(np.int32)
