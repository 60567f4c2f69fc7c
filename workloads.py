"""Seeded synthetic inputs for banded Sinkhorn attention.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic.  Both the float64 oracle (through the tests and the
benchmark's CPU leg) and the GPU path consume the arrays built here, so the two
sides always see bit-identical inputs.

Every generator uses numpy's PCG64 (``numpy.random.default_rng(seed)``) and
draws in a fixed order: Q, K, V, dO, then the extras a config lists.  Values
are drawn in float64, rounded to float32 (round to nearest even) and, for the
bf16 configurations, rounded once more to bfloat16 (round to nearest even).
The returned float32 arrays hold exactly those rounded values, so upcasting
them to float64 reproduces what the GPU reads bit for bit.

The five named workloads follow the shapes of the Blockwise Differentiable
Sinkhorn Attention summaries: a tiny problem, a mid-size problem, a
protein-like batch with ragged lengths (it stands in for the Pfam task of
section 4.2, whose data is not used here), a dustbin-augmented batch
(section 2.3) and the long-context problem.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Problem", "make", "custom", "round_bf16", "CONFIG_NAMES"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    NaN/Inf are not expected in generated inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return rounded.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Problem:
    """One batch of inputs for the attention operator.

    Q, K, V, dO: float32 arrays [B, H, L, d] holding the exact input values
    (bf16-representable when dtype == "bf16").
    a, b: float32 [B, L] marginals, shared by all heads (zero on inactive
    tokens).
    lengths: int32 [B] number of real tokens per sequence, or None (= L).
    dustbin: when True the token at index lengths[b] is the dustbin.
    """

    name: str
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    dO: np.ndarray
    a: np.ndarray
    b: np.ndarray
    W: int
    T: int
    R: int
    dtype: str = "f32"
    lengths: Optional[np.ndarray] = None
    dustbin: bool = False

    @property
    def shape(self):
        return self.Q.shape

    @property
    def B(self):
        return self.Q.shape[0]

    @property
    def H(self):
        return self.Q.shape[1]

    @property
    def L(self):
        return self.Q.shape[2]

    @property
    def d(self):
        return self.Q.shape[3]

    def n_real(self) -> np.ndarray:
        """Real-token count per sequence (dustbin and filler excluded)."""
        if self.lengths is None:
            return np.full(self.B, self.L, dtype=np.int64)
        return self.lengths.astype(np.int64)

    def n_active(self) -> np.ndarray:
        """Active tokens per sequence: real ones plus the dustbin if present."""
        return self.n_real() + (1 if self.dustbin else 0)

    def real_tokens(self) -> int:
        return int(self.n_real().sum())


def _normal(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _uniform_marginals(B, L, n_real, dustbin=False, dustbin_mass=0.1):
    a = np.zeros((B, L), dtype=np.float64)
    for bi in range(B):
        n = int(n_real[bi])
        if dustbin:
            a[bi, :n] = (1.0 - dustbin_mass) / n if n > 0 else 0.0
            a[bi, n] = dustbin_mass if n > 0 else 1.0
        elif n > 0:
            a[bi, :n] = 1.0 / n
    a = a.astype(np.float32)
    return a, a.copy()


def _random_marginals(rng, B, L, n_real, sigma, dustbin=False, dustbin_mass=0.1):
    """Marginals proportional to exp(N(0, sigma^2)) on the real tokens,
    normalised to 1 (to 1 - dustbin_mass with a dustbin, which keeps its
    mass); a and b drawn independently, a first."""
    out = []
    for _ in range(2):
        m = np.zeros((B, L), dtype=np.float64)
        for bi in range(B):
            n = int(n_real[bi])
            if n == 0:
                if dustbin:
                    m[bi, 0] = 1.0
                continue
            w = np.exp(rng.standard_normal(n) * sigma)
            real = (1.0 - dustbin_mass) if dustbin else 1.0
            m[bi, :n] = real * w / w.sum()
            if dustbin:
                m[bi, n] = dustbin_mass
        out.append(m.astype(np.float32))
    return out[0], out[1]


def custom(B=1, H=1, L=64, d=16, W=17, T=20, R=2, dtype="f32", seed=0,
           scale=None, lengths=None, dustbin=False, dustbin_mass=0.1,
           filler="zero", marginals_sigma=None, name="custom") -> Problem:
    """A generic seeded problem: Q, K, V ~ N(0, scale^2), dO ~ N(0, 1).

    scale defaults to 1/sqrt(d).  lengths (list/array of B ints) makes the
    batch ragged; positions >= lengths[b] (+1 with a dustbin) are filler and
    are zeroed (filler="zero") or left random (filler="random").  Marginals
    are uniform over the real tokens, or, with marginals_sigma, drawn after
    dO as exp(N(0, sigma^2)) weights normalised per sequence.
    """
    rng = np.random.default_rng(seed)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    shp = (B, H, L, d)
    Q = _normal(rng, shp, scale)
    K = _normal(rng, shp, scale)
    V = _normal(rng, shp, scale)
    dO = _normal(rng, shp, 1.0)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int32)
        n_real = lengths
    else:
        n_real = np.full(B, L, dtype=np.int32)
    if filler == "zero" and (lengths is not None):
        for bi in range(B):
            first_filler = int(n_real[bi]) + (1 if dustbin else 0)
            for X in (Q, K, V):
                X[bi, :, first_filler:, :] = 0.0
    if marginals_sigma is None:
        a, b = _uniform_marginals(B, L, n_real, dustbin, dustbin_mass)
    else:
        a, b = _random_marginals(rng, B, L, n_real, marginals_sigma, dustbin, dustbin_mass)
    return Problem(name, _finish(Q, dtype), _finish(K, dtype), _finish(V, dtype),
                   _finish(dO, dtype), a, b, W, T, R, dtype, lengths, dustbin)


def _config1(dtype, seed, R):
    rng = np.random.default_rng(seed)
    shp = (1, 1, 64, 16)
    Q, K, V, dO = (_normal(rng, shp) for _ in range(4))
    a, b = _uniform_marginals(1, 64, [64])
    return Problem("tiny", _finish(Q, dtype), _finish(K, dtype), _finish(V, dtype),
                   _finish(dO, dtype), a, b, W=17, T=20, R=2 if R is None else R,
                   dtype=dtype)


def _config2(dtype, seed, R):
    rng = np.random.default_rng(seed)
    B, H, L, d = 4, 4, 1024, 64
    s = 1.0 / np.sqrt(d)
    Q = _normal(rng, (B, H, L, d), s)
    K = _normal(rng, (B, H, L, d), s)
    V = _normal(rng, (B, H, L, d), s)
    dO = _normal(rng, (B, H, L, d), 1.0)
    a, b = _uniform_marginals(B, L, [L] * B)
    return Problem("mid", _finish(Q, dtype), _finish(K, dtype), _finish(V, dtype),
                   _finish(dO, dtype), a, b, W=128, T=50, R=2 if R is None else R,
                   dtype=dtype)


def _config3(dtype, seed, R, filler="zero"):
    """Protein-like batch: 20-letter token ids, ragged lengths in [128, 512].

    Embedding table E ~ N(0, 0.02^2) [20, 512]; projections W_q, W_k, W_v ~
    N(0, 1/512) [512, 512]; Q = E[ids] @ W_q split into 8 heads of 64.
    """
    rng = np.random.default_rng(seed)
    B, H, L, d = 8, 8, 512, 64
    D = H * d
    # draw order: dO first (shape known up front), then the extras.
    dO = _normal(rng, (B, H, L, d), 1.0)
    ids = rng.integers(0, 20, size=(B, L))
    lengths = rng.integers(128, 513, size=B).astype(np.int32)
    E = rng.standard_normal((20, D)) * 0.02
    Wq = rng.standard_normal((D, D)) / np.sqrt(D)
    Wk = rng.standard_normal((D, D)) / np.sqrt(D)
    Wv = rng.standard_normal((D, D)) / np.sqrt(D)
    X = E[ids]  # [B, L, D]
    proj = []
    for Wm in (Wq, Wk, Wv):
        Y = (X @ Wm).reshape(B, L, H, d).transpose(0, 2, 1, 3).astype(np.float32)
        proj.append(np.ascontiguousarray(Y))
    Q, K, V = proj
    if filler == "zero":
        for bi in range(B):
            for Y in (Q, K, V):
                Y[bi, :, lengths[bi]:, :] = 0.0
    elif filler == "random":
        frng = np.random.default_rng(seed + 1000)
        for bi in range(B):
            n = lengths[bi]
            for Y in (Q, K, V):
                Y[bi, :, n:, :] = frng.standard_normal((H, L - n, d)).astype(np.float32)
    a, b = _uniform_marginals(B, L, lengths)
    return Problem("protein", _finish(Q, dtype), _finish(K, dtype), _finish(V, dtype),
                   _finish(dO, dtype), a, b, W=64, T=30, R=2 if R is None else R,
                   dtype=dtype, lengths=lengths)


def _config4(dtype, seed, R, tile=128):
    """Dustbin-augmented batch: n = 2048 real tokens, one dustbin at index n."""
    rng = np.random.default_rng(seed)
    B, H, n, d = 2, 8, 2048, 64
    L = ((n + 1 + tile - 1) // tile) * tile
    s = 1.0 / np.sqrt(d)
    shp = (B, H, L, d)
    Q = _normal(rng, shp, s)
    K = _normal(rng, shp, s)
    V = _normal(rng, shp, s)
    dO = _normal(rng, shp, 1.0)
    for Y in (Q, K, V):
        Y[:, :, n + 1:, :] = 0.0
    lengths = np.full(B, n, dtype=np.int32)
    a, b = _uniform_marginals(B, L, lengths, dustbin=True, dustbin_mass=0.1)
    return Problem("dustbin", _finish(Q, dtype), _finish(K, dtype), _finish(V, dtype),
                   _finish(dO, dtype), a, b, W=128, T=50, R=2 if R is None else R,
                   dtype=dtype, lengths=lengths, dustbin=True)


def _config5(dtype, seed, R, heads=None):
    rng = np.random.default_rng(seed)
    B, H, L, d = 1, 8, 32768, 128
    s = 1.0 / np.sqrt(d)
    shp = (B, H, L, d)
    Q = _normal(rng, shp, s)
    K = _normal(rng, shp, s)
    V = _normal(rng, shp, s)
    dO = _normal(rng, shp, 1.0)
    if heads is not None:
        sel = list(heads)
        Q, K, V, dO = (np.ascontiguousarray(X[:, sel]) for X in (Q, K, V, dO))
    a, b = _uniform_marginals(B, L, [L])
    return Problem("long", _finish(Q, dtype), _finish(K, dtype), _finish(V, dtype),
                   _finish(dO, dtype), a, b, W=256, T=100, R=2 if R is None else R,
                   dtype=dtype)


CONFIG_NAMES = {1: "tiny", 2: "mid", 3: "protein", 4: "dustbin", 5: "long"}


def make(config, dtype=None, seed=0, R=None, **kw) -> Problem:
    """Build one of the five named workloads (1..5 or its name).

    dtype defaults to "f32" for configs 1-4 and "bf16" for config 5.
    Config 3 accepts filler="zero"|"random"; config 5 accepts heads=[...] to
    keep a subset of the 8 heads (each head is an independent problem and the
    draws are made for all 8 first, so a subset is bit-identical to the same
    heads of the full batch).
    """
    if isinstance(config, str):
        inv = {v: k for k, v in CONFIG_NAMES.items()}
        config = inv[config]
    if dtype is None:
        dtype = "bf16" if config == 5 else "f32"
    if config == 1:
        return _config1(dtype, seed, R)
    if config == 2:
        return _config2(dtype, seed, R)
    if config == 3:
        return _config3(dtype, seed, R, **kw)
    if config == 4:
        return _config4(dtype, seed, R, **kw)
    if config == 5:
        return _config5(dtype, seed, R, **kw)
    raise ValueError(f"unknown config {config}")
