"""Seeded synthetic inputs for the any4 quantizer (shared by tests, smoke and bench).

This module only draws random numbers; it holds none of the quantizer's arithmetic.
Both the HIP path and the CPU oracle consume what it returns, and neither imports
the other.

Distributions stand in for the Llama workloads of "any4: Learned 4-bit Numeric
Representation for LLMs" (arXiv 2507.04610): weights that are roughly Gaussian
with heavier tails (Section 3, background on numeric formats), a few outlier weights,
and per-channel mean-absolute activations E|x_j| with outlier channels (Section 4.1,
the calibration statistic).  The real checkpoints and the calibration prompt are not
used; these seeded arrays replace them.

Recipe (numpy ``Generator(PCG64(seed))``, drawn in this order):
  1. W = standard_t(5, (N, K)) * 0.02 in float64
  2. outlier entries: choice(N*K, round(0.001*N*K), replace=False), multiplied by 10
  3. cast to float32, then to bfloat16 with round-to-nearest-even (torch)
  4. act = lognormal(0, 0.5, K)
  5. outlier channels: choice(K, n_ch, replace=False), multiplied by 20
  6. act cast to float32
For a whole decoder layer, W and act come from separate seeds (steps 1-3 and 4-6).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

F32 = 0
BF16 = 1


@dataclasses.dataclass
class Matrix:
    name: str
    w: np.ndarray            # [N, K]; float32, or uint16 holding bfloat16 bits
    dtype: int               # F32 or BF16
    act: np.ndarray          # [K] float32, E|x_j|
    matrix_index: int = 0    # position in a batch (a Philox counter word)

    @property
    def shape(self):
        return self.w.shape


@dataclasses.dataclass
class Workload:
    name: str
    matrices: List[Matrix]
    group: int
    n_clusters: int
    iters: int
    seed: int = 0            # Philox key

    @property
    def elements(self) -> int:
        return int(sum(m.w.shape[0] * m.w.shape[1] for m in self.matrices))

    @property
    def rows(self) -> int:
        return int(sum(m.w.shape[0] for m in self.matrices))


def outlier_channels(k: int) -> int:
    """Number of x20 activation channels: 1% of K (4 for the 512-wide toy)."""
    return 4 if k == 512 else int(round(0.01 * k))


def _to_bf16_bits(w32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(w32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_weights(rng: np.random.Generator, n: int, k: int, dtype: int) -> np.ndarray:
    w = rng.standard_t(5, size=(n, k)) * 0.02
    n_out = int(round(0.001 * n * k))
    if n_out:
        idx = rng.choice(n * k, n_out, replace=False)
        w.reshape(-1)[idx] *= 10.0
    w32 = w.astype(np.float32)
    del w
    if dtype == F32:
        return w32
    return _to_bf16_bits(w32)


def draw_act(rng: np.random.Generator, k: int, n_ch: Optional[int] = None) -> np.ndarray:
    act = rng.lognormal(0.0, 0.5, size=k)
    n_ch = outlier_channels(k) if n_ch is None else n_ch
    if n_ch:
        ch = rng.choice(k, n_ch, replace=False)
        act[ch] *= 20.0
    return act.astype(np.float32)


def make_matrix(name: str, n: int, k: int, dtype: int, seed: int, matrix_index: int = 0) -> Matrix:
    rng = np.random.Generator(np.random.PCG64(seed))
    w = draw_weights(rng, n, k, dtype)
    act = draw_act(rng, k)
    return Matrix(name, w, dtype, act, matrix_index)


LAYER_SHAPES = [  # (name, N, K, W seed, act seed) of a Llama3-8B-like decoder layer
    ("q_proj", 4096, 4096, 105, 121),
    ("k_proj", 1024, 4096, 106, 121),
    ("v_proj", 1024, 4096, 107, 121),
    ("o_proj", 4096, 4096, 108, 122),
    ("gate_proj", 14336, 4096, 109, 123),
    ("up_proj", 14336, 4096, 110, 123),
    ("down_proj", 4096, 14336, 111, 124),
]

CONFIGS = {
    # name: (builder description) -- see make()
    "tiny": "W 128x512 fp32, g=128, 16 clusters, 20 iters",
    "q_proj_g128": "W 2048x2048 bf16, g=128, 16 clusters, 20 iters",
    "q_proj_g64": "W 2048x2048 bf16, g=64, 16 clusters, 20 iters",
    "up_proj": "W 14336x4096 bf16, g=128, 16 clusters, 20 iters",
    "down_70b": "W 8192x28672 bf16, g=128, 16 clusters, 20 iters",
    "layer_any4": "7 matrices of a Llama3-8B-like layer, bf16, g=128, 16 clusters, 20 iters",
    "layer_any3": "same layer, 8 clusters",
    "layer_any2": "same layer, 4 clusters",
}


def make(name: str, rows: Optional[int] = None) -> Workload:
    """Build a named workload.  ``rows`` truncates every matrix to its first rows
    (the row-level draws are unchanged only for rows=None; truncation draws fresh,
    smaller matrices from the same seeds and is meant for quick runs)."""
    def nrows(n):
        return n if rows is None else min(n, rows)

    if name == "tiny":
        m = make_matrix("tiny", nrows(128), 512, F32, 101)
        return Workload(name, [m], 128, 16, 20)
    if name in ("q_proj_g128", "q_proj_g64"):
        m = make_matrix("q_proj", nrows(2048), 2048, BF16, 102)
        return Workload(name, [m], 128 if name.endswith("128") else 64, 16, 20)
    if name == "up_proj":
        m = make_matrix("up_proj", nrows(14336), 4096, BF16, 103)
        return Workload(name, [m], 128, 16, 20)
    if name == "down_70b":
        m = make_matrix("down_proj", nrows(8192), 28672, BF16, 104)
        return Workload(name, [m], 128, 16, 20)
    if name.startswith("layer_any"):
        bits = int(name[-1])
        acts = {}
        mats = []
        for idx, (mname, n, k, wseed, aseed) in enumerate(LAYER_SHAPES):
            rng = np.random.Generator(np.random.PCG64(wseed))
            w = draw_weights(rng, nrows(n), k, BF16)
            if aseed not in acts:
                acts[aseed] = draw_act(np.random.Generator(np.random.PCG64(aseed)), k)
            mats.append(Matrix(mname, w, BF16, acts[aseed], idx))
        return Workload(name, mats, 128, 1 << bits, 20)
    raise KeyError(name)


def draw_activations(rng: np.random.Generator, n_tokens: int, profile: np.ndarray,
                     dtype: int = BF16, chunk: int = 8192) -> np.ndarray:
    """Calibration activations [T, K]: x_tj = s_j * l_tj with l ~ Laplace(0, 1), whose
    mean absolute value is 1, so E|x_j| is close to the profile s_j (an E|x| profile from
    draw_act: lognormal channels with outlier channels x20).  Drawn in row chunks of
    ``chunk`` tokens (float64, scaled, cast to float32, then to bfloat16 with RNE)."""
    k = profile.shape[0]
    s = profile.astype(np.float64)
    out = np.empty((n_tokens, k), np.float32 if dtype == F32 else np.uint16)
    for t0 in range(0, n_tokens, chunk):
        t1 = min(n_tokens, t0 + chunk)
        x = (rng.laplace(0.0, 1.0, size=(t1 - t0, k)) * s).astype(np.float32)
        out[t0:t1] = x if dtype == F32 else _to_bf16_bits(x)
    return out


# Calibration batches: (name, tokens, channels, seed).  "calib_32x2048" stands in for a
# multi-sample calibration set (the pages compare their single prompt with 128 samples)
# at the hidden size of Llama3-8B: 32 sequences of 2048 tokens, 512 MiB of bf16, large
# enough to stream from HBM; "calib_small" is a quick case for parity tests.
CALIB = {
    "calib_32x2048": (32 * 2048, 4096, 131),
    "calib_small": (1000, 4096, 132),
}


def make_activations(name: str, tokens: Optional[int] = None) -> np.ndarray:
    """Seeded bf16 activations [T, K] (uint16 bits) for the E|x| reduction: the profile
    is drawn first, then the tokens, from one PCG64 stream."""
    T, k, seed = CALIB[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    profile = draw_act(rng, k)
    return draw_activations(rng, T if tokens is None else tokens, profile, BF16)


def random_matrix(n: int, k: int, dtype: int, seed: int) -> Matrix:
    """Small ad-hoc matrices for edge-case tests (same distributions)."""
    return make_matrix(f"rand{n}x{k}", n, k, dtype, seed)
