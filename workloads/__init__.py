"""Seeded synthetic inputs for the bitmap int4 / fp16 SpMM workloads.

This module only draws random numbers into dense arrays. It holds none of the
method's arithmetic (no bitmap encoding, no packing, no products): both the
oracle side and the GPU side start from the dense arrays returned here.

The shapes follow the decode-phase projection / FFN layers that UnionSparse
(IEEE TCAD, "UnionSparse: An Index-Efficient Sparsity Framework for Low-Bit
Sparse LLM Inference on Edge") evaluates in Sec. VII-A: W4A4 weights with
30-70 % unstructured sparsity and decode widths N = 1..32. The fp16 case
follows SPDP ("Unified Static-Dynamic Pruning for Efficient LLM Inference"),
Sec. 2.2 (static magnitude pruning with a fixed mask). The pages' model
weights are not available, so iid masks stand in for pruned real weights.

Recipe (numpy ``default_rng(seed)``, PCG64), draw order inside a config is
mask -> values -> X:

* int4 nonzeros: ``rng.integers(0, 15, dtype=int8)`` mapped d -> d-8 if
  d < 8 else d-7, i.e. uniform over {-8..-1, 1..7};
* int4 activations: ``rng.integers(-8, 8, dtype=int8)``, uniform over [-8, 7];
* masks: ``rng.integers(0, 65536, dtype=uint16) < round(keep * 65536)`` per
  element (keep probability quantised to 1/65536);
* per-row density (low-sparsity case): ``rng.uniform(0.6, 0.8, M)`` drawn
  before the mask, then element kept with its row's probability;
* fp16 case: W = N(0, 0.02) cast to fp16, then the round(0.6*M*K) entries of
  smallest |W| (stable argsort on the flat index) are set to +0; X = N(0, 1)
  cast to fp16.
* row-wise pruning (``rows=True`` in the random problems): every row keeps
  the same count, as a pruner that ranks the weights of each output row
  separately leaves them (Wanda, which both pages use for their end-to-end
  runs, does so). int4: ``rng.random((M, K))`` keys, the round(keep*K)
  smallest of each row (stable argsort) kept, then the values; fp16: the
  round(sparsity*K) entries of smallest |W| of each row set to +0.

X is returned as an ``[N][K]`` array (the K x N activation matrix stored
column by column), drawn at the largest N of the config; a smaller N uses the
leading rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

__all__ = ["Problem", "CONFIGS", "make", "int4_nonzero_values", "int4_mask_matrix", "int4_mask_rows_exact",
           "random_int4_problem", "config_names", "int2_nonzero_values", "int2_like", "random_int2_problem"]


@dataclass
class Problem:
    """One W (M x K) and X ([N][K]) pair. ``dtype`` is "int4" or "fp16"."""
    name: str
    dtype: str
    W: np.ndarray            # int8 values in [-8, 7] or float16, shape (M, K)
    X: np.ndarray            # int8 values in [-8, 7] or float16, shape (N, K)
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def M(self) -> int:
        return int(self.W.shape[0])

    @property
    def K(self) -> int:
        return int(self.W.shape[1])

    @property
    def N(self) -> int:
        return int(self.X.shape[0])

    def with_n(self, n: int) -> "Problem":
        """The same W with the first ``n`` activation columns."""
        if n < 0 or n > self.X.shape[0]:
            raise ValueError(f"n={n} outside 0..{self.X.shape[0]}")
        return Problem(self.name, self.dtype, self.W, self.X[:n], dict(self.meta, N=n))


def int4_nonzero_values(rng: np.random.Generator, size) -> np.ndarray:
    d = rng.integers(0, 15, size=size, dtype=np.int8)
    return (d - np.int8(8) + (d >= 8).astype(np.int8)).astype(np.int8)


def int4_activations(rng: np.random.Generator, size) -> np.ndarray:
    return rng.integers(-8, 8, size=size, dtype=np.int8)


def int4_mask_matrix(rng: np.random.Generator, M: int, K: int, keep) -> np.ndarray:
    """Bernoulli keep-mask. ``keep`` is a scalar or a per-row array of length M;
    the probability is quantised to 1/65536."""
    thresh = np.round(np.asarray(keep, dtype=np.float64) * 65536.0).astype(np.uint32)
    if thresh.ndim == 1:
        thresh = thresh[:, None]
    return rng.integers(0, 65536, size=(M, K), dtype=np.uint16) < thresh


def int4_mask_rows_exact(rng: np.random.Generator, M: int, K: int, keep: float) -> np.ndarray:
    """Keep-mask with exactly round(keep * K) entries in every row: those of
    the smallest uniform keys of the row."""
    k = int(round(keep * K))
    order = np.argsort(rng.random((M, K)), axis=1, kind="stable")
    mask = np.zeros((M, K), dtype=bool)
    np.put_along_axis(mask, order[:, :k], True, axis=1)
    return mask


def _int4_weights(rng, M, K, keep, rows: bool = False) -> np.ndarray:
    mask = int4_mask_rows_exact(rng, M, K, keep) if rows else int4_mask_matrix(rng, M, K, keep)
    vals = int4_nonzero_values(rng, (M, K))
    return (vals * mask).astype(np.int8)


def int2_nonzero_values(rng: np.random.Generator, size) -> np.ndarray:
    """Uniform over the nonzero 2-bit codes {-2, -1, 1}."""
    d = rng.integers(0, 3, size=size, dtype=np.int8)
    return (d - np.int8(2) + (d >= 2).astype(np.int8)).astype(np.int8)


def int2_like(W: np.ndarray, seed: int = 0) -> np.ndarray:
    """2-bit weights with the nonzero pattern of W (W2A4 runs on the same
    masks as the int4 workloads): fresh values in {-2, -1, 1} where W != 0."""
    rng = np.random.default_rng(seed)
    return (int2_nonzero_values(rng, W.shape) * (W != 0)).astype(np.int8)


def random_int2_problem(seed: int, M: int, K: int, N: int, keep: float = 0.5, name: str = "random_w2") -> Problem:
    """Small seeded W2A4 case of any shape: 2-bit weights, int4 activations."""
    rng = np.random.default_rng(seed)
    mask = int4_mask_matrix(rng, M, K, keep)
    W = (int2_nonzero_values(rng, (M, K)) * mask).astype(np.int8)
    X = int4_activations(rng, (N, K))
    return Problem(name, "int2", W, X, dict(seed=seed, keep=keep, N=N))


def random_int4_problem(seed: int, M: int, K: int, N: int, keep: float = 0.5,
                        name: str = "random", rows: bool = False) -> Problem:
    """Seeded int4 case of any shape (tests, edge cases); ``rows``: the same
    count kept in every row."""
    rng = np.random.default_rng(seed)
    W = _int4_weights(rng, M, K, keep, rows)
    X = int4_activations(rng, (N, K))
    return Problem(name, "int4", W, X, dict(seed=seed, keep=keep, N=N, rows=rows))


def random_fp16_problem(seed: int, M: int, K: int, N: int, sparsity: float = 0.6,
                        name: str = "random_f16", rows: bool = False) -> Problem:
    """Seeded fp16 case of any shape; ``rows``: each row pruned by magnitude
    to the same count."""
    rng = np.random.default_rng(seed)
    W = _fp16_pruned_rows(rng, M, K, sparsity) if rows else _fp16_pruned(rng, M, K, sparsity)
    X = rng.normal(0.0, 1.0, size=(N, K)).astype(np.float16)
    return Problem(name, "fp16", W, X, dict(seed=seed, sparsity=sparsity, N=N, rows=rows))


def _fp16_pruned(rng, M, K, sparsity) -> np.ndarray:
    W = rng.normal(0.0, 0.02, size=(M, K)).astype(np.float16)
    n_prune = int(round(sparsity * M * K))
    flat = W.reshape(-1)
    order = np.argsort(np.abs(flat.astype(np.float32)), kind="stable")
    flat[order[:n_prune]] = np.float16(0.0)
    return flat.reshape(M, K)


def _fp16_pruned_rows(rng, M, K, sparsity) -> np.ndarray:
    W = rng.normal(0.0, 0.02, size=(M, K)).astype(np.float16)
    order = np.argsort(np.abs(W.astype(np.float32)), axis=1, kind="stable")
    np.put_along_axis(W, order[:, :int(round(sparsity * K))], np.float16(0.0), axis=1)
    return W


# ---------------------------------------------------------------------------
# The five named workloads.

def _c1() -> List[Problem]:
    rng = np.random.default_rng(0)
    W = _int4_weights(rng, 512, 512, 0.5)
    X = int4_activations(rng, (1, 512))
    return [Problem("tiny_512x512_n1", "int4", W, X, dict(seed=0, keep=0.5, N=1))]


def _c2() -> List[Problem]:
    rng = np.random.default_rng(1)
    W = _int4_weights(rng, 12288, 4096, 0.5)
    X = int4_activations(rng, (32, 4096))   # drawn at 32 so the N sweep shares one X
    return [Problem("qkv_12288x4096", "int4", W, X[:8], dict(seed=1, keep=0.5, N=8, X_full=X))]


def _c3() -> List[Problem]:
    rng = np.random.default_rng(2)
    Wu = _int4_weights(rng, 11008, 4096, 0.3)
    Xu = int4_activations(rng, (16, 4096))
    Wd = _int4_weights(rng, 4096, 11008, 0.3)
    Xd = int4_activations(rng, (16, 11008))
    return [Problem("ffn_up_11008x4096", "int4", Wu, Xu, dict(seed=2, keep=0.3, N=16)),
            Problem("ffn_down_4096x11008", "int4", Wd, Xd, dict(seed=2, keep=0.3, N=16))]


def _c4() -> List[Problem]:
    rng = np.random.default_rng(3)
    dens = rng.uniform(0.6, 0.8, size=8192)
    W = _int4_weights(rng, 8192, 8192, dens)
    X = int4_activations(rng, (32, 8192))
    return [Problem("lowsparse_8192x8192", "int4", W, X, dict(seed=3, keep="U[0.6,0.8] per row", N=32))]


def _c5() -> List[Problem]:
    rng = np.random.default_rng(4)
    W = _fp16_pruned(rng, 4096, 4096, 0.6)
    X = rng.normal(0.0, 1.0, size=(32, 4096)).astype(np.float16)
    return [Problem("fp16_4096x4096_n1", "fp16", W, X[:1], dict(seed=4, sparsity=0.6, N=1)),
            Problem("fp16_4096x4096_n32", "fp16", W, X, dict(seed=4, sparsity=0.6, N=32))]


CONFIGS = {
    "tiny": _c1,
    "qkv": _c2,
    "ffn": _c3,
    "lowsparse": _c4,
    "fp16": _c5,
}


def config_names() -> List[str]:
    return list(CONFIGS)


_CACHE: Dict[str, List[Problem]] = {}


def make(config: str) -> List[Problem]:
    """Problems of a named workload (cached per process)."""
    if config not in CONFIGS:
        raise KeyError(f"unknown workload {config!r}; have {list(CONFIGS)}")
    if config not in _CACHE:
        _CACHE[config] = CONFIGS[config]()
    return _CACHE[config]
