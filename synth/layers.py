"""Seeded synthetic linear layers (shapes of the OPT-350m, 7B, 13B and 65B workloads).

Every tensor comes from its own stream::

    numpy.random.default_rng([config_id, layer_id, tensor_id, variant_id])

with tensor_id 0 = bulk activations, 1 = planted outlier columns, 2 = weight,
3 = bias.  The tuple is returned with the tensors so that a result line can
name exactly what it ran on.

Recipe (a reading; the pages give shapes and magnitudes, not distributions):

* bulk activations: N(0, 1) (or Student-t with 3 degrees of freedom scaled by
  1/sqrt(3) for the heavy-tailed 65B workload), rounded to fp16; any draw whose
  fp16 magnitude reaches the threshold magnitude is re-drawn from the same
  stream, so that the planted columns are the only outlier columns;
* outlier columns: ``n_outlier`` distinct columns chosen uniformly; every row of
  each (or a seeded fraction of the rows, for edge-case tests) gets
  sign * U(lo, hi) with an equiprobable sign, rounded to fp16;
* weight: N(0, 0.02) rounded to fp16 (nn.Linear orientation, out x in);
* bias: N(0, bias_std) rounded to fp16, or absent.

Nothing here quantizes or multiplies; the threshold is used only to shape the
random draws.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

TAU_DEFAULT = 6.0


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer of a workload: out[m, n] = sum_k x[m, k] * w[n, k] (+ bias)."""

    config_id: int
    layer_id: int
    name: str
    m: int
    k: int
    n: int
    n_outlier: int
    outlier_lo: float
    outlier_hi: float
    bulk: str = "normal"          # "normal" | "t3"
    bias_std: Optional[float] = None
    tau: float = TAU_DEFAULT
    variant_id: int = 0
    truncate: bool = True         # False: the bulk keeps its raw tail (stress input)

    @property
    def ops(self) -> int:
        """Multiply-accumulate count times two (the usual GEMM op count)."""
        return 2 * self.m * self.n * self.k


def _workloads() -> Dict[str, List[LayerSpec]]:
    w: Dict[str, List[LayerSpec]] = {}
    # 1: tiny layer with a bias.
    w["tiny"] = [LayerSpec(1, 0, "L", 16, 1024, 1024, 4, 8.0, 20.0, bias_std=0.01)]
    # 2: OPT-350m-shaped MLP pair (hidden 1024, FFN 4096), 512 tokens.
    w["opt350m_mlp_pair_m512"] = [
        LayerSpec(2, 0, "fc1", 512, 1024, 4096, 1, 6.0, 60.0),
        LayerSpec(2, 1, "fc2", 512, 4096, 1024, 4, 6.0, 60.0),
    ]
    # 3: 7B-shaped prefill, 2048 tokens.
    p7 = []
    for lid, nm in enumerate(["q", "k", "v", "o"]):
        p7.append(LayerSpec(3, lid, nm, 2048, 4096, 4096, 7, 10.0, 60.0))
    p7.append(LayerSpec(3, 4, "gate", 2048, 4096, 11008, 7, 10.0, 60.0))
    p7.append(LayerSpec(3, 5, "up", 2048, 4096, 11008, 7, 10.0, 60.0))
    p7.append(LayerSpec(3, 6, "down", 2048, 11008, 4096, 7, 10.0, 60.0))
    w["llama7b_prefill_m2048"] = p7
    # 4: 13B-shaped decode; m in {1, 4, 16}, 0..8 outlier columns.  Variant id
    # encodes (m, o) so every combination has its own stream.
    d13 = []
    for vi, (m, o) in enumerate([(1, 0), (1, 8), (4, 0), (4, 8), (16, 0), (16, 8),
                                 (1, 1), (4, 4)]):
        d13.append(LayerSpec(4, 0, f"up_m{m}_o{o}", m, 5120, 13824, o, 6.0, 60.0, variant_id=vi))
        d13.append(LayerSpec(4, 1, f"down_m{m}_o{o}", m, 13824, 5120, o, 6.0, 60.0, variant_id=vi))
    w["llama13b_decode"] = d13
    # 5: 65B-shaped prefill, 4096 tokens, heavy-tailed bulk.
    w["llama65b_prefill_m4096"] = [
        LayerSpec(5, 0, "up", 4096, 8192, 22016, 20, 6.0, 100.0, bulk="t3"),
        LayerSpec(5, 1, "down", 4096, 22016, 8192, 20, 6.0, 100.0, bulk="t3"),
    ]
    # the same layers with the heavy tail left untruncated: nearly every
    # column reaches the threshold somewhere, so the linear is almost all fp16
    w["llama65b_prefill_m4096_stress"] = [
        LayerSpec(5, 0, "up", 4096, 8192, 22016, 20, 6.0, 100.0, bulk="t3", variant_id=1, truncate=False),
        LayerSpec(5, 1, "down", 4096, 22016, 8192, 20, 6.0, 100.0, bulk="t3", variant_id=1, truncate=False),
    ]
    return w


WORKLOADS: Dict[str, List[LayerSpec]] = _workloads()


def layer_specs(workload: str) -> List[LayerSpec]:
    return list(WORKLOADS[workload])


def _rng(config_id: int, layer_id: int, tensor_id: int, variant_id: int) -> np.random.Generator:
    return np.random.default_rng([config_id, layer_id, tensor_id, variant_id])


def _bulk(rng: np.random.Generator, size: int, bulk: str) -> np.ndarray:
    if bulk == "normal":
        return rng.standard_normal(size, dtype=np.float32)
    if bulk == "t3":
        return (rng.standard_t(3, size) / np.sqrt(3.0)).astype(np.float32)
    raise ValueError(f"unknown bulk distribution {bulk!r}")


def draw_activations(m: int, k: int, n_outlier: int, lo: float, hi: float, *,
                     bulk: str = "normal", tau: float = TAU_DEFAULT,
                     seed: Tuple[int, int, int] = (0, 0, 0),
                     outlier_row_frac: float = 1.0,
                     truncate: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 activations [m, k] with ``n_outlier`` planted columns.

    ``seed`` = (config_id, layer_id, variant_id).  Returns (x, planted_cols),
    planted_cols sorted ascending.  With ``outlier_row_frac`` < 1 only a seeded
    subset of rows in each planted column is large (the others keep their bulk
    draw), which exercises rows whose largest small element sits in an outlier
    column.  ``truncate=False`` keeps the raw heavy tail (stress input).
    """
    cfg, lay, var = seed
    r0 = _rng(cfg, lay, 0, var)
    x = _bulk(r0, m * k, bulk).astype(np.float16)
    if truncate and tau > 0:
        lim = np.float16(tau)
        bad = np.abs(x) >= lim
        while bad.any():
            x[bad] = _bulk(r0, int(bad.sum()), bulk).astype(np.float16)
            bad = np.abs(x) >= lim
    x = x.reshape(m, k)
    r1 = _rng(cfg, lay, 1, var)
    n_outlier = min(n_outlier, k)
    cols = np.sort(r1.choice(k, size=n_outlier, replace=False)) if n_outlier else np.zeros(0, np.int64)
    for c in cols:
        sign = np.where(r1.random(m) < 0.5, -1.0, 1.0)
        mag = r1.uniform(lo, hi, m)
        vals = (sign * mag).astype(np.float16)
        if outlier_row_frac >= 1.0:
            x[:, c] = vals
        else:
            rows = r1.random(m) < outlier_row_frac
            if not rows.any():
                rows[r1.integers(m)] = True
            x[rows, c] = vals[rows]
    return x, cols.astype(np.int64)


def draw_weight(n: int, k: int, *, seed: Tuple[int, int, int] = (0, 0, 0),
                std: float = 0.02) -> np.ndarray:
    cfg, lay, var = seed
    r2 = _rng(cfg, lay, 2, var)
    return (r2.standard_normal(n * k, dtype=np.float32) * np.float32(std)).astype(np.float16).reshape(n, k)


def draw_bias(n: int, *, seed: Tuple[int, int, int] = (0, 0, 0), std: float = 0.01) -> np.ndarray:
    cfg, lay, var = seed
    r3 = _rng(cfg, lay, 3, var)
    return (r3.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float16)


def draw_grad(m: int, n: int, *, seed: Tuple[int, int, int] = (0, 0, 0), std: float = 1.0) -> np.ndarray:
    """fp16 upstream gradient dL/dy [m, n]: seeded normal draws times ``std``."""
    cfg, lay, var = seed
    r4 = _rng(cfg, lay, 4, var)
    return (r4.standard_normal(m * n, dtype=np.float32) * np.float32(std)).astype(np.float16).reshape(m, n)


@dataclass
class Layer:
    spec: LayerSpec
    x: np.ndarray                 # fp16 [m, k]
    w: np.ndarray                 # fp16 [n, k]
    bias: Optional[np.ndarray]    # fp16 [n] or None
    planted_cols: np.ndarray      # int64, sorted
    seed: Tuple[int, int, int, int] = field(default=(0, 0, 0, 0))


def make_inputs(m: int, k: int, n: int, *, n_outlier: int = 0, lo: float = 6.0, hi: float = 60.0,
                bulk: str = "normal", bias_std: Optional[float] = None, tau: float = TAU_DEFAULT,
                seed: Tuple[int, int, int] = (0, 0, 0), outlier_row_frac: float = 1.0,
                with_weight: bool = True) -> Layer:
    """Any-shape seeded layer (used by the parity tests' edge cases)."""
    x, cols = draw_activations(m, k, n_outlier, lo, hi, bulk=bulk, tau=tau, seed=seed,
                               outlier_row_frac=outlier_row_frac)
    w = draw_weight(n, k, seed=seed) if with_weight else np.zeros((0, k), np.float16)
    b = draw_bias(n, seed=seed, std=bias_std) if bias_std is not None else None
    spec = LayerSpec(seed[0], seed[1], "custom", m, k, n, n_outlier, lo, hi, bulk, bias_std, tau, seed[2])
    return Layer(spec, x, w, b, cols, (seed[0], seed[1], -1, seed[2]))


def make_layer(spec: LayerSpec, *, with_weight: bool = True, m: Optional[int] = None) -> Layer:
    """Draw the tensors of one workload layer (``m`` overrides the row count)."""
    seed = (spec.config_id, spec.layer_id, spec.variant_id)
    mm = spec.m if m is None else m
    x, cols = draw_activations(mm, spec.k, spec.n_outlier, spec.outlier_lo, spec.outlier_hi,
                               bulk=spec.bulk, tau=spec.tau, seed=seed, truncate=spec.truncate)
    w = draw_weight(spec.n, spec.k, seed=seed) if with_weight else np.zeros((0, spec.k), np.float16)
    b = draw_bias(spec.n, seed=seed, std=spec.bias_std) if spec.bias_std is not None else None
    return Layer(spec, x, w, b, cols, (spec.config_id, spec.layer_id, -1, spec.variant_id))
