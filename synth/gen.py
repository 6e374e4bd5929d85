"""Seeded synthetic workloads.

Recipe (one numpy Generator per tensor, spawned from one SeedSequence):
  stream 0: X ~ N(0, 1) of shape [M, K];
  stream 1: the outlier channels: max(1, rint(0.01*K)) distinct columns of X,
            each multiplied by 30 (the pages' "1% of channels" outlier
            structure of diffusion-transformer activations);
  stream 2: W = noise + planted, noise ~ N(0, 0.02^2) of shape [K, N] and
            planted = A @ B with A [K, k], B [k, N] standard normal, rescaled so
            that ||planted||_F = 5 ||noise||_F (a steep leading spectrum);
  stream 3: bias ~ N(0, 0.01^2) of shape [N].
Every tensor is rounded to fp16 once, at the end.  The draws are float64.

The configurations are the five workloads the layer is measured on: a tiny
layer, a FLUX-like fused QKV projection, a FLUX-like MLP pair, a small-batch
sweep of the MLP's first linear, and the FP4 / INT8 settings of that linear.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class LayerShape:
    name: str
    M: int
    K: int
    N: int
    r: int
    fmt: str            # "int4", "int8" or "fp4"
    seed: int
    planted_rank: int
    m_rows: Optional[int] = None   # evaluate on the first m_rows tokens only


@dataclass
class RawLayer:
    """Raw (unsmoothed) fp16 operands of one linear layer, Y = X W + b."""
    shape: LayerShape
    x: np.ndarray      # fp16 [M, K]
    w: np.ndarray      # fp16 [K, N]
    b: np.ndarray      # fp16 [N]
    outlier_cols: np.ndarray = field(default=None)


def _streams(seed: int, n: int = 4) -> List[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def draw_activations(seed: int, M: int, K: int):
    """X ~ N(0,1) [M,K] with 1% of its channels scaled x30; returns (fp16 X, outlier columns)."""
    g = _streams(seed)
    x = g[0].standard_normal((M, K))
    n_out = max(1, int(np.rint(0.01 * K)))
    cols = np.sort(g[1].choice(K, size=n_out, replace=False))
    x[:, cols] *= 30.0
    return x.astype(np.float16), cols


def draw_weight(seed: int, K: int, N: int, planted_rank: int) -> np.ndarray:
    """W = N(0, 0.02^2) noise + a rank-`planted_rank` part with 5x the noise's Frobenius norm (fp16 [K,N])."""
    g = _streams(seed)[2]
    noise = g.standard_normal((K, N)) * 0.02
    a = g.standard_normal((K, planted_rank))
    bm = g.standard_normal((planted_rank, N))
    planted = a @ bm
    planted *= 5.0 * np.linalg.norm(noise) / np.linalg.norm(planted)
    return (noise + planted).astype(np.float16)


def draw_bias(seed: int, N: int) -> np.ndarray:
    g = _streams(seed)[3]
    return (g.standard_normal(N) * 0.01).astype(np.float16)


def draw_layer(shape: LayerShape, weight_seed: Optional[int] = None) -> RawLayer:
    ws = shape.seed if weight_seed is None else weight_seed
    x, cols = draw_activations(shape.seed, shape.M, shape.K)
    w = draw_weight(ws, shape.K, shape.N, shape.planted_rank)
    b = draw_bias(ws, shape.N)
    return RawLayer(shape, x, w, b, cols)


def gelu_tanh_f64(y: np.ndarray) -> np.ndarray:
    """The tanh form of GELU, 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))), in float64."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)))


def fc2_calibration_input(fc1: RawLayer) -> np.ndarray:
    """Input the 16-bit MLP feeds its second linear: fp16(gelu(fp16(X W1 + b1))).

    This is the unquantized model's activation (the workload), used to calibrate
    the second layer's smoothing; it is not part of the quantized layer.
    """
    y1 = fc1.x.astype(np.float32) @ fc1.w.astype(np.float32) + fc1.b.astype(np.float32)
    return gelu_tanh_f64(y1.astype(np.float16)).astype(np.float16)


# --------------------------------------------------------------------------- configs
# name -> list of layer shapes.  M/K/N/r/format follow the five workloads.
CONFIGS: Dict[str, List[LayerShape]] = {
    "c0_tiny": [LayerShape("c0", 128, 256, 256, 32, "int4", 1000, 8)],
    "c1_qkv": [LayerShape("c1_qkv", 4608, 3072, 9216, 32, "int4", 1001, 16)],
    "c2_mlp": [LayerShape("c2_fc1", 4608, 3072, 12288, 32, "int4", 1002, 16),
               LayerShape("c2_fc2", 4608, 12288, 3072, 32, "int4", 1012, 16)],
    "c3_sweep": [LayerShape(f"c3_m{m}", 4608, 3072, 12288, 32, "int4", 1002, 16, m_rows=m)
                 for m in (64, 256, 1024)],
    "c4_formats": [LayerShape("c4_fp4", 4608, 3072, 12288, 32, "fp4", 1002, 16),
                   LayerShape("c4_int8", 4608, 3072, 12288, 16, "int8", 1002, 16)],
}


def config_layers(name: str) -> List[LayerShape]:
    return CONFIGS[name]
