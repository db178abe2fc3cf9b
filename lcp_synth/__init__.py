"""Seeded synthetic inputs for one learnable-channel-permutation (LCP) step.

This module is shared by the tests, the smoke check and the benchmark. It
draws random numbers and rounds them to the storage type; it performs none of
the method's arithmetic (no Sinkhorn, no permutation, no mask, no error), so
the float64 oracle and the GPU library stay independent of each other.

The pages measure on real LLaMA / Qwen / OPT layers with C4 calibration text
(PermLLM summary page, "Experimental setup: datasets and models"). Neither the
weights nor the data exist here, so seeded synthetic layers with LLaMA layer
shapes stand in for them. Each generated layer carries:

* ``W``      Cout x Cin weight, row-major like a linear layer, N(0, w_std^2);
* ``X``      T x Cin calibration activations, N(0, 1) times a per-channel
             structure (lognormal channel scales, or a few outlier channels
             multiplied by a constant factor);
* ``logits`` nb x B x B block logits, 3*I + N(0, 1e-3^2) per block.

Storage types: ``"bf16"`` layers are drawn in float32 and rounded to bfloat16
with round-to-nearest-even; ``"f32"`` layers stay float32. Logits are always
float32. The arrays returned are float32 holding exactly the stored values,
plus the raw bfloat16 bit patterns (uint16) for bf16 layers.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BASE_SEED = 20251010


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    cout: int
    cin: int
    T: int
    dtype: str          # "f32" or "bf16"
    w_std: float
    x_kind: str         # "lognormal" or "outliers"
    x_param: float      # lognormal sigma, or outlier fraction
    x_factor: float     # outlier multiplier (unused for lognormal)
    B: int
    iters: int
    tau: float
    N: int
    M: int
    backward: bool

    @property
    def nb(self) -> int:
        return self.cin // self.B


# Five synthetic layers. Shapes follow LLaMA projections; B, iterations, N:M
# and the forward/backward split per layer are the ones the hot path is
# specified and measured on. tau = 1 is the start of the 1 -> 0.1 linear
# temperature schedule of the PermLLM implementation details.
CONFIGS = [
    LayerSpec("C1-256x256-f32", 256, 256, 256, "f32", 0.02, "lognormal", 0.5, 0.0,
              32, 5, 1.0, 2, 4, False),
    LayerSpec("C2-llama7b-q_proj", 4096, 4096, 2048, "bf16", 0.02, "outliers", 0.01, 20.0,
              64, 5, 1.0, 2, 4, False),
    LayerSpec("C3-llama7b-down_proj", 4096, 11008, 2048, "bf16", 0.02, "lognormal", 1.0, 0.0,
              64, 5, 1.0, 2, 4, True),
    LayerSpec("C4-llama13b-up_proj", 13824, 5120, 4096, "bf16", 0.02, "outliers", 0.005, 50.0,
              128, 7, 1.0, 4, 8, True),
    LayerSpec("C5-llama70b-up_proj", 28672, 8192, 2048, "bf16", 0.015, "lognormal", 1.0, 0.0,
              64, 5, 1.0, 2, 4, True),
]

# the same layers by name
F32_256x256, Q_PROJ_4096x4096, DOWN_PROJ_4096x11008, UP_PROJ_13824x5120, UP_PROJ_28672x8192 = CONFIGS

BENCH_CONFIG = CONFIGS.index(DOWN_PROJ_4096x11008)  # forward + backward, the measured layer


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs here are finite, so no NaN special case is needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    W: np.ndarray            # float32, exactly the stored values
    X: np.ndarray            # float32, exactly the stored values
    logits: np.ndarray       # float32 [nb, B, B]
    W_bits: Optional[np.ndarray] = None   # uint16 when dtype == "bf16"
    X_bits: Optional[np.ndarray] = None

    @property
    def cout(self): return self.W.shape[0]

    @property
    def cin(self): return self.W.shape[1]

    @property
    def T(self): return self.X.shape[0]


def make_logits(rng: np.random.Generator, nb: int, B: int, diag: float = 3.0,
                noise_std: float = 1e-3) -> np.ndarray:
    """Per block diag*I + N(0, noise_std^2), float32 [nb, B, B]."""
    eye = np.eye(B, dtype=np.float64)[None, :, :]
    lg = diag * eye + rng.normal(0.0, noise_std, size=(nb, B, B))
    return lg.astype(np.float32)


def make_layer(spec: LayerSpec, seed: Optional[int] = None, cout: Optional[int] = None,
               cin: Optional[int] = None, T: Optional[int] = None,
               dtype: Optional[str] = None) -> Layer:
    """Draw one seeded layer. Sizes default to the spec's; smaller sizes give
    layers with the same value distributions for tests the oracle can finish
    quickly. Streams for W, X, channel scales, outlier picks and logits come
    from one SeedSequence so changing one size does not shift the others.
    """
    cout = spec.cout if cout is None else cout
    cin = spec.cin if cin is None else cin
    T = spec.T if T is None else T
    dtype = spec.dtype if dtype is None else dtype
    if cin % spec.B:
        raise ValueError("cin must be a multiple of B")
    if seed is None:
        seed = BASE_SEED + CONFIGS.index(spec) if spec in CONFIGS else BASE_SEED
    ss = np.random.SeedSequence(seed)
    s_w, s_x, s_scale, s_out, s_log = [np.random.Generator(np.random.PCG64(s))
                                        for s in ss.spawn(5)]

    W = s_w.normal(0.0, spec.w_std, size=(cout, cin)).astype(np.float32)
    X = s_x.normal(0.0, 1.0, size=(T, cin)).astype(np.float32)
    if spec.x_kind == "lognormal":
        scale = s_scale.lognormal(0.0, spec.x_param, size=cin).astype(np.float32)
        X *= scale[None, :]
    elif spec.x_kind == "outliers":
        n_out = int(round(spec.x_param * cin))
        idx = s_out.choice(cin, size=n_out, replace=False)
        X[:, idx] *= np.float32(spec.x_factor)
    else:
        raise ValueError(spec.x_kind)
    logits = make_logits(s_log, cin // spec.B, spec.B)

    if dtype == "bf16":
        wb = f32_to_bf16_bits(W)
        xb = f32_to_bf16_bits(X)
        return Layer(spec, bf16_bits_to_f32(wb), bf16_bits_to_f32(xb), logits, wb, xb)
    if dtype == "f32":
        return Layer(spec, W, X, logits)
    raise ValueError(dtype)


def random_logits(seed: int, nb: int, B: int, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) logits, float32 [nb, B, B] (harder than the 3*I start)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (scale * rng.standard_normal((nb, B, B))).astype(np.float32)


def planted_logits(seed: int, nb: int, B: int, peak: float = 3.0, noise_std: float = 0.1):
    """Per block peak*Pi_b + N(0, noise_std^2) with a random permutation matrix
    Pi_b (Pi_b[j, pi_b(j)] = 1); returns (float32 logits [nb, B, B], Pi as
    float64 [nb, B, B])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Pi = np.zeros((nb, B, B))
    for b in range(nb):
        Pi[b, np.arange(B), rng.permutation(B)] = 1.0
    lg = peak * Pi + rng.normal(0.0, noise_std, size=(nb, B, B))
    return lg.astype(np.float32), Pi


def random_matrix(seed: int, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """Seeded N(0, std^2) matrix as float32 values (bf16-representable for bf16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = (std * rng.standard_normal(shape)).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    return a
