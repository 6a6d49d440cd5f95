"""Seeded synthetic inputs for the H-BitLinear forward pass.

This module only draws numbers; it holds none of the method's arithmetic.  It
serves both the CPU oracle and the HIP path, which read the same host arrays.

The pages measure on trained BitNet v2 models (1.3B / 3B / 7B) and public
evaluation suites that are not available here; these generators stand in for
the activations that reach the attention output projection Wo and the FFN
down projection Wdown.  Their shape follows what the pages say about those
activations: a few outlier channels and most of the mass near zero (the
activation-distribution figures of the "新智元: 微软 BitNet v2" repost,
section "H-BitLinear模块"), Gaussian inputs for the other projections (same
section), and a SwiGLU product in front of Wdown (section
"BitNet v2：原生4位激活").  Layer widths are those of LLaMA-like 1.3B / 3B / 7B
models.

Conventions
  * ``numpy.random.default_rng(seed)``; draw order: X, then the outlier-channel
    choice, then the latent weights W.
  * bf16 inputs are produced by round-to-nearest-even from fp32 and returned as
    uint16 bit patterns (numpy has no bf16 dtype).
  * Latent weights: W ~ N(0, 0.02) in fp32, shape [N][K] (out x in).
"""
from __future__ import annotations

import dataclasses

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN-free inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- X draws --
def x_outlier_gaussian(rng, M, K, n_outliers=4, factor=30.0):
    """N(0,1) with `n_outliers` channels (columns) scaled by `factor`."""
    X = rng.standard_normal((M, K), dtype=np.float32)
    ch = rng.choice(K, size=min(n_outliers, K), replace=False)
    X[:, ch] *= np.float32(factor)
    return X, ch


def x_laplace_mixture(rng, M, K, p_laplace=0.9, b=0.05, outlier_frac=0.01, factor=50.0):
    """Each element Laplace(0, b) with probability p, else N(0,1); then a
    fraction of channels (rounded to nearest, at least 1) scaled by `factor`."""
    lap = rng.laplace(0.0, b, size=(M, K)).astype(np.float32)
    nrm = rng.standard_normal((M, K), dtype=np.float32)
    pick = rng.random((M, K)) < p_laplace
    X = np.where(pick, lap, nrm).astype(np.float32)
    n_out = max(1, int(round(outlier_frac * K)))
    ch = rng.choice(K, size=n_out, replace=False)
    X[:, ch] *= np.float32(factor)
    return X, ch


def x_swiglu(rng, M, K):
    """SiLU(a) * b with a, b iid N(0,1) (heavy tailed, like a SwiGLU output)."""
    a = rng.standard_normal((M, K), dtype=np.float32)
    b = rng.standard_normal((M, K), dtype=np.float32)
    silu = a / (np.float32(1.0) + np.exp(-a))
    return (silu * b).astype(np.float32), np.zeros(0, np.int64)


def x_gaussian(rng, M, K):
    return rng.standard_normal((M, K), dtype=np.float32), np.zeros(0, np.int64)


def head_states(rng, M, H, D):
    """Post-RoPE attention states [M][H][D]: N(0,1) values with a log-normal
    scale per (token, head) (sigma 1), so head vectors span several orders of
    magnitude as keys and values of different heads do."""
    x = rng.standard_normal((M, H, D)).astype(np.float32)
    return (x * np.exp(rng.standard_normal((M, H, 1))).astype(np.float32)).astype(np.float32)


# Attention states of a 3B-like model (hidden 4096 = 32 heads x 128) for 8192
# tokens, quantised to a 3-bit KV cache: (name, M, H, D, bits).
KV_3B = ("kv_3b", 8192, 32, 128, 3)


def w_latent(rng, N, K, std=0.02):
    return (rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


# ----------------------------------------------------------------- layers --
@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer of a workload."""
    name: str
    M: int
    K: int
    N: int
    act_bits: int          # 8 or 4
    hadamard: bool         # True: H-BitLinear, False: plain BitLinear
    x_dtype: str           # "f32" or "bf16"
    y_dtype: str           # "f32" or "bf16"
    gen: str               # X generator name
    gen_args: tuple = ()

    @property
    def desc(self) -> str:
        kind = "H-BitLinear" if self.hadamard else "BitLinear"
        return "%s %s M=%d K=%d N=%d a%d %s->%s" % (self.name, kind, self.M, self.K, self.N,
                                                   self.act_bits, self.x_dtype, self.y_dtype)


_GENS = {
    "outlier_gaussian": x_outlier_gaussian,
    "laplace_mixture": x_laplace_mixture,
    "swiglu": x_swiglu,
    "gaussian": x_gaussian,
}


def make_inputs(layer: Layer, seed: int = 0, M: int | None = None):
    """Draw (X, W, outlier_channels) for a layer.  X is fp32 or bf16 bits per
    layer.x_dtype; W is fp32 [N][K].  `M` overrides the row count (the draws for
    the first rows do not depend on it only when the generator draws row-major,
    so callers that sample rows should draw the full layer)."""
    rng = np.random.default_rng(seed)
    rows = layer.M if M is None else M
    X, ch = _GENS[layer.gen](rng, rows, layer.K, *layer.gen_args)
    W = w_latent(rng, layer.N, layer.K)
    if layer.x_dtype == "bf16":
        X = f32_to_bf16_bits(X)
    return X, W, ch


# --------------------------------------------------------------- workloads --
# Small single layer (parity case the oracle finishes in well under a second).
SMALL = Layer("small", 8, 256, 256, 8, True, "f32", "f32", "outlier_gaussian", (4, 30.0))
# Attention output projection Wo of a 1.3B-like model (hidden 2048), INT8 activations.
WO_1P3B = Layer("wo_1.3b", 4096, 2048, 2048, 8, True, "bf16", "bf16", "laplace_mixture", (0.9, 0.05, 0.01, 50.0))
# FFN down projection Wdown of a 7B-like model (FFN 16384 -> hidden 4096), INT4 activations.
WDOWN_7B = Layer("wdown_7b", 8192, 16384, 4096, 4, True, "bf16", "bf16", "swiglu")


def decode_layer(M: int) -> Layer:
    """Decode regime: M tokens against a K=8192 -> N=4096 ternary layer, INT4."""
    return Layer("decode_m%d" % M, M, 8192, 4096, 4, True, "f32", "bf16", "outlier_gaussian", (4, 30.0))


DECODE = tuple(decode_layer(m) for m in (1, 16, 64))

# Full 3B-like layer chain at hidden 4096, FFN 16384, 8192 tokens, all INT4:
# QKV and gate/up are plain BitLinear (Gaussian inputs), Wo and Wdown are
# H-BitLinear (outlier / SwiGLU inputs).
CHAIN_3B = (
    Layer("qkv_3b", 8192, 4096, 12288, 4, False, "bf16", "bf16", "gaussian"),
    Layer("gateup_3b", 8192, 4096, 32768, 4, False, "bf16", "bf16", "gaussian"),
    Layer("wo_3b", 8192, 4096, 4096, 4, True, "bf16", "bf16", "laplace_mixture", (0.9, 0.05, 0.01, 50.0)),
    Layer("wdown_3b", 8192, 16384, 4096, 4, True, "bf16", "bf16", "swiglu"),
)

ALL = (SMALL, WO_1P3B, WDOWN_7B) + DECODE + CHAIN_3B


def by_name(name: str) -> Layer:
    for l in ALL:
        if l.name == name:
            return l
    raise KeyError(name)


def sample_rows(M: int, count: int = 64) -> np.ndarray:
    """Evenly spaced row indices including the first and the last."""
    if M <= count:
        return np.arange(M)
    return np.unique(np.linspace(0, M - 1, count).round().astype(np.int64))
