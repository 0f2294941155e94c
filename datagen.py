"""Seeded synthetic inputs for the AWQ W4A16 hot path.

This module only draws random numbers and holds the workload table. It
contains none of the method's arithmetic (no statistics, no scaling, no
quantization), so that the CPU oracle and the HIP path can both be fed from
it without sharing any computation.

Every tensor comes from its own counter-seeded stream:
``numpy.random.default_rng(SeedSequence([0xA3A, workload_id, stream_id]))``.
Values are drawn as float32 standard normals, scaled in float32 and cast to
float16 with round-half-to-even.

Workloads are LLM-shaped linear layers (the pages name LLaMA-class models as
the usual AWQ targets but ship no weights). Weights are N(0, 0.02) (0.02 is
read as the standard deviation). Activations are N(0, 1) with a fixed set of
"outlier" input channels multiplied by a constant: the salient-channel
premise of the pages (a small fraction, about 1%, of input channels carry
much larger activation magnitudes; AWQ Explained: Protecting the Weights That
Matter Most -- "The premise: 1% of channels" and "Why the activations pick,
not the weights"). The same channel set is used for the calibration batch and
for the decode/prefill activations, because outliers are a property of the
hidden dimension, not of a token.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_ROOT = 0xA3A

# stream ids inside one workload
STREAM_WEIGHT = 1
STREAM_OUTLIER_CHANNELS = 2
STREAM_CALIB = 3
STREAM_GATE_WEIGHT = 4
STREAM_ACT = 100  # + M, so that every batch size has its own stream


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int           # seed id of the workload
    K: int             # input channels
    N: int             # output channels
    bits: int
    group: int
    T: int             # calibration tokens
    n_outlier: int     # outlier input channels
    outlier_gain: float
    decode_M: tuple = ()
    prefill_M: tuple = ()
    n_alpha: int = 20

    @property
    def all_M(self):
        return tuple(self.decode_M) + tuple(self.prefill_M)


def _pct_outliers(K: int) -> int:
    return int(round(0.01 * K))


WORKLOADS = {w.name: w for w in [
    Workload("tiny_512x512_int4", 1, 512, 512, 4, 128, 64, 5, 40.0,
             decode_M=(1,)),
    Workload("llama7b_attn_4096x4096_int4", 2, 4096, 4096, 4, 128, 512,
             _pct_outliers(4096), 50.0, decode_M=(1, 4, 16)),
    Workload("llama7b_mlp_up_4096x11008_int4", 3, 4096, 11008, 4, 128, 512,
             _pct_outliers(4096), 50.0, decode_M=(1, 8)),
    Workload("llama7b_mlp_down_11008x4096_int4", 4, 11008, 4096, 4, 128, 512,
             _pct_outliers(11008), 50.0, decode_M=(1, 8)),
    Workload("llama7b_mlp_up_4096x11008_int3", 5, 4096, 11008, 3, 128, 512,
             _pct_outliers(4096), 50.0, decode_M=(1,), prefill_M=(256,)),
    Workload("llama7b_mlp_down_11008x4096_int3", 6, 11008, 4096, 3, 128, 512,
             _pct_outliers(11008), 50.0, decode_M=(1,), prefill_M=(256,)),
    Workload("llama70b_mlp_8192x28672_int4", 7, 8192, 28672, 4, 128, 512,
             _pct_outliers(8192), 50.0, decode_M=(1,), prefill_M=(2048,)),
]}

# the workload the headline numbers are quoted on
HEADLINE = "llama70b_mlp_8192x28672_int4"
SMALL = "tiny_512x512_int4"


def rng(wid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, wid, stream]))


def normal_f16(shape, std: float, wid: int, stream: int) -> np.ndarray:
    g = rng(wid, stream)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x.astype(np.float16)


def outlier_channels(K: int, count: int, wid: int) -> np.ndarray:
    """Sorted indices of `count` distinct input channels."""
    g = rng(wid, STREAM_OUTLIER_CHANNELS)
    return np.sort(g.choice(K, size=count, replace=False)).astype(np.int64)


def weight(w: Workload) -> np.ndarray:
    """fp16 [N, K], row = output channel (PyTorch Linear layout)."""
    return normal_f16((w.N, w.K), 0.02, w.wid, STREAM_WEIGHT)


def gate_weight(w: Workload) -> np.ndarray:
    """fp16 [N, K]: the gate projection beside an up projection of the same
    shape (a gated MLP), drawn like `weight` from its own stream."""
    return normal_f16((w.N, w.K), 0.02, w.wid, STREAM_GATE_WEIGHT)


def activations(w: Workload, rows: int, stream: int) -> np.ndarray:
    """fp16 [rows, K] ~ N(0,1) with the workload's outlier channels scaled."""
    x = rng(w.wid, stream).standard_normal(size=(rows, w.K), dtype=np.float32)
    ch = outlier_channels(w.K, w.n_outlier, w.wid)
    x[:, ch] *= np.float32(w.outlier_gain)
    return x.astype(np.float16)


def calibration(w: Workload) -> np.ndarray:
    return activations(w, w.T, STREAM_CALIB)


def decode_input(w: Workload, M: int) -> np.ndarray:
    return activations(w, M, STREAM_ACT + M)


def alpha_grid(n: int = 20) -> np.ndarray:
    """Default grid: alpha_i = i/n for i = 0..n-1 (includes 0, stays in [0,1])."""
    return (np.arange(n, dtype=np.float64) / n).astype(np.float32)


def small_layer(K: int, N: int, T: int, n_outlier: int, gain: float, seed: int):
    """A small ad-hoc layer for tests: (W fp16 [N,K], Xcal fp16 [T,K], channels)."""
    wid = 1000 + seed
    W = normal_f16((N, K), 0.02, wid, STREAM_WEIGHT)
    x = rng(wid, STREAM_CALIB).standard_normal(size=(T, K), dtype=np.float32)
    ch = np.sort(rng(wid, STREAM_OUTLIER_CHANNELS).choice(K, size=n_outlier, replace=False))
    x[:, ch] *= np.float32(gain)
    return W, x.astype(np.float16), ch


def random_f16(shape, std: float, seed: int) -> np.ndarray:
    return normal_f16(shape, std, 2000 + seed, 0)


def random_f32_positive(n: int, lo: float, hi: float, seed: int) -> np.ndarray:
    g = rng(3000 + seed, 0)
    return g.uniform(lo, hi, size=n).astype(np.float32)
