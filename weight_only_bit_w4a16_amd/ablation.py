"""The pages' ablations, reported as layer-output errors on the device.

AWQ Explained: Protecting the Weights That Matter Most ("The premise: 1% of
channels", "Why the activations pick, not the weights") and the Real Python
glossary compare, by perplexity, keeping about 1% of salient input channels
in FP16 with plain round-to-nearest, choosing those channels by activation
or by weight magnitude, and AWQ's scaling. With no model or corpus here the
same comparison is made on one layer's output error on the calibration
batch, ||Xcal (W - What)^T||_F^2, with every loss evaluated by the library:

* rtn: plain round-to-nearest (the search at alpha = 0);
* awq: the best loss of the alpha grid search;
* fp16_act / fp16_weight: RTN with the salient channels kept in FP16,
  chosen by mean |x| (the activation statistic) or by mean |W| over the
  column. Keeping a column exact zeroes that column of W - What, which is
  the RTN loss of a batch whose column is zero; the batch is masked with
  the library's fold, dividing the masked channels by 2^127 (an fp16 value
  over 2^127 rounds to zero).

Only the choice of the salient channels (a sort of K scores) runs on the
host.
"""
from __future__ import annotations

import numpy as np

from . import act_stats, fold_inv_scale, scale_search

_MASK_SCALE = np.float32(2.0 ** 127)


def _torch():
    import torch
    return torch


def weight_channel_magnitude(W, chunk_rows: int = 4096):
    """mean_n |W[n, k]| per input channel (float64 [K], numpy), from the
    activation-statistic kernel over equal row chunks (an exact float64 sum
    per chunk)."""
    N = W.shape[0]
    c = min(chunk_rows, N)
    while N % c:
        c -= 1
    parts = [act_stats(W[i:i + c]).cpu().numpy() for i in range(0, N, c)]
    return np.mean(parts, axis=0)


def salient(score, count: int) -> np.ndarray:
    """The `count` largest scores, ties to the lower index, sorted."""
    score = np.asarray(score, dtype=np.float64)
    order = np.lexsort((np.arange(len(score)), -score))
    return np.sort(order[:count])


def masked(xcal, channels):
    """xcal with the given input channels set to zero (on the device)."""
    torch = _torch()
    s = np.ones(xcal.shape[1], dtype=np.float32)
    s[np.asarray(channels, dtype=np.int64)] = _MASK_SCALE
    return fold_inv_scale(xcal, torch.from_numpy(s).to(xcal.device))


def ablation(W, xcal, bits: int = 4, group: int = 128, frac: float = 0.01, alpha_grid=None,
             zero_point: bool = True):
    """Layer-output errors of RTN, AWQ and FP16-kept salient channels.

    W: fp16 [N, K] and xcal: fp16 [T, K] device tensors. Returns a dict
    with the four losses, the chosen alpha index and the channel sets.
    """
    K = W.shape[1]
    n = max(1, int(round(frac * K)))
    sel_act = salient(act_stats(xcal).cpu().numpy(), n)
    sel_w = salient(weight_channel_magnitude(W), n)
    zero = np.zeros(1, dtype=np.float32)
    rtn = scale_search(W, xcal, zero, bits, group, zero_point=zero_point)[2][0]
    _, best, losses = scale_search(W, xcal, alpha_grid, bits, group, zero_point=zero_point)
    kept_act = scale_search(W, masked(xcal, sel_act), zero, bits, group,
                            zero_point=zero_point)[2][0]
    kept_w = scale_search(W, masked(xcal, sel_w), zero, bits, group, zero_point=zero_point)[2][0]
    return {
        "rtn": float(rtn), "awq": float(losses[best]), "awq_best_index": int(best),
        "fp16_act": float(kept_act), "fp16_weight": float(kept_w),
        "channels_act": sel_act, "channels_weight": sel_w, "kept": n,
    }
