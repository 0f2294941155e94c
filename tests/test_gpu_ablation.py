"""GPU parity of the ablation harness (weight_only_bit_w4a16_amd.ablation):
every loss within 1e-4 of the oracle's direct evaluation (FP16 columns
restored into the dequantized matrix), the same salient channels, and the
pages' orderings on the 4096-wide layer."""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from weight_only_bit_w4a16_amd import ablation as A  # noqa: E402
from tests.test_gpu_parity import dev, host, say  # noqa: E402


def _check(W, Xc, bits, group, zero_point=True):
    r = A.ablation(dev(W), dev(Xc), bits, group, zero_point=zero_point)
    n = r["kept"]
    sa = O.salient_channels(O.act_stats(Xc), n)
    sw = O.salient_channels(O.weight_channel_magnitude(W), n)
    assert np.array_equal(r["channels_act"], sa)
    assert np.array_equal(r["channels_weight"], sw)
    ref = {
        "rtn": O.layer_loss(Xc, W, np.ones(W.shape[1], np.float32), bits, group, zero_point),
        "fp16_act": O.layer_loss_fp16_kept(Xc, W, sa, bits, group, zero_point),
        "fp16_weight": O.layer_loss_fp16_kept(Xc, W, sw, bits, group, zero_point),
        "awq": O.layer_loss(Xc, W, O.scale_from_stats(O.act_stats(Xc),
                                                      datagen.alpha_grid(20)[r["awq_best_index"]]),
                            bits, group, zero_point),
    }
    for k, v in ref.items():
        assert abs(r[k] - v) <= 1e-4 * v, (k, r[k], v)
    return r


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("zero_point", [True, False])
def test_ablation_tiny(bits, zero_point):
    w = datagen.WORKLOADS["tiny_512x512_int4"]
    _check(datagen.weight(w), datagen.calibration(w), bits, 128, zero_point)


def test_ablation_orderings():
    w = datagen.WORKLOADS["llama7b_attn_4096x4096_int4"]
    say("ablation", w.name)
    r = _check(datagen.weight(w)[:512], datagen.calibration(w), 4, 128)
    assert r["fp16_act"] < 0.1 * r["rtn"]
    assert r["fp16_weight"] > 0.9 * r["rtn"]
    assert r["awq"] < 0.3 * r["rtn"]


def test_masked_batch_is_zero_on_the_channels():
    X = datagen.random_f16((7, 512), 30.0, seed=9)
    ch = [0, 5, 511]
    Xm = host(A.masked(dev(X), ch))
    assert np.all(Xm[:, ch] == 0)
    keep = np.setdiff1d(np.arange(512), ch)
    assert np.array_equal(Xm[:, keep], X[:, keep])
