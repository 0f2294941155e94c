"""The search and the quantize-and-pack step on every workload layer at full
size, against the oracle.

Search: the device's 20-point loss curve over the whole matrix against the
oracle's full curve (tests/golden/workload_search.json, written by
make_workload_search.py in the same folder from the oracle alone: a full
curve costs the oracle minutes per layer). Contract (AWQ Explained:
Protecting the Weights That Matter Most -- "How the scale is chosen": the
exponent is the grid point with the smallest layer-output error):
  * every loss within 1e-4 relative of the oracle's;
  * the device's index is the first minimum of its own curve, and equals the
    oracle's or is a near-tie: L_oracle[i_dev] <= (1 + 1e-4) L_oracle[i_oracle];
  * s bit-exact when the indices agree.

Pack: codes, scales and zero points of the whole matrix at the oracle's
chosen s, bit for bit, with the oracle computed here.
"""
import functools
import json
import os

import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import assert_same_bits, dev, host, say  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "workload_search.json")


@functools.lru_cache(maxsize=1)
def golden():
    with open(GOLDEN) as f:
        doc = json.load(f)
    return {(e["kind"], e["workload"], e["zero_point"]): e for e in doc["entries"]}


def check_curve(loss_g, best_g, entry, grid):
    assert np.array_equal(np.asarray(entry["alpha_grid"], np.float32), grid)
    loss_o = np.asarray(entry["losses"], np.float64)
    best_o = entry["best_index"]
    rel = np.abs(loss_g - loss_o) / loss_o
    assert np.all(rel <= 1e-4), (int(np.argmax(rel)), float(rel.max()))
    assert best_g == int(np.argmin(loss_g))
    assert np.all(loss_g[:best_g] > loss_g[best_g])
    assert best_g == best_o or loss_o[best_g] <= (1 + 1e-4) * loss_o[best_o], (best_g, best_o)
    say(f"  losses within {rel.max():.2e}; best {best_g} (oracle {best_o})")
    return best_o


@pytest.mark.parametrize("name", list(datagen.WORKLOADS))
def test_search_and_pack_workload_full(name):
    w = datagen.WORKLOADS[name]
    say("search + pack, full size:", name)
    W = datagen.weight(w)
    Xc = datagen.calibration(w)
    grid = datagen.alpha_grid(w.n_alpha)
    Wd = dev(W)
    s_g, best_g, loss_g = awq.scale_search(Wd, dev(Xc), grid, w.bits, w.group)
    best_o = check_curve(loss_g, best_g, golden()[("single", name, True)], grid)
    s_o = O.scale_from_stats(O.act_stats(Xc), grid[best_o])
    if best_g == best_o:
        assert_same_bits(host(s_g), s_o)
    q, sc, z = awq.quantize_pack(Wd, dev(s_o), w.bits, w.group)
    qh, sch, zh = host(q), host(sc), host(z)
    del q, sc, z, Wd
    qo, so, zo = O.quantize_pack(W, s_o, w.bits, w.group)
    assert_same_bits(qh, qo)
    assert_same_bits(sch, so)
    assert_same_bits(zh, zo)


def test_joint_search_gate_up_full():
    """Gate and up of the 4096 x 11008 MLP, every row of both, all 20 points."""
    w = datagen.WORKLOADS["llama7b_mlp_up_4096x11008_int4"]
    say("joint search gate/up, full size")
    Xc = datagen.calibration(w)
    grid = datagen.alpha_grid(w.n_alpha)
    s_g, best_g, loss_g = awq.scale_search_joint(
        [dev(datagen.gate_weight(w)), dev(datagen.weight(w))], dev(Xc), grid, w.bits, w.group)
    best_o = check_curve(loss_g, best_g, golden()[("joint_gate_up", w.name, True)], grid)
    if best_g == best_o:
        assert_same_bits(host(s_g), O.scale_from_stats(O.act_stats(Xc), grid[best_o]))
