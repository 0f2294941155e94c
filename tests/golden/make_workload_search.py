"""Write tests/golden/workload_search.json: the oracle's full alpha-search
loss curves on every workload layer at full size.

    python tests/golden/make_workload_search.py [--jobs 4]

Calls only the CPU oracle (``oracle.awq_oracle``) and the seeded input
generator (``datagen``); nothing here touches the GPU library. For each
workload it records the oracle's 20-point loss curve L(alpha) =
||Xcal D_alpha^T||_F^2 and its first argmin (AWQ Explained: Protecting the
Weights That Matter Most -- "How the scale is chosen": the scale exponent is
picked on a small grid in [0, 1] to minimise the layer-output error on the
calibration batch), plus the joint curve of the gate and up projections of
the 4096 x 11008 MLP, which share one input and so one s (same page --
"Scaling instead of mixed precision": the division is folded into the norm
that feeds both). A full-size curve costs the oracle about 5 TFLOP of
float64 products and 20 quantizations of the matrix (minutes per layer), so
the values are stored instead of recomputed on every GPU test run.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "workload_search.json")


def _job(kind, name, zero_point):
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import numpy as np

    import datagen
    from oracle import awq_oracle as O

    w = datagen.WORKLOADS[name]
    grid = datagen.alpha_grid(w.n_alpha)
    Xc = datagen.calibration(w)
    if kind == "single":
        _, best, losses = O.scale_search(datagen.weight(w), Xc, grid, w.bits, w.group,
                                         zero_point)
    else:  # gate then up, summed in that order
        _, best, losses = O.joint_scale_search([datagen.gate_weight(w), datagen.weight(w)], Xc,
                                               grid, w.bits, w.group, zero_point)
    return {
        "kind": kind,
        "workload": name,
        "zero_point": zero_point,
        "bits": w.bits,
        "group": w.group,
        "alpha_grid": [float(a) for a in grid],
        "losses": [float(v) for v in np.asarray(losses, dtype=np.float64)],
        "best_index": int(best),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    # BLAS threads per worker, set before any worker imports numpy
    per = max(1, (os.cpu_count() or 4) // args.jobs)
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = str(per)
    sys.path.insert(0, ROOT)
    import datagen
    jobs = [("single", name, True) for name in datagen.WORKLOADS]
    jobs.append(("joint_gate_up", "llama7b_mlp_up_4096x11008_int4", True))
    import multiprocessing as mp
    with ProcessPoolExecutor(args.jobs, mp_context=mp.get_context("spawn")) as ex:
        futs = [ex.submit(_job, *j) for j in jobs]
        entries = []
        for j, f in zip(jobs, futs):
            e = f.result()
            print(f"{j[0]} {j[1]}: best {e['best_index']}", flush=True)
            entries.append(e)
    doc = {
        "source": "oracle.awq_oracle.scale_search / joint_scale_search on datagen inputs",
        "cite": "AWQ Explained: Protecting the Weights That Matter Most -- How the scale is chosen",
        "entries": entries,
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
