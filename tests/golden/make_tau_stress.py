"""Write gptoss20b_tau_stress.json: the confidence threshold of the gpt-oss-20b-shaped
stress workload, taken from the oracle.

The gpt-oss-20b-shaped workload draws its logits at temperature T ~ U[1.5, 3] per step
and sequence.  Its stated intent is that c sits near tau and budgets flip often.  With
tau = 0.5, the oracle's c never reaches tau on these logits (median about 0.29, max
about 0.5).  The stress variant therefore sets tau to the median of the oracle's c over
every step and sequence of the workload's own seeded logits (seed 0, the seed the bench
and the full-size tests use), drawn where they draw them: on the GPU, whose generator
gives other numbers than the CPU's for the same seed (hence --device cuda).  It takes the lower median, the middle row's own c, so
that one (step, sequence) sits exactly at tau and the threshold's tie rule (c >= tau
picks the tight budget) is met at full size.

Calls only the oracle and the seeded input generator:

    python tests/golden/make_tau_stress.py --device cuda
"""
from __future__ import annotations

import argparse
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from adaptive_kv_cache_amd import synth  # noqa: E402
from adaptive_kv_cache_amd.workloads import WORKLOADS  # noqa: E402

BASE = "gptoss20b_gqa_b32_16k"
SEED = 0
OUT = os.path.join(HERE, "gptoss20b_tau_stress.json")


def _row_cs(z) -> list:
    wl = WORKLOADS[BASE]
    return [O.confidence(z[b], wl.w_H, wl.w_m, wl.w_p)["c"] for b in range(z.shape[0])]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--device", default="cuda", help="where the logits are drawn (the bench's: cuda)")
    ap.add_argument("--workers", type=int, default=8)
    args = ap.parse_args()
    wl = WORKLOADS[BASE]
    zs = (synth.logits(wl, step, SEED, device=args.device).cpu().numpy().astype(np.float64)
          for step in range(wl.steps))
    with ProcessPoolExecutor(max_workers=args.workers) as ex:
        cs = np.array(list(ex.map(_row_cs, zs)), dtype=np.float64)  # [steps][B]
    flat = cs.ravel()
    order = np.argsort(flat, kind="stable")
    k = (flat.size - 1) // 2                       # lower median: a row's own value
    i = int(order[k])
    step, seq = divmod(i, wl.batch)
    tau = float(flat[i])
    tau32 = float(np.float32(tau))
    above = cs >= tau32
    flips = float(np.mean(above[1:] != above[:-1]))
    res = {
        "_source": ("oracle.confidence over the seeded logits of workload " + BASE +
                    f" (seed {SEED}, steps 0..{wl.steps - 1}, sequences 0..{wl.batch - 1}, "
                    f"drawn on {args.device}); written by tests/golden/make_tau_stress.py"),
        "device": args.device,
        "rows": int(flat.size),
        "tau": tau,
        "tau_f32": tau32,
        "median_step": int(step),
        "median_seq": int(seq),
        "c_min": float(flat.min()),
        "c_max": float(flat.max()),
        "fraction_at_or_above_tau_f32": float(above.mean()),
        "budget_flip_rate": flips,
    }
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
