"""Calibrate the Zipf amplitude of the decode workload's selection bias.

The decode workload (T=64, V3 layer) skews its router bias b with a Zipf law
(exponent 1.1) over a random expert permutation so that about 40% of the 256
routed experts receive no token.  This script bisects the amplitude on the
seed-4 inputs with the fp64 oracle router and prints the value to freeze in
datagen (ZIPF_BETA_V3_DECODE).  The target is 102 idle experts (40% of 256).

    python tests/golden/calibrate_zipf_beta.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import datagen  # noqa: E402
import oracle  # noqa: E402


def idle_experts(beta: float) -> int:
    cfg = datagen.get_config("v3_decode", bias_param=beta)
    inp = datagen.MoEInputs(cfg)
    x64 = oracle.widen(inp.x(), cfg.act_dtype)
    r = oracle.route(cfg, x64, inp.router_w().astype(np.float64), inp.router_b())
    return int((r["counts"] == 0).sum())


def main(target: int = 102):
    lo, hi = 0.0, 4.0
    for _ in range(20):
        mid = (lo + hi) / 2
        n = idle_experts(mid)
        print(f"beta={mid:.10f} idle={n}")
        if n < target:
            lo = mid
        else:
            hi = mid
        if n == target:
            break
    beta = float(np.float32(mid))
    print("frozen beta:", repr(beta), "idle:", idle_experts(beta))


if __name__ == "__main__":
    main()
