"""Calibrate the power-law constant c of the 128K LLaMA-shaped workload.

The workload draws per-64-token-block key alignments lam_g = c * ln(P_g),
P_g ~ Pareto(1).  This script bisects c so that the oracle keeps 40% of the
blocks at p = 0.99 on the seed-2 draw of the single 131072-token request, and
prints the value to freeze in synth.POWERLAW_C.  It calls only the oracle and
the generator.  Run from the repository root:

    python tests/golden/calibrate_generator.py [lo hi iters]
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
import synth   # noqa: E402

TARGET = 0.40


def keep_ratio(c: float) -> float:
    wl = synth.llama_128k(c=c)
    cu, q, k = synth.make_qk(wl)
    r = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    return float(r["keep_block"].mean())


def main():
    lo, hi, iters = 2.0, 3.0, 10
    if len(sys.argv) == 4:
        lo, hi, iters = float(sys.argv[1]), float(sys.argv[2]), int(sys.argv[3])
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        kr = keep_ratio(mid)
        print(f"c={mid:.6f} keep={kr:.4f}", flush=True)
        if kr > TARGET:
            lo = mid          # too many blocks kept: concentrate more
        else:
            hi = mid
    c = 0.5 * (lo + hi)
    print(f"POWERLAW_C = {c:.4f}  keep={keep_ratio(c):.4f}")


if __name__ == "__main__":
    main()
