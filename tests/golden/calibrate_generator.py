"""Calibrate the synthetic workloads' structure constants against the oracle.

Two modes; each bisects one constant so that the oracle's selection keeps a
target share, and prints the value to freeze in synth.  It calls only the
oracle and the generator.  Run from the repository root:

    python tests/golden/calibrate_generator.py powerlaw [lo hi iters]
    python tests/golden/calibrate_generator.py varlen

powerlaw: the power-law constant c of the 128K LLaMA-shaped workload (per-
64-token-block key alignments lam_g = c * ln(P_g), P_g ~ Pareto(1)), so that
40% of the blocks of the seed-2 draw of the 131072-token request are kept at
p = 0.99 (synth.POWERLAW_C).

varlen: the hot-block alignment of each request of the 4-request varlen batch
(lengths 4096 / 8192 / 16384 / 2048 with 2 / 8 / 20 / 25 hot blocks), so that
the first three requests keep about 10%, 35% and 60% of their tokens; the
2048-token request has 28 blocks that are neither sink nor window, 25 of them
hot at alignment 8, and keeps 29 of its 32 blocks (90.6%) by construction
(synth.HOT_LAMBDA_VARLEN).  Each
request draws from its own streams, so its keep ratio depends on its own
alignment only and the bisections are independent.
"""
import os
import sys
from dataclasses import replace

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
import synth   # noqa: E402

TARGET_POWERLAW = 0.40
TARGET_VARLEN = (0.10, 0.35, 0.60)   # requests 0-2; request 3 keeps everything


def keep_ratio(c: float) -> float:
    wl = synth.llama_128k(c=c)
    cu, q, k = synth.make_qk(wl)
    r = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    return float(r["keep_block"].mean())


def varlen_ratios(lams):
    """Token keep ratio of each request of the varlen batch at alignments lams."""
    wl = synth.llama_varlen4(hot_lambda=tuple(lams))
    cu, q, k = synth.make_qk(wl)
    r = oracle.select(q, k, cu, wl.hq, wl.hkv, wl.d, wl.G, wl.A, wl.n, wl.p)
    return [int(r["kept"][i]) / int(cu[i + 1] - cu[i]) for i in range(wl.num_reqs)]


def bisect(f, lo, hi, target, iters, decreasing=True):
    """Bisect x in [lo, hi] so that f(x) ~ target, f decreasing in x."""
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        v = f(mid)
        print(f"  x={mid:.6f} -> {v:.4f}", flush=True)
        if (v > target) == decreasing:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def main():
    mode = sys.argv[1] if len(sys.argv) > 1 else "powerlaw"
    if mode == "powerlaw":
        lo, hi, iters = 2.0, 3.0, 10
        if len(sys.argv) == 5:
            lo, hi, iters = float(sys.argv[2]), float(sys.argv[3]), int(sys.argv[4])
        c = bisect(keep_ratio, lo, hi, TARGET_POWERLAW, iters)
        print(f"POWERLAW_C = {c:.4f}  keep={keep_ratio(c):.4f}")
    elif mode == "varlen":
        lams = [8.0, 8.0, 8.0, 8.0]
        for i in (1, 2):
            def f(x, i=i):
                ll = list(lams)
                ll[i] = x
                return varlen_ratios(ll)[i]
            print(f"request {i}: target {TARGET_VARLEN[i]}", flush=True)
            lams[i] = round(bisect(f, 5.5, 8.0, TARGET_VARLEN[i], 12), 4)
        print(f"HOT_LAMBDA_VARLEN = {tuple(lams)}  keep ratios {[round(x, 4) for x in varlen_ratios(lams)]}")
    else:
        raise SystemExit(f"unknown mode {mode!r}")


if __name__ == "__main__":
    main()
