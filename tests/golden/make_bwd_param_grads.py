"""Writes tests/golden/bwd_param_grads.npz: the oracle's dw and dgain for the
two full-size Block backward workloads (T=8192, d=4096, N=8, S=4; H=1 with
reps ~ N(0,(1+0.3n)^2), and the MHAR H=8 workload with N(0,(1+0.1n)^2)),
summed over every token.

dw and dgain are sums over tokens, and tokens are independent, so the oracle
(oracle/attnres_oracle.py, block_bwd, float64) runs over token chunks of 512
and the chunk results are added in chunk order.  Inputs come from the seeded
generators in workloads/synth.py, exactly as the GPU test draws them.  This
script calls only the oracle and the input generators.

    python tests/golden/make_bwd_param_grads.py      (about a minute on 8 cores)
"""

import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import attnres_oracle as orc  # noqa: E402
from workloads import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bwd_param_grads.npz")
CHUNK = 512


def _workload(H):
    return synth.config_block_fwd_bwd() if H == 1 else synth.config_mhar_fwd_bwd(H=H)


def _chunk(args):
    H, lo = args
    wl = _workload(H)
    sl = slice(lo, min(wl.T, lo + CHUNK))
    _, _, dw, dg = orc.block_bwd(wl.reps[:, sl], wl.partials[:, sl], wl.w, wl.gain, wl.eps, H, wl.dh[:, sl])
    return dw, dg


def main():
    out = {}
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ProcessPoolExecutor(workers) as ex:
        for H in (1, 8):
            T = _workload(H).T
            parts = list(ex.map(_chunk, [(H, lo) for lo in range(0, T, CHUNK)]))
            dw = np.zeros_like(parts[0][0])
            dg = np.zeros_like(parts[0][1])
            for a, b in parts:  # chunk order
                dw += a
                dg += b
            out[f"dw_H{H}"], out[f"dgain_H{H}"] = dw, dg
            print(f"H={H}: {len(parts)} chunks, |dw| rms {np.sqrt(np.mean(dw ** 2)):.3e}", flush=True)
    np.savez(OUT, **out)
    print(OUT)


if __name__ == "__main__":
    main()
