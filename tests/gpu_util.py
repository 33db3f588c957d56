"""Helpers shared by the GPU tests: running the oracle on the same inputs and the
error metric the tolerances are stated in."""
import sys

import numpy as np
import torch

from oracle import gdn_oracle as orc

# Tolerances (normwise max relative error against the fp64 oracle): 2e-2 on outputs and
# 1e-2 on the final state, for bf16 q/k/v/o with an fp32 state and for an all-fp32 call.
TOL_O = 2e-2
TOL_S = 1e-2


# Parity figures of the run, printed by tests/conftest.py in pytest's terminal summary (so
# they show for passing tests and under -q as well).
REPORT = []


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crashed run).  Lines that
    carry error figures also go to the end-of-run parity summary."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()
    if any("error" in str(x) for x in a):
        REPORT.append(" ".join(f"{x:.3e}" if isinstance(x, float) else str(x) for x in a))


def nrel(x, ref):
    """max_i |x_i - ref_i| / max_i |ref_i|, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def np32(t):
    """Exact fp32 numpy copy of a CPU/GPU tensor (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def oracle_prefill(d, state_in=None, pairs=None, nthreads=None, qk_norm=False):
    s = None if state_in is None else np.asarray(state_in, dtype=np.float64)
    return orc.seq(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]), np32(d["beta"]), s,
                   pairs=pairs, nthreads=nthreads, rows_per_item=8, qk_norm=qk_norm)


def to_dev(d, device="cuda:0"):
    return {k: (None if v is None else v.to(device)) for k, v in d.items()}
