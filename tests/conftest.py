import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU oracle run")


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# The parity gate: max |gpu - oracle| <= 1e-2 (fp32 accumulation), plus,
# for bf16 output only, half a unit in the last place of the output format
# at |oracle| (the rounding of the output itself: 2^(e-8) for |x| in
# [2^e, 2^(e+1))), elementwise. fp32 outputs get exactly 1e-2.
ABS_TOL = 1e-2
REL_RMS_TOL = 1e-2


def half_ulp_bf16(ref):
    import numpy as np

    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def gate_excess(got, ref, out_bf16):
    """How far the worst element lies beyond the gate (<= 0: within it)."""
    import numpy as np

    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    bound = ABS_TOL + (half_ulp_bf16(ref) if out_bf16 else 0.0)
    return float((err - bound).max()) if err.size else 0.0
