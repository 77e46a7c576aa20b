"""Flash deformable attention on seeded random problems against the oracle,
through the C ABI: level count and map sizes (1 to 120 pixels a side),
batch, query count (or encoder queries, one per value pixel), heads, head
width, points per level, location spread, storage dtype, and the grad_value path
(sorted with a workspace, or device atomics without one) all drawn from one
seeded generator.  Tolerances as in test_gpu_fdattn.
"""
import numpy as np
import pytest

from dynamic_sparse_vision_amd.workloads import FdaWorkload
from tests.test_gpu_fdattn import run_case, say

pytestmark = pytest.mark.gpu


def _draw_cases(n_cases, seed=4051, side=(1, 25), prefix="frnd"):
    rng = np.random.RandomState(seed)
    cases = []
    for i in range(n_cases):
        L = int(rng.randint(1, 6))
        shapes = tuple((int(rng.randint(*side)), int(rng.randint(*side))) for _ in range(L))
        K = int(rng.randint(1, min(8, 128 // L) + 1))
        dtype = ["fp32", "fp16", "bf16"][rng.randint(3)]
        D = int(rng.choice([8, 16, 32, 64]))
        Q = 0 if rng.rand() < 0.25 else int(rng.randint(1, 200))
        w = FdaWorkload(f"{prefix}{i:02d}_{dtype}_L{L}K{K}_D{D}", N=int(rng.randint(1, 4)), shapes=shapes,
                        M=int(rng.randint(1, 7)), D=D, K=K, dtype=dtype, seed=3000 + i,
                        sigma_px=float(rng.choice([0.5, 2.0, 6.0, 15.0])), Q=Q)
        cases.append((w, bool(rng.rand() < 0.75)))
    return cases


CASES = _draw_cases(80)
# levels of 20 to 120 pixels a side: many sort blocks per slice, slices of up
# to about 36 000 corner bins
CASES += _draw_cases(16, seed=4052, side=(20, 121), prefix="fbig")


@pytest.mark.parametrize("w,sorted_gv", CASES, ids=lambda x: getattr(x, "name", None) or f"sorted={x}")
def test_fdattn_random(w, sorted_gv):
    say(f"[fdattn random] {w.name} N={w.N} levels={w.shapes} Q={w.queries} M={w.M} sigma={w.sigma_px} "
        f"sorted={sorted_gv}")
    run_case(w, sorted_grad_value=sorted_gv)
