"""GPU: a seeded sweep of small random shapes through every main entry point, the same checks as
the fixed small cases (mask, lists, kept mass, sparse, epilogue, dense, capture, row statistics,
and the FP8 path). Shapes cover degenerate sizes (N = 1, N below one block, N at and around
block boundaries), batch and head counts, D in {64, 128}, block in {64, 128} and both tensor
layouts. Per-head p and residual scales are drawn as well."""
import numpy as np
import pytest

import synth
from gpu_common import bsa  # noqa: F401  (fixture)
from test_gpu_fp8 import run_fp8
from test_gpu_parity import run_small

pytestmark = pytest.mark.gpu


def _draw(seed):
    g = np.random.default_rng(7000 + seed)
    fixed_n = [1, 2, 63, 64, 65, 127, 129]
    n = fixed_n[seed] if seed < len(fixed_n) else int(g.integers(1, 1500))
    return dict(batch=int(g.integers(1, 4)), heads=int(g.integers(1, 6)),
                head_dim=int(g.choice([64, 128])), block=int(g.choice([64, 128])), seq=n,
                layout=str(g.choice(["bhnd", "bnhd"])), top_p_lo=float(g.uniform(0.3, 0.9)),
                seed=seed)


CASES = [_draw(i) for i in range(12)]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c['seed']}_N{c['seq']}_D{c['head_dim']}_b{c['block']}"
                                            for c in CASES])
def test_random_shape(bsa, case):
    g = np.random.default_rng(8000 + case["seed"])
    H = case["heads"]
    cfg = synth.workload("tiny", grid=(1, 1, case["seq"]), batch=case["batch"], heads=H,
                         head_dim=case["head_dim"], block=case["block"])
    p = g.uniform(case["top_p_lo"], 1.0, size=H)
    c = g.uniform(0.0, 1.0, size=H)
    run_small(bsa, cfg, layout=case["layout"], top_p=p, res_scale=c)
    run_fp8(bsa, cfg, case["layout"], p, residual=True)
