"""The host glue bench.py uses for its 1-u figures and sweeps, against the
oracle: the schedule-only run (library scheduler) and the Table 2 same-peak
count.  CPU only (the scheduler is host code)."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("policy", sorted(oracle.POLICIES))
@pytest.mark.parametrize("m,start", [(1, None), (2, None), (3, (0, 2, 5, 1, 0))])
def test_schedule_only_matches_oracle(policy, m, start):
    rng = np.random.default_rng(len(policy) * 10 + m)
    n, L, D = 5, 7, 4
    wt = rng.integers(0, 50, size=(n, L, D))
    wt[1, 3] = 0                                  # an empty micro-batch at one layer
    om, steps, _ = bench.schedule_only_u(wt, D, oracle.POLICIES[policy], m, start)
    trace, _, u = oracle.run_schedule_only([[list(r) for r in wj] for wj in wt], n, L, D, m,
                                           oracle.POLICIES[policy], start_layers=start)
    assert steps == len(trace)
    assert abs(om - (1 - float(u))) < 1e-12


@pytest.mark.parametrize("policy", sorted(oracle.POLICIES))
@pytest.mark.parametrize("m,start", [(1, None), (3, None), (2, (0, 2, 5, 1, 0))])
def test_plan_run_is_the_oracle_schedule(policy, m, start):
    """The whole-run plan the expert-parallel projection launches: every step's
    members and their layers equal the oracle's Algorithm 1 trace."""
    rng = np.random.default_rng(len(policy) * 7 + m)
    n, L, D = 5, 6, 4
    wt = rng.integers(0, 40, size=(n, L, D))
    steps = bench.plan_run(wt, D, oracle.POLICIES[policy], m, start)
    trace, _, _ = oracle.run_schedule_only([[list(r) for r in wj] for wj in wt], n, L, D, m,
                                           oracle.POLICIES[policy], start_layers=start)
    assert steps == [list(zip(R, ls)) for R, ls in trace]


def test_same_peak_matches_oracle():
    rng = np.random.default_rng(3)
    for D in (2, 4, 8):
        wt = rng.integers(0, 6, size=(6, 48, D))     # small values: many ties
        for run in (1, 2, 3):
            ref = [oracle.same_peak_windows(list(wj), run) for wj in wt]
            assert bench.same_peak(wt, run) == (sum(h for h, _ in ref), sum(w for _, w in ref))


def test_fit_linear_recovers_a_line():
    # exact points on y = 3 + 0.5 x: the fit returns them with R^2 = 1; one
    # more regressor that is pure noise gets a coefficient near zero
    rng = np.random.default_rng(7)
    x = rng.integers(0, 2000, size=200).astype(float)
    X = np.stack([np.ones_like(x), x], 1)
    c, r2, rel = bench.fit_linear(X, 3.0 + 0.5 * x)
    assert np.allclose(c, [3.0, 0.5]) and abs(r2 - 1.0) < 1e-12 and rel < 1e-12
    z = rng.normal(size=200)
    y = 3.0 + 0.5 * x + 0.01 * rng.normal(size=200)
    c2, r2b, _ = bench.fit_linear(np.stack([np.ones_like(x), x, z], 1), y)
    assert abs(c2[1] - 0.5) < 1e-4 and abs(c2[2]) < 0.01 and r2b > 0.999
    # constant response: R^2 is defined as 1 (nothing to explain)
    assert bench.fit_linear(X, np.full(200, 4.0))[1] == 1.0
