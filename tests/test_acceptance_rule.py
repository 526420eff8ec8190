"""The acceptance rule the GPU parity tests and the sweep bench apply
(oracle.compare_keep / band_exceptions), checked on the CPU against oracle
results whose boundary is known: a kept set equal to the oracle's passes, a
swap across a boundary with a clear score gap is flagged outside the band, a
swap among exactly tied candidates is inside it, and structural faults (size,
order, window) are reported."""
import numpy as np

import oracle


def _slice(n=40, budget=24, alpha=4, seed=3):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, 128)).astype(np.float32)
    q = rng.standard_normal((2, alpha, 128)).astype(np.float32)
    return oracle.slice_eval(k, q, budget=budget, obs_window=alpha, beta=2, lam=0.1, tau=0.5, amb_eps=oracle.TAU_BAND)


def test_oracle_keep_passes():
    ref = _slice()
    problems, nd, out = oracle.compare_keep(ref.keep, ref, 40, 24, 4, 0.1, oracle.REL_TOL)
    assert problems == [] and nd == 0 and out == []


def test_clear_swap_is_outside_the_band():
    n, budget, alpha = 40, 24, 4
    ref = _slice(n, budget, alpha)
    nc = n - alpha
    kept = [i for i in ref.keep if i < nc]
    dropped = sorted(set(range(nc)) - set(kept))
    # the best kept candidate for the worst dropped one: a gap far above the tolerance
    best = max(kept, key=lambda i: ref.Z[i])
    worst = min(dropped, key=lambda i: ref.Z[i])
    assert ref.Z[best] - ref.Z[worst] > 1e-2
    bad = np.array(sorted((set(ref.keep) - {best}) | {worst}))
    problems, nd, out = oracle.compare_keep(bad, ref, n, budget, alpha, 0.1, oracle.REL_TOL)
    assert problems == [] and nd == 2 and set(out) == {best, worst}


def test_tied_swap_is_inside_the_band():
    """Identical keys and zero queries tie every candidate's score: any
    choice of candidates is correct, and the rule accepts it."""
    n, budget, alpha = 12, 8, 2
    k = np.tile(np.random.default_rng(1).standard_normal((1, 128)).astype(np.float32), (n, 1))
    q = np.zeros((1, alpha, 128), np.float32)
    ref = oracle.slice_eval(k, q, budget=budget, obs_window=alpha, beta=2, lam=0.1, tau=0.5)
    other = np.array(list(range(budget - alpha)) + list(range(n - alpha, n)))  # the oldest instead of the newest
    assert not np.array_equal(np.sort(other), ref.keep)
    problems, nd, out = oracle.compare_keep(other, ref, n, budget, alpha, 0.1, oracle.REL_TOL)
    assert problems == [] and nd > 0 and out == []


def test_structural_faults_are_reported():
    n, budget, alpha = 40, 24, 4
    ref = _slice(n, budget, alpha)
    assert oracle.compare_keep(ref.keep[:-1], ref, n, budget, alpha, 0.1, oracle.REL_TOL)[0]  # size
    assert oracle.compare_keep(ref.keep[::-1], ref, n, budget, alpha, 0.1, oracle.REL_TOL)[0]  # order
    no_window = np.array(sorted(set(ref.keep) - {n - 1} | {int(min(set(range(n)) - set(ref.keep)))}))
    assert "observation window not kept" in oracle.compare_keep(no_window, ref, n, budget, alpha, 0.1,
                                                                 oracle.REL_TOL)[0]
    # a short sequence keeps everything
    assert oracle.compare_keep(np.arange(10), ref, 10, budget, alpha, 0.1, oracle.REL_TOL)[0] == []
    assert oracle.compare_keep(np.arange(1, 10), ref, 10, budget, alpha, 0.1, oracle.REL_TOL)[0]
