"""Pins of the CPU oracle: checks against what the R-KV pages and mathematics fix.

Each check raises AssertionError on a mismatch. They run against whatever
library ``oracle.lib()`` returns, so the mutant tests can point them at a copy
of the oracle with a planted mistake and require that some check fails.

Kinds of pin (none of them re-types the oracle's own loops):
  * hand-derived cases with exact closed forms (tests/golden/hand_cases.json);
  * textbook special cases computed with library routines (torch float64
    softmax / mean / amax / topk; scipy softmax);
  * closed-form identities (row-mean identity through the sum of unit keys);
  * invariants (budget, window, ordering, exact duplicates, orthogonal keys,
    bitwise scale invariance, probability sums);
  * brute force over all k-subsets on tiny inputs.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def _ev(expr: str) -> float:
    """Evaluates a closed-form string of the golden file (fractions, e, exp)."""
    if all(ch in "0123456789/-" for ch in expr):
        return float(Fraction(expr))
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "exp": math.exp}))


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}\n got {a}\n exp {b}"


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _pad(arr, d):
    arr = np.asarray(arr, dtype=np.float32)
    out = np.zeros(arr.shape[:-1] + (d,), dtype=np.float32)
    out[..., : arr.shape[-1]] = arr
    return out


def check_hand_case(case, pad_to: int = 0):
    keys = np.asarray(case["keys"], dtype=np.float32)
    q = np.asarray(case["queries"], dtype=np.float32)
    if pad_to:
        # zero padding keeps every dot product and cosine; the attention
        # scale changes, so only zero-query cases are padded
        assert not np.any(q)
        keys, q = _pad(keys, pad_to), _pad(q, pad_to)
    r = oracle.slice_eval(keys, q, budget=case["budget"], obs_window=case["obs_window"], beta=case["beta"],
                          lam=case["lambda"], tau=case["tau"])
    name = case["name"]
    assert list(r.keep) == case["keep"], f"{name}: keep {list(r.keep)} != {case['keep']}"
    n_c = keys.shape[0] - case["obs_window"]
    if "counts" in case:
        assert list(r.counts) == case["counts"], f"{name}: counts {list(r.counts)} != {case['counts']}"
    if "rowmean" in case:
        _close(r.rowmean, [_ev(x) for x in case["rowmean"]], what=f"{name} rowmean")
    if "rbar" in case:
        _close(r.rbar, [_ev(x) for x in case["rbar"]], what=f"{name} rbar")
    if "importance" in case:
        exp_i = [_ev(x) for x in case["importance"]]
        _close(r.importance[: len(exp_i)], exp_i, what=f"{name} importance")
    if "R_candidates" in case:
        exp_r = [_ev(x) for x in case["R_candidates"]]
        _close(r.R[:n_c], exp_r, what=f"{name} R")
        exp_z = [case["lambda"] * r.importance[i] - (1 - case["lambda"]) * exp_r[i] for i in range(n_c)]
        _close(r.Z[:n_c], exp_z, what=f"{name} Z")


def check_hand_cases():
    for case in golden_cases():
        check_hand_case(case)
        if not np.any(np.asarray(case["queries"])):
            check_hand_case(case, pad_to=128)


def _bf16_f64(bits):
    """bf16 bit patterns (uint16) widened exactly to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rand_slice(seed, n, d, g, alpha, dtype="bf16", scale=1.0):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((n, d)) * scale).astype(np.float32)
    q = rng.standard_normal((g, alpha, d)).astype(np.float32)
    if dtype == "bf16":
        return synth.bf16_bits(k), synth.bf16_bits(q)
    return k, q


def check_lambda1_textbook():
    """lambda = 1: Z = I, so the kept candidates are the top-k of the GQA-max of
    the mean causal attention, built here from torch float64 primitives."""
    import torch

    for seed, (n, d, g, alpha, budget) in enumerate([(40, 16, 3, 4, 24), (70, 32, 5, 8, 40), (33, 8, 1, 1, 20)]):
        k_bits, q_bits = _rand_slice(100 + seed, n, d, g, alpha)
        r = oracle.slice_eval(k_bits, q_bits, budget=budget, obs_window=alpha, lam=1.0)
        K = torch.from_numpy(synth.to_float(k_bits, "bf16"))
        Qm = torch.from_numpy(synth.to_float(q_bits, "bf16"))  # [g, alpha, d]
        logits = torch.einsum("gtd,jd->gtj", Qm, K) / math.sqrt(d)
        pos = torch.arange(n - alpha, n).view(1, alpha, 1)
        mask = torch.arange(n).view(1, 1, n) > pos
        attn = torch.softmax(logits.masked_fill(mask, float("-inf")), dim=-1)
        imp = attn.mean(dim=1).amax(dim=0)
        _close(r.importance, imp.numpy(), tol=1e-12, what=f"lambda1 importance seed {seed}")
        cand = imp[: n - alpha]
        top = torch.topk(cand, budget - alpha).indices.tolist()
        exp_keep = sorted(top + list(range(n - alpha, n)))
        assert list(r.keep) == exp_keep, f"lambda1 keep seed {seed}"


def check_single_query_softmax():
    """G = 1, alpha = 1: importance is one textbook softmax row (scipy)."""
    from scipy.special import softmax

    k_bits, q_bits = _rand_slice(7, 50, 64, 1, 1, dtype="f32")
    r = oracle.slice_eval(k_bits, q_bits, budget=30, obs_window=1)
    logits = (k_bits.astype(np.float64) @ q_bits.reshape(-1).astype(np.float64)) / 8.0
    _close(r.importance, softmax(logits), tol=1e-12, what="single-query softmax")


def check_probability_sums():
    """Attention rows sum to 1, so with G = 1 the importance sums to 1; the
    redundancy softmax sums to 1 over the candidates."""
    k_bits, q_bits = _rand_slice(11, 90, 32, 1, 6)
    r = oracle.slice_eval(k_bits, q_bits, budget=50, obs_window=6)
    assert abs(r.importance.sum() - 1.0) < 1e-12, r.importance.sum()
    assert abs(r.R[:84].sum() - 1.0) < 1e-12
    assert np.all(r.R[84:] == 0.0)


def check_rowmean_identity():
    """sum_{j != i} S_ij = khat_i . (sum_j khat_j) - khat_i . khat_i."""
    for seed in range(3):
        k_bits, q_bits = _rand_slice(20 + seed, 64, 16, 2, 4)
        r = oracle.slice_eval(k_bits, q_bits, budget=40, obs_window=4)
        K = synth.to_float(k_bits, "bf16")
        Kh = K / np.linalg.norm(K, axis=1, keepdims=True)
        s = Kh.sum(axis=0)
        ident = (Kh @ s - np.einsum("id,id->i", Kh, Kh)) / (K.shape[0] - 1)
        _close(r.rowmean, ident, tol=1e-12, what="row-mean identity")


def _basis_keys(n, d, rng, scales=True):
    assert n <= d
    perm = rng.permutation(d)[:n]
    k = np.zeros((n, d), dtype=np.float32)
    for i, c in enumerate(perm):
        k[i, c] = (rng.uniform(0.5, 4.0) if scales else 1.0) * rng.choice([-1.0, 1.0])
    return k


def check_exact_duplicates():
    """A cluster of m identical keys among mutually orthogonal keys: S = 1
    inside the cluster, 0 elsewhere; exactly the min(m, beta) newest members
    are protected; an unprotected member has redundancy (m-1)/(N-1)."""
    rng = np.random.default_rng(5)
    for m, beta in [(2, 2), (3, 2), (5, 2), (4, 1), (4, 3)]:
        n, d, alpha = 40, 64, 4
        k = _basis_keys(n, d, rng)
        members = sorted(rng.choice(n - alpha, size=m, replace=False).tolist())
        proto = np.zeros(d, dtype=np.float32)
        used = set(np.nonzero(k)[1].tolist())
        free = [c for c in range(d) if c not in used]
        proto[free[0]] = 1.0
        proto[free[1]] = -2.0
        for i in members:
            k[i] = proto * rng.choice([0.5, 1.0, 2.0])  # positive rescale: identical direction
        q = rng.standard_normal((1, alpha, d)).astype(np.float32)
        r = oracle.slice_eval(k, q, budget=20, obs_window=alpha, beta=beta)
        for rank, i in enumerate(members):
            newer = m - 1 - rank
            assert r.counts[i] == newer, (m, beta, i, r.counts[i], newer)
            if newer < beta:
                assert r.rbar[i] == 0.0
            else:
                assert abs(r.rbar[i] - (m - 1) / (n - 1)) < 1e-12
        others = [i for i in range(n) if i not in members]
        assert np.all(r.counts[others] == 0) and np.all(r.rbar[others] == 0.0)


def check_orthogonal_keys():
    """Orthogonal keys: no similar pair, all protected, R = 1/|C| exactly,
    selection is the top-k of importance."""
    rng = np.random.default_rng(9)
    n, d, alpha, budget = 48, 64, 8, 24
    k = _basis_keys(n, d, rng)
    q = rng.standard_normal((2, alpha, d)).astype(np.float32)
    r = oracle.slice_eval(k, q, budget=budget, obs_window=alpha)
    nc = n - alpha
    assert np.all(r.counts == 0) and np.all(r.rbar == 0.0)
    _close(r.R[:nc], np.full(nc, 1.0 / nc), tol=1e-15, what="orthogonal R")
    top = np.argsort(-r.importance[:nc], kind="stable")[: budget - alpha]
    assert list(r.keep) == sorted(top.tolist() + list(range(nc, n)))


def check_scale_invariance():
    """Keys times 2 and queries times 1/2 give bitwise identical results."""
    k, q = _rand_slice(31, 80, 32, 3, 8, dtype="f32")
    a = oracle.slice_eval(k, q, budget=40)
    b = oracle.slice_eval(k * np.float32(2.0), q * np.float32(0.5), budget=40)
    for name in ("importance", "rowmean", "counts", "rbar", "R", "Z", "keep"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


def check_budget_invariants():
    """|keep| = min(N, B); the window is kept; keep is strictly ascending with keep[j] >= j."""
    rng = np.random.default_rng(3)
    for trial in range(60):
        n = int(rng.integers(2, 64))
        alpha = int(rng.integers(1, 9))
        budget = int(rng.integers(alpha + 1, alpha + 40))
        g = int(rng.integers(1, 4))
        k, q = _rand_slice(1000 + trial, n, 16, g, alpha)
        r = oracle.slice_eval(k, q, budget=budget, obs_window=alpha, beta=int(rng.integers(0, 4)))
        keep = r.keep
        assert r.kept == len(keep) == min(n, budget)
        assert np.all(np.diff(keep) > 0)
        assert np.all(keep >= np.arange(len(keep)))
        if n > budget:
            assert set(range(n - alpha, n)) <= set(keep.tolist())


def check_bruteforce_topk():
    """Tiny slices: the chosen candidates maximise sum(Z) over every k-subset,
    and no excluded candidate beats an included one (ties: newer wins)."""
    for trial in range(12):
        rng = np.random.default_rng(2000 + trial)
        n = int(rng.integers(7, 13))
        alpha = 2
        budget = int(rng.integers(3, n))
        k, q = _rand_slice(3000 + trial, n, 8, 2, alpha)
        if trial % 3 == 0:
            k[3] = k[1]  # an exact duplicate pair
        r = oracle.slice_eval(k, q, budget=budget, obs_window=alpha, beta=1)
        nc, kk = n - alpha, budget - alpha
        chosen = [i for i in r.keep if i < nc]
        best = max(sum(r.Z[list(s)]) for s in itertools.combinations(range(nc), kk))
        assert abs(sum(r.Z[chosen]) - best) < 1e-15
        for c in range(nc):
            if c in chosen:
                continue
            for s in chosen:
                assert r.Z[s] > r.Z[c] or (r.Z[s] == r.Z[c] and s > c)


def check_lambda0_least_redundant():
    """lambda = 0: Z = -R, so the k least redundant candidates are kept."""
    k, q = _rand_slice(44, 60, 16, 2, 4)
    kf = synth.to_float(k, "bf16").astype(np.float32)
    for i in range(10, 40, 3):  # near-duplicates of earlier keys make redundancy spread out
        kf[i] = kf[i - 7] + np.float32(0.01) * kf[i]
    r = oracle.slice_eval(kf, synth.to_float(q, "bf16").astype(np.float32), budget=30, obs_window=4, beta=1,
                          lam=0.0)
    nc = 56
    order = sorted(range(nc), key=lambda i: (r.rbar[i], -i))
    assert list(r.keep) == sorted(order[:26] + list(range(nc, 60)))


def check_step_noop_and_compaction():
    """The whole step: a no-op below the trigger; above it, every slice's kept
    rows land in order in [B - kept, B), bitwise equal to the source rows."""
    w = synth.small(num_layers=2, batch=3, num_kv_heads=2, group=2, budget=96, buffer=32,
                    lengths=("uniform", 60, 128), span_len=16, extra_capacity=8)
    c = synth.build_cache(w, seed=1)
    # below the trigger: nothing changes
    K0, V0, s0 = c.K.copy(), c.V.copy(), c.seq_start.copy()
    ev, ns, _ = oracle.evict_step(K0, V0, c.Q, s0, w.n_slots - 1, w.budget, w.buffer)
    assert not ev and ns == w.n_slots - 1
    assert np.array_equal(K0.view(np.uint8), c.K.view(np.uint8)) and np.array_equal(s0, c.seq_start)
    K1, V1, s1 = c.K.copy(), c.V.copy(), c.seq_start.copy()
    ev, ns, keep = oracle.evict_step(K1, V1, c.Q, s1, w.n_slots, w.budget, w.buffer)
    assert ev and ns == w.budget
    B = w.budget
    for l in range(w.num_layers):
        for b in range(w.batch):
            n = int(c.lengths[b])
            kept = min(n, B)
            assert s1[b] == B - kept
            for h in range(w.num_kv_heads):
                kr = keep[l, b, h]
                assert np.all(kr[: B - kept] == -1)
                src = kr[B - kept:]
                ref = oracle.slice_eval(c.K[l, b, h, c.seq_start[b]:w.n_slots],
                                        c.Q[l, b, h * w.group:(h + 1) * w.group], budget=B)
                assert np.array_equal(src, ref.keep + c.seq_start[b])
                assert np.array_equal(K1[l, b, h, B - kept:B], c.K[l, b, h][src])  # numpy fancy-index gather
                assert np.array_equal(V1[l, b, h, B - kept:B], c.V[l, b, h][src])
                # canary rows past n_slots are untouched
                assert np.array_equal(K1[l, b, h, w.n_slots:].view(np.uint16), c.K[l, b, h, w.n_slots:].view(np.uint16))


HOLEFILL = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "holefill_cases.json")


def holefill_cases():
    with open(HOLEFILL) as f:
        return json.load(f)["cases"]


def check_holefill_hand_cases():
    """Hole-filling compaction: the hand-derived cases (physical row p holds
    the value p; every row is 2 values wide, K and V alike)."""
    for c in holefill_cases():
        n, B = c["n_slots"], c["budget"]
        K = np.repeat(np.arange(n, dtype=np.float32)[:, None], 2, axis=1)
        V = K + 1000.0
        K2, V2, o2, lead = oracle.holefill_slice(K, V, np.array(c["order"]), np.array(c["keep"]), B)
        assert lead == c["start_after"], (c["name"], lead)
        assert o2.tolist() == c["order_after"], (c["name"], o2.tolist())
        assert K2[:, 0].tolist() == c["rows_after"], (c["name"], K2[:, 0].tolist())
        assert (V2[:, 0] - 1000.0).tolist() == c["rows_after"], c["name"]


def _rand_holefill(rng, B, n_slots, n_valid, n_keep):
    """A random permutation order and a valid ascending keep list of n_keep
    virtual slots among the n_valid newest (right-aligned, -1 before)."""
    order = rng.permutation(B).astype(np.int32)
    s0 = n_slots - n_valid
    kept = np.sort(rng.choice(np.arange(s0, n_slots), size=n_keep, replace=False)).astype(np.int32)
    keep = np.full(B, -1, np.int32)
    keep[B - n_keep:] = kept
    return order, keep


def check_holefill_invariants():
    """Random cases: the new order is a permutation; every kept token's row is
    found at its new physical row; kept tokens below the budget did not move;
    only rows that received a mover changed, at most n_slots - budget of them."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        B = int(rng.integers(2, 40))
        buf = int(rng.integers(1, 20))
        n = B + buf
        n_valid = int(rng.integers(1, n + 1))
        n_keep = min(n_valid, B)
        order, keep = _rand_holefill(rng, B, n, n_valid, n_keep)
        K = rng.standard_normal((n, 3)).astype(np.float32)
        V = rng.standard_normal((n, 3)).astype(np.float32)
        virt = lambda X, v: X[order[v]] if v < B else X[v]
        K2, V2, o2, lead = oracle.holefill_slice(K, V, order, keep, B)
        assert lead == B - n_keep
        assert sorted(o2.tolist()) == list(range(B))
        for j in range(lead, B):
            assert np.array_equal(K2[o2[j]], virt(K, keep[j])) and np.array_equal(V2[o2[j]], virt(V, keep[j]))
            if keep[j] < B:
                assert o2[j] == order[keep[j]]
        changed = [r for r in range(n) if not np.array_equal(K2[r], K[r])]
        movers = int((keep >= B).sum())
        assert len(changed) <= movers <= buf
        assert all(r < B for r in changed)
        assert np.array_equal(K2[B:], K[B:])


def check_holefill_rejects_bad_order():
    """An order row that is not a permutation is refused."""
    K = np.zeros((6, 2), np.float32)
    for bad in ([0, 0, 1, 2], [0, 1, 2, 4], [-1, 1, 2, 3]):
        try:
            oracle.holefill_slice(K, K, np.array(bad), np.array([0, 1, 2, 3]), 4)
        except ValueError:
            continue
        raise AssertionError(f"accepted {bad}")


def _uniforms(rng, n):
    """Uniforms strictly inside (0, 1), exact in float32."""
    return ((rng.integers(0, 1 << 24, size=n) + 0.5) / float(1 << 24)).astype(np.float32)


def check_sampled_top_k_is_deterministic():
    """With top_k = budget - keep_newest the draw has nothing to choose: the
    kept set is the plain top of the scores (equal scores: the later
    position) plus the newest tokens, whatever the uniforms."""
    rng = np.random.default_rng(21)
    for _ in range(100):
        n = int(rng.integers(5, 40))
        B = int(rng.integers(2, n))
        L = int(rng.integers(0, B))
        sc = rng.integers(-3, 4, size=n).astype(np.float32)  # many equal scores
        got = oracle.select_sampled(sc, _uniforms(rng, n), B, L, B - L)
        cand = sorted(range(n - L), key=lambda i: (-float(sc[i]), -i))[:B - L]
        assert got.tolist() == sorted(cand + list(range(n - L, n))), (n, B, L)


def check_sampled_equal_scores():
    """Equal scores and no Top-K restriction: exp(score / T) is the same for
    every candidate and -log(-log u) is increasing in u, so the draw keeps
    the candidates with the largest uniforms."""
    rng = np.random.default_rng(22)
    for _ in range(50):
        n = int(rng.integers(5, 60))
        B = int(rng.integers(2, n))
        L = int(rng.integers(0, B))
        u = _uniforms(rng, n)
        got = oracle.select_sampled(np.full(n, 0.3, np.float32), u, B, L, n, temperature=0.5)
        cand = sorted(range(n - L), key=lambda i: -float(u[i]))[:B - L]
        assert got.tolist() == sorted(cand + list(range(n - L, n)))


def _inclusion_exact(w, m):
    """Probability that each item is among m drawn without replacement, each
    draw proportional to w among those left (enumerating ordered draws)."""
    import itertools
    K = len(w)
    inc = np.zeros(K)
    for seq in itertools.permutations(range(K), m):
        pr, left = 1.0, float(sum(w))
        for i in seq:
            pr *= w[i] / left
            left -= w[i]
        for i in seq:
            inc[i] += pr
    return inc


def check_sampled_inclusion_probabilities():
    """The draw's law: over many seeded uniform vectors, how often each
    candidate is kept matches the exact inclusion probability of drawing
    budget - keep_newest items one at a time with probability proportional to
    exp(score / T) among the top_k left (within 4.5 standard errors); items
    outside the top_k are never kept."""
    rng = np.random.default_rng(23)
    sc = np.array([0.0, 0.5, 1.0, 1.5, -1.0, 0.25, 2.0], np.float32)
    n, L, T, D = len(sc), 1, 0.7, 40000
    for top_k, B in ((6, 3), (4, 3), (6, 4)):
        nc, m = n - L, B - L
        order = sorted(range(nc), key=lambda i: (-float(sc[i]), -i))[:top_k]
        p = np.zeros(nc)
        p[order] = _inclusion_exact([np.exp(float(sc[i]) / T) for i in order], m)
        cnt = np.zeros(nc)
        for _ in range(D):
            kept = oracle.select_sampled(sc, _uniforms(rng, n), B, L, top_k, temperature=T)
            assert kept[-1] == n - 1 and len(kept) == B
            cnt[kept[:-1]] += 1
        f = cnt / D
        tol = 4.5 * np.sqrt(p * (1 - p) / D) + 1e-9
        assert np.all(np.abs(f - p) <= tol), (top_k, B, f.round(4).tolist(), p.round(4).tolist())


def check_sampled_scale_invariance():
    """Scores and temperature scaled by the same power of two keep the same
    set (score / T is unchanged exactly)."""
    rng = np.random.default_rng(24)
    for _ in range(30):
        n = int(rng.integers(8, 50))
        B = int(rng.integers(3, n))
        L = int(rng.integers(0, B))
        sc = rng.standard_normal(n).astype(np.float32)
        u = _uniforms(rng, n)
        k = int(rng.integers(B - L, n))
        a = oracle.select_sampled(sc, u, B, L, k, temperature=0.8)
        b = oracle.select_sampled(sc * np.float32(4), u, B, L, k, temperature=3.2)
        assert np.array_equal(a, b)


def check_sentence_penalty_closed_forms():
    """Sentence redundancy: exact cosines of small vectors. (1,0) against the
    later (0.75,1) and (3,4) has cosine 0.6 > 0.5; (0.75,1) against (3,4)
    has 1; (3,4) against (0,-1) has -0.8; the last sentence has no later one.
    Scaled copies have cosine 1, orthogonal vectors 0, a zero vector 0."""
    v = np.array([[1, 0], [0.75, 1], [3, 4], [0, -1]], np.float32)
    pen = oracle.sentence_penalty(v, 0.5)
    assert abs(pen[0] - 0.6) < 1e-15 and abs(pen[1] - 1.0) < 1e-15
    assert pen[2] == 0.0 and pen[3] == 0.0
    assert np.all(oracle.sentence_penalty(v, 0.99) == np.array([0.0, 1.0, 0.0, 0.0]))
    rng = np.random.default_rng(31)
    base = rng.standard_normal((1, 64)).astype(np.float32)
    copies = np.concatenate([base * np.float32(c) for c in (1, 2, 0.5, 4)])
    assert np.allclose(oracle.sentence_penalty(copies, 0.5), [1, 1, 1, 0], atol=1e-12)
    eye = np.eye(5, 8, dtype=np.float32)
    assert np.all(oracle.sentence_penalty(eye, 0.0) == 0.0)  # cosine 0 is not above 0
    z = np.vstack([np.zeros((1, 8), np.float32), eye[:1] * np.float32(3), eye[:1]])
    assert oracle.sentence_penalty(z, 0.5).tolist() == [0.0, 1.0, 0.0]  # a zero vector is never similar


def check_penalized_selection():
    """The sentence penalty enters Z as a subtraction on the candidates: a zero
    penalty reproduces the plain selection, a constant one leaves the kept
    set unchanged, and a penalty larger than any score gap evicts the
    penalised candidates first while budget allows."""
    rng = np.random.default_rng(32)
    for _ in range(20):
        n, d, g, a = int(rng.integers(24, 48)), 16, 2, 4
        B = int(rng.integers(a + 4, n - 2))
        k, q = _rand_slice(int(rng.integers(1 << 30)), n, d, g, a)
        plain = oracle.slice_eval(k, q, budget=B, obs_window=a)
        zero = oracle.slice_eval(k, q, budget=B, obs_window=a, token_penalty=np.zeros(n))
        assert np.array_equal(plain.keep, zero.keep) and np.array_equal(plain.Z, zero.Z)
        const = oracle.slice_eval(k, q, budget=B, obs_window=a, token_penalty=np.full(n, 0.25))
        assert np.array_equal(plain.keep, const.keep)
        nc = n - a
        hit = rng.choice(nc, size=int(rng.integers(1, n - B + 1)), replace=False)
        pen = np.zeros(n)
        pen[hit] = 10.0
        r = oracle.slice_eval(k, q, budget=B, obs_window=a, token_penalty=pen)
        assert not (set(hit.tolist()) & set(r.keep.tolist())), "a penalised candidate was kept"
        assert np.allclose(r.Z[:nc], plain.Z[:nc] - pen[:nc], atol=0)


def check_decode_attention_textbook():
    """Decode attention against torch float64's scaled_dot_product_attention
    (default scale 1/sqrt(D)) and torch.softmax for the weights, on bf16 and
    fp32 slices with n from 1 to 70 keys and G from 1 to 5 query heads."""
    import torch

    rng = np.random.default_rng(40)
    for it, (n, d, g) in enumerate([(1, 16, 1), (2, 8, 3), (37, 16, 4), (70, 32, 5), (64, 128, 4)]):
        k = rng.standard_normal((n, d)).astype(np.float32)
        v = rng.standard_normal((n, d)).astype(np.float32)
        q = rng.standard_normal((g, d)).astype(np.float32)
        for bf in (False, True):
            if bf:
                kb, vb, qb = synth.bf16_bits(k), synth.bf16_bits(v), synth.bf16_bits(q)
                kd, vd, qd = (_bf16_f64(x) for x in (kb, vb, qb))
            else:
                kb, vb, qb = k, v, q
                kd, vd, qd = (x.astype(np.float64) for x in (k, v, q))
            out, w = oracle.decode_attention(kb, vb, qb)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qd)[None], torch.from_numpy(kd)[None], torch.from_numpy(vd)[None])[0]
            wref = torch.softmax(torch.from_numpy(qd) @ torch.from_numpy(kd).T / math.sqrt(d), dim=-1)
            _close(out, ref.numpy(), 1e-12, f"decode attention output, case {it} bf16={bf}")
            _close(w, wref.numpy(), 1e-12, f"decode attention weights, case {it} bf16={bf}")


def check_decode_attention_special_cases():
    """One key: its value comes back exactly with weight 1. Identical keys (or
    a zero query): uniform weights 1/n and the mean of the values. Unit keys
    against a query of 32 on one axis (D = 16): logit 8 for that key, 0 for
    the rest, weights e^8 / (e^8 + n - 1) and 1 / (e^8 + n - 1). No keys:
    the output is 0."""
    rng = np.random.default_rng(41)
    d = 16
    v1 = rng.standard_normal((1, d)).astype(np.float32)
    k1 = rng.standard_normal((1, d)).astype(np.float32)
    q = rng.standard_normal((3, d)).astype(np.float32)
    out, w = oracle.decode_attention(k1, v1, q)
    assert np.all(w == 1.0) and np.all(out == v1.astype(np.float64))
    n = 9
    krow = rng.standard_normal((1, d)).astype(np.float32)
    vals = rng.standard_normal((n, d)).astype(np.float32)
    out, w = oracle.decode_attention(np.repeat(krow, n, 0), vals, q)
    _close(w, np.full((3, n), 1.0 / n), 1e-15, "identical keys: uniform weights")
    _close(out, np.repeat(vals.astype(np.float64).mean(0, keepdims=True), 3, 0), 1e-14, "identical keys: mean")
    out, w = oracle.decode_attention(rng.standard_normal((n, d)).astype(np.float32), vals,
                                     np.zeros((2, d), np.float32))
    _close(w, np.full((2, n), 1.0 / n), 1e-15, "zero query: uniform weights")
    e = np.eye(n, d, dtype=np.float32)
    qq = np.zeros((1, d), np.float32)
    qq[0, 4] = 32.0  # logit 32 / 4 = 8 for key 4, 0 for the others
    out, w = oracle.decode_attention(e, vals, qq)
    want = math.exp(8) / (math.exp(8) + n - 1)
    assert abs(w[0, 4] - want) < 1e-15 and abs(w[0, 0] - 1 / (math.exp(8) + n - 1)) < 1e-15
    out, w = oracle.decode_attention(np.zeros((0, d), np.float32), np.zeros((0, d), np.float32), q)
    assert out.shape == (3, d) and np.all(out == 0)


def check_captured_importance():
    """The importance that decode attention can capture: the weights of the
    alpha window steps (the step of the token at position N - alpha + t sees
    keys 0 .. N - alpha + t, its own included), summed per key, divided by
    alpha and maxed over the group, equal the oracle's importance, which is
    pinned on its own by the hand cases and the textbook pipeline."""
    for seed, (n, d, g, a, budget) in enumerate([(40, 16, 3, 4, 24), (70, 32, 5, 8, 40), (33, 8, 1, 1, 20),
                                                 (50, 16, 2, 6, 30)]):
        k_bits, q_bits = _rand_slice(300 + seed, n, d, g, a)
        v_bits = synth.bf16_bits(np.random.default_rng(400 + seed).standard_normal((n, d)).astype(np.float32))
        acc = np.zeros((g, n))
        for t in range(a):
            m = n - a + t + 1
            _, w = oracle.decode_attention(k_bits[:m], v_bits[:m], q_bits[:, t])
            acc[:, :m] += w
        ref = oracle.slice_eval(k_bits, q_bits, budget=budget, obs_window=a)
        _close(acc.max(0) / a, ref.importance, 1e-15, f"captured importance, case {seed}")


ALL_CHECKS = [
    check_hand_cases,
    check_lambda1_textbook,
    check_single_query_softmax,
    check_probability_sums,
    check_rowmean_identity,
    check_exact_duplicates,
    check_orthogonal_keys,
    check_scale_invariance,
    check_budget_invariants,
    check_bruteforce_topk,
    check_lambda0_least_redundant,
    check_step_noop_and_compaction,
    check_holefill_hand_cases,
    check_holefill_invariants,
    check_holefill_rejects_bad_order,
    check_sampled_top_k_is_deterministic,
    check_sampled_equal_scores,
    check_sampled_inclusion_probabilities,
    check_sampled_scale_invariance,
    check_sentence_penalty_closed_forms,
    check_penalized_selection,
    check_decode_attention_textbook,
    check_decode_attention_special_cases,
    check_captured_importance,
]
