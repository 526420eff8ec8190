"""The sampled selection (ForesightKV explainer, technical summary: keep the
newest L tokens, compress the rest to budget - L by a Top-K followed by
multinomial sampling on a scorer's importance) on the GPU against the
oracle, with the caller-side scores and uniforms from the seeded generator.

The Top-K stage compares the same float32 scores on both sides, so it must
agree exactly. The draw compares Gumbel keys score/T - log(-log u), float32
on the GPU and double in the oracle: kept sets may differ only at candidates
whose key lies within GUMBEL_BAND of the oracle's last kept key.
"""
import numpy as np
import pytest

import _gpu
import oracle
import synth

pytestmark = pytest.mark.gpu

# float32 logf is within a few ulp; |key| stays below ~30 for u in
# [2^-25, 1 - 2^-25] and unit-variance scores: 2e-5 covers the rounding.
GUMBEL_BAND = 2e-5

WORKLOADS = {
    "small_ragged": synth.small("small_ragged", 101, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                                lengths=("uniform", 200, 384)),
    "small_b96": synth.small("small_b96", 120, num_layers=1, batch=2, num_kv_heads=3, group=4, budget=96, buffer=40),
    "llama8b_b1": synth.WORKLOADS["llama8b_b1"],
    # the largest capacity: one slice of 16,384 slots (16,376 candidates)
    "max_capacity": synth.small("max_capacity_sampled", 150, num_layers=1, batch=1, num_kv_heads=1, group=1,
                                budget=16384 - 128),
}


def keys_double(sc, un, T):
    return sc.astype(np.float64) / T - np.log(-np.log(un.astype(np.float64)))


def check_sampled(keep_rel, ref, sc, un, N, B, L, top_k, T, what):
    assert len(keep_rel) == min(N, B), what
    if N <= B:
        assert keep_rel.tolist() == list(range(N)), what
        return 0
    nc, kk = N - L, B - L
    assert set(range(nc, N)) <= set(keep_rel.tolist()), what
    K = min(max(top_k, kk), nc)
    top = set(sorted(range(nc), key=lambda i: (-float(sc[i]), -i))[:K])
    g = set(int(i) for i in keep_rel if i < nc)
    assert g <= top, f"{what}: kept outside the top {K} by score"
    r = set(int(i) for i in ref if i < nc)
    diff = g ^ r
    if diff:
        key = keys_double(sc[:nc], un[:nc], T)
        kth = min(key[i] for i in r)
        outside = [i for i in diff if abs(key[i] - kth) > GUMBEL_BAND]
        assert not outside, f"{what}: kept sets differ outside the band at {sorted(outside)[:8]}"
    return len(diff)


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("mode", ["deterministic", "top_2x", "all", "hot"])
def test_select_sampled_parity(name, mode):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    sc, un = synth.sampled_inputs(w, seed=0)
    L = w.buffer if w.buffer < w.budget else w.budget // 2
    kk = w.budget - L
    top_k, T = {"deterministic": (kk, 1.0), "top_2x": (2 * kk, 1.0), "all": (1 << 20, 1.0),
                "hot": (2 * kk, 0.25)}[mode]
    p = _gpu.params_of(w)
    keep = torch.full((w.slices * w.budget,), -9, dtype=torch.int32, device=dev)
    S = torch.from_numpy(cs.seq_start.copy()).to(dev)
    rkv.rkv_select_sampled(p, _gpu.to_dev(sc.reshape(-1)), _gpu.to_dev(un.reshape(-1)), S, cs.n_slots, L, top_k, T,
                           keep)
    torch.cuda.synchronize()
    keep = keep.cpu().numpy().reshape(w.slices, w.budget)
    picks = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    if name == "llama8b_b1":
        picks = picks[::17]
    ndiff = 0
    for (l, b, h) in picks:
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        x, u = sc[l, b, h, s0:cs.n_slots], un[l, b, h, s0:cs.n_slots]
        ref = oracle.select_sampled(x, u, w.budget, L, top_k, T)
        rel = _gpu.keep_rel_of(keep[s], s0)
        ndiff += check_sampled(rel, ref, x, u, N, w.budget, L, top_k, T, f"{name} {mode} {(l, b, h)}")
        if N > w.budget:
            assert np.all(keep[s][: w.budget - min(N, w.budget)] == -1)
    if mode == "deterministic":
        assert ndiff == 0
    print(f"{name} {mode}: kept-set differences inside the Gumbel band: {ndiff}")


def run_sampled(w, cs, sc, un, L, top_k, T):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    keep = torch.full((w.slices * w.budget,), -9, dtype=torch.int32, device=dev)
    S = torch.from_numpy(cs.seq_start.copy()).to(dev)
    rkv.rkv_select_sampled(_gpu.params_of(w), _gpu.to_dev(sc.reshape(-1)), _gpu.to_dev(un.reshape(-1)), S,
                           cs.n_slots, L, top_k, T, keep)
    torch.cuda.synchronize()
    return keep.cpu().numpy().reshape(w.slices, w.budget)


def check_all_slices(w, cs, sc, un, keep, L, top_k, T, what):
    ndiff = 0
    for l in range(w.num_layers):
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                s = _gpu.slice_index(w, l, b, h)
                s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
                x, u = sc[l, b, h, s0:cs.n_slots], un[l, b, h, s0:cs.n_slots]
                ref = oracle.select_sampled(x, u, w.budget, L, top_k, T)
                ndiff += check_sampled(_gpu.keep_rel_of(keep[s], s0), ref, x, u, N, w.budget, L, top_k, T,
                                       f"{what} {(l, b, h)}")
    return ndiff


@pytest.mark.parametrize("mode", ["deterministic", "top_2x"])
def test_select_sampled_tied_scores(mode):
    """Scores rounded to multiples of 0.5: most candidates share their score
    with many others, so the Top-K threshold falls inside a large run of equal
    keys and the tie rule (the later slot) decides which of them stay. That
    stage compares the same float32 values on both sides: with top_k equal to
    budget - L the kept sets must match exactly."""
    w = WORKLOADS["small_ragged"]
    cs = synth.build_cache(w, seed=0)
    sc, un = synth.sampled_inputs(w, seed=2)
    sc = (np.round(sc * 2.0) / 2.0).astype(np.float32)
    L = 64
    kk = w.budget - L
    top_k = kk if mode == "deterministic" else 2 * kk
    keep = run_sampled(w, cs, sc, un, L, top_k, 1.0)
    ndiff = check_all_slices(w, cs, sc, un, keep, L, top_k, 1.0, f"tied {mode}")
    if mode == "deterministic":
        assert ndiff == 0


@pytest.mark.parametrize("L", [0, 1, 255])
def test_select_sampled_keep_newest_limits(L):
    """keep_newest at its limits (0 <= L < budget): no protected window, a
    window of one, and a single drawn candidate (budget - L = 1)."""
    w = WORKLOADS["small_ragged"]
    assert L < w.budget
    cs = synth.build_cache(w, seed=0)
    sc, un = synth.sampled_inputs(w, seed=3)
    for top_k, T in ((0, 1.0), (3 * (w.budget - L), 0.5)):
        keep = run_sampled(w, cs, sc, un, L, top_k, T)
        ndiff = check_all_slices(w, cs, sc, un, keep, L, top_k, T, f"L={L} top_k={top_k}")
        if top_k == 0:  # raised to budget - L: the pure Top-K, exact
            assert ndiff == 0


def test_evict_step_sampled():
    """The step: the sampled keep lists (in the workspace) and the
    order-preserving compaction of K and V by them, bit-exact."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = WORKLOADS["small_ragged"]
    cs = synth.build_cache(w, seed=0)
    sc, un = synth.sampled_inputs(w, seed=1)
    dc = _gpu.DevCache.of(cs)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    L, top_k = 64, 300
    st, ns = rkv.rkv_evict_step_sampled(p, dc.k_layers(), dc.v_layers(), _gpu.to_dev(sc.reshape(-1)),
                                        _gpu.to_dev(un.reshape(-1)), dc.seq_start, cs.n_slots, L, top_k, 1.0, ws, wsb)
    torch.cuda.synchronize()
    assert ns == w.budget
    keep = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).cpu().numpy().reshape(w.slices, w.budget)
    K1, V1 = _gpu.to_host(dc.K, cs.K.dtype), _gpu.to_host(dc.V, cs.V.dtype)
    s_new = dc.seq_start.cpu().numpy()
    for l in range(w.num_layers):
        for b in range(w.batch):
            N, s0 = int(cs.lengths[b]), int(cs.seq_start[b])
            kept = min(N, w.budget)
            assert s_new[b] == w.budget - kept
            for h in range(w.num_kv_heads):
                s = _gpu.slice_index(w, l, b, h)
                src = keep[s][w.budget - kept:]
                assert np.array_equal(K1[l, b, h, w.budget - kept:w.budget], cs.K[l, b, h][src])
                assert np.array_equal(V1[l, b, h, w.budget - kept:w.budget], cs.V[l, b, h][src])
                ref = oracle.select_sampled(sc[l, b, h, s0:cs.n_slots], un[l, b, h, s0:cs.n_slots], w.budget, L,
                                            top_k, 1.0)
                check_sampled(_gpu.keep_rel_of(keep[s], s0), ref, sc[l, b, h, s0:cs.n_slots],
                              un[l, b, h, s0:cs.n_slots], N, w.budget, L, top_k, 1.0, f"step {(l, b, h)}")
