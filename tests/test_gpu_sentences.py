"""SkipKV's sentence-level redundancy (SkipKV notes page, summary table rows
"sentence-level KV storage skipping", "final eviction score" and "cache range
monitoring") on the GPU against the oracle, on synthetic sentence structure:
the sentence penalties, the eviction step with the penalty subtracted from Z,
and the sentence-id sidecar that moves with the compacted rows.
"""
import numpy as np
import pytest

import _gpu
import oracle
import synth

pytestmark = pytest.mark.gpu

TAU_S = 0.8
# fp32 dot products over 1024 dims: the cosine is within ~1e-6 of the double
# one; 1e-5 leaves headroom, for the values and for the threshold decision.
PEN_TOL = 1e-5

WORKLOADS = {
    "small_ragged": synth.small("small_ragged", 101, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                                lengths=("uniform", 200, 384)),
    "small_a4": synth.small("small_a4", 103, num_layers=1, batch=2, num_kv_heads=2, group=3, budget=200, buffer=77,
                            obs_window=4, extra_capacity=40),
    "llama8b_b1": synth.WORKLOADS["llama8b_b1"],
}


def dev_i32(a):
    torch, dev = _gpu.torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def oracle_penalties(se):
    return [oracle.sentence_penalty(se.vectors[b, :se.n_sent[b]], TAU_S) for b in range(len(se.n_sent))]


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_sentence_penalty_parity(name):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    se = synth.sentences(cs)
    s_max, dim = se.vectors.shape[1], se.vectors.shape[2]
    pen = torch.full((w.batch * s_max,), -5.0, dtype=torch.float32, device=dev)
    rkv.rkv_sentence_penalty(_gpu.params_of(w), _gpu.to_dev(se.vectors), dev_i32(se.n_sent), s_max, dim, TAU_S, pen)
    torch.cuda.synchronize()
    gpu = pen.cpu().numpy().reshape(w.batch, s_max)
    for b in range(w.batch):
        n = int(se.n_sent[b])
        v = se.vectors[b, :n].astype(np.float64)
        nr = np.linalg.norm(v, axis=1)
        cos = (v @ v.T) / np.outer(nr, nr)
        ref = oracle.sentence_penalty(se.vectors[b, :n], TAU_S)
        assert np.all(gpu[b, n:] == 0)
        for i in range(n):
            later = cos[i, i + 1:]
            at_threshold = np.any(np.abs(later - TAU_S) <= PEN_TOL)
            if gpu[b, i] > 0 and ref[i] > 0:
                assert abs(gpu[b, i] - ref[i]) <= PEN_TOL, (name, b, i, gpu[b, i], ref[i])
            else:
                assert (gpu[b, i] == 0) == (ref[i] == 0) or at_threshold, (name, b, i, gpu[b, i], ref[i])
    print(f"{name}: redundant sentences {int((gpu > 0).sum())} of {int(se.n_sent.sum())}")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_evict_step_sentences(name):
    """The step's kept sets against the oracle's penalised selection (the
    band rule, widened by the penalty tolerance), the order-preserving
    compaction of K and V and of the sentence sidecar, bit-exact."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    se = synth.sentences(cs)
    s_max, dim = se.vectors.shape[1], se.vectors.shape[2]
    dc = _gpu.DevCache.of(cs)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sid = dev_i32(se.sent_id)
    pen = torch.empty(w.batch * s_max, dtype=torch.float32, device=dev)
    st, ns = rkv.rkv_evict_step_sentences(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, sid,
                                          _gpu.to_dev(se.vectors), dev_i32(se.n_sent), s_max, dim, TAU_S, pen, ws,
                                          wsb)
    torch.cuda.synchronize()
    assert ns == w.budget
    keep = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).cpu().numpy().reshape(w.slices, w.budget)
    K1, V1 = _gpu.to_host(dc.K, cs.K.dtype), _gpu.to_host(dc.V, cs.V.dtype)
    sid1 = sid.cpu().numpy()
    refpen = oracle_penalties(se)
    picks = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    oracle_picks = picks[::37] if name == "llama8b_b1" else picks
    ndiff = 0
    for (l, b, h) in picks:
        s = _gpu.slice_index(w, l, b, h)
        N, s0 = int(cs.lengths[b]), int(cs.seq_start[b])
        kept = min(N, w.budget)
        src = keep[s][w.budget - kept:]
        assert np.all(keep[s][:w.budget - kept] == -1)
        assert np.array_equal(K1[l, b, h, w.budget - kept:w.budget], cs.K[l, b, h][src])
        assert np.array_equal(V1[l, b, h, w.budget - kept:w.budget], cs.V[l, b, h][src])
        assert np.array_equal(sid1[l, b, h, w.budget - kept:w.budget], se.sent_id[l, b, h][src])
        assert np.all(sid1[l, b, h, :w.budget - kept] == -1)
        if (l, b, h) not in oracle_picks:
            continue
        tokpen = np.zeros(N)
        ids = se.sent_id[l, b, h, s0:cs.n_slots]
        tokpen[ids >= 0] = refpen[b][ids[ids >= 0]]
        ref = oracle.slice_eval(cs.K[l, b, h, s0:cs.n_slots], cs.Q[l, b, h * w.group:(h + 1) * w.group],
                                budget=w.budget, obs_window=w.obs_window, beta=w.beta, lam=w.lam, tau=w.tau,
                                amb_eps=_gpu.TAU_BAND, token_penalty=tokpen)
        rel = _gpu.keep_rel_of(keep[s], s0)
        assert len(rel) == kept
        if N <= w.budget:
            assert rel.tolist() == list(range(N))
            continue
        nc, kk = N - w.obs_window, w.budget - w.obs_window
        g_set = set(int(x) for x in rel if x < nc)
        r_set = set(int(x) for x in ref.keep if x < nc)
        diff = g_set ^ r_set
        if diff:
            Z, I, R = ref.Z[:nc], ref.importance[:nc], ref.R[:nc]
            eps = _gpu.REL_TOL * (w.lam * np.abs(I) + (1 - w.lam) * np.abs(R)) + PEN_TOL
            order = sorted(range(nc), key=lambda i: (-Z[i], -i))
            kth = order[kk - 1]
            band = (np.abs(Z - Z[kth]) <= eps + eps[kth]) | ref.ambiguous[:nc].astype(bool)
            outside = [i for i in diff if not band[i]]
            assert not outside, f"{name} {(l, b, h)}: kept sets differ outside the band at {sorted(outside)[:8]}"
        ndiff += len(diff)
        # tokens of sentences with a large penalty go first
        # (a penalty above 0.5 outweighs every |Z| difference, which stays below 0.1)
        pen_c = tokpen[:nc]
        evicted = set(range(nc)) - g_set
        if (pen_c > 0.5).sum() >= nc - kk:
            assert all(pen_c[i] > 0.5 for i in evicted), f"{name} {(l, b, h)}: an unpenalised token went first"
        else:
            assert all(i in evicted for i in np.nonzero(pen_c > 0.5)[0]), f"{name} {(l, b, h)}: a penalised token stayed"
    print(f"{name}: kept-set differences inside the band: {ndiff}")


@pytest.mark.parametrize("dim", [4, 12, 100, 260, 8192])
def test_sentence_penalty_shapes(dim):
    """Vector widths that leave partial chunks (4, 12, 100, 260) and the
    largest accepted (8192); sequences with no sentence, one sentence, two,
    and more; a repeat planted in each longer sequence. Against the oracle to
    PEN_TOL, with the threshold exception of test_sentence_penalty_parity."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    rng = np.random.default_rng(dim)
    counts = np.array([0, 1, 2, 37], np.int32)
    s_max = 40
    vec = rng.standard_normal((len(counts), s_max, dim)).astype(np.float32)
    for b, n in enumerate(counts):
        if n >= 2:  # the first sentence is repeated by the last, with noise
            vec[b, n - 1] = vec[b, 0] + np.float32(0.1) * rng.standard_normal(dim).astype(np.float32)
    w = synth.small("sent_shapes", 140, num_layers=1, batch=len(counts), num_kv_heads=1, group=1, budget=64)
    pen = torch.full((len(counts) * s_max,), -5.0, dtype=torch.float32, device=dev)
    rkv.rkv_sentence_penalty(_gpu.params_of(w), _gpu.to_dev(vec), dev_i32(counts), s_max, dim, TAU_S, pen)
    torch.cuda.synchronize()
    gpu = pen.cpu().numpy().reshape(len(counts), s_max)
    for b, n in enumerate(counts):
        assert np.all(gpu[b, n:] == 0)
        if n == 0:
            continue
        ref = oracle.sentence_penalty(vec[b, :n], TAU_S)
        v = vec[b, :n].astype(np.float64)
        cos = (v @ v.T) / np.outer(np.linalg.norm(v, axis=1), np.linalg.norm(v, axis=1))
        for i in range(n):
            near = np.any(np.abs(cos[i, i + 1:] - TAU_S) <= PEN_TOL)
            if gpu[b, i] > 0 and ref[i] > 0:
                assert abs(gpu[b, i] - ref[i]) <= PEN_TOL, (dim, b, i, gpu[b, i], ref[i])
            else:
                assert (gpu[b, i] == 0) == (ref[i] == 0) or near, (dim, b, i, gpu[b, i], ref[i])
        if n >= 2:
            assert gpu[b, 0] > 0.9  # the planted repeat
