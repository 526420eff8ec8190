"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same
seeded inputs. Small workloads compare every slice; the full-size workloads
compare a fixed sample of slices the oracle can afford, plus properties that
hold at any size (self-consistent top-k, bit-exact compaction of every slice).
"""
import numpy as np
import pytest

import _gpu
import oracle
import synth

pytestmark = pytest.mark.gpu

SMALL = {
    # ragged lengths (some sequences below the budget), several 128-key tiles, ragged tail
    "small_ragged": synth.small("small_ragged", 101, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                                lengths=("uniform", 200, 384)),
    # group 5 (40 query rows: two MFMA row tiles), n_slots 400 is not a multiple of 64
    "small_g5": synth.small("small_g5", 102, num_layers=1, batch=1, num_kv_heads=3, group=5, budget=300, buffer=100),
    # window 4, group 3, capacity past n_slots (canary rows)
    "small_a4": synth.small("small_a4", 103, num_layers=1, batch=2, num_kv_heads=2, group=3, budget=200, buffer=77,
                            obs_window=4, extra_capacity=40),
    # stronger repetition so that many tokens lose protection
    "small_dup": synth.small("small_dup", 104, num_layers=1, batch=1, num_kv_heads=4, group=4, budget=256,
                             copy_frac=0.6, span_len=16),
    # window sums not aligned to the MFMA row layout (window 6, 18 query rows)
    "small_a6": synth.small("small_a6", 105, num_layers=1, batch=2, num_kv_heads=2, group=3, budget=192, buffer=64,
                            obs_window=6),
    # window 16 over two query-row tiles; window 64 spans both tiles (group 1)
    "small_a16": synth.small("small_a16", 106, num_layers=1, batch=1, num_kv_heads=2, group=4, budget=160, buffer=96,
                             obs_window=16),
    "small_a64": synth.small("small_a64", 107, num_layers=1, batch=1, num_kv_heads=2, group=1, budget=320, buffer=50,
                             obs_window=64),
    "single_f32": synth.WORKLOADS["single_f32"],
    # more tokens than the scoring kernel keeps norms of in LDS: the later
    # column groups recompute the newest blocks' norms
    "small_long": synth.small("small_long", 108, num_layers=1, batch=1, num_kv_heads=2, group=4, budget=5600),
    # the largest capacity the library takes (RKV_MAX_CAPACITY = 16384 slots): 32 column groups,
    # norms past the scoring kernel's LDS cache, the selection's full key array
    "max_capacity": synth.small("max_capacity", 122, num_layers=1, batch=1, num_kv_heads=1, group=4,
                                budget=16384 - 128),
    # a negative similarity threshold on ragged sequences whose slot count (356) is not a multiple of the
    # scoring kernel's 64-row blocks: rows past a slice must never count as similar, whatever tau's sign
    "small_negtau": synth.small("small_negtau", 124, num_layers=1, batch=3, num_kv_heads=2, group=4, budget=256,
                                buffer=100, lengths=("uniform", 200, 356), tau=-0.25),
    # fp32 keys over three compaction chunks of 256 rows (an odd count, a partial last chunk), ragged
    "f32_chunks": synth.small("f32_chunks", 126, num_layers=1, batch=2, num_kv_heads=2, group=2, budget=700,
                              dtype="f32", lengths=("uniform", 500, 828)),
}

# the full-size workloads; their slices are sampled by sample_of
FULL = ["llama8b_b1", "llama8b_b32_ragged", "qwen14b_b8"]
SAMPLE = 64  # slices per sampled full-size workload

_cache = {}
_refs = {}


def cache_of(name):
    """Host inputs of a workload (seed 0) and a fresh device copy."""
    if name not in _cache:
        w = SMALL.get(name) or synth.WORKLOADS[name]
        _cache.clear()  # keep at most one workload resident
        _cache[name] = synth.build_cache(w, seed=0)
    cs = _cache[name]
    return cs, _gpu.DevCache.of(cs)


def sample_of(name, cs):
    """Every slice of a small workload and of the 256-slice batch-1 cache;
    otherwise a fixed seeded sample of SAMPLE slices: the first, middle and
    last layer x every KV head of the first evicting sequence, plus random
    evicting slices (and, on the ragged batch, four non-evicting ones)."""
    w = cs.w
    every = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    if name in SMALL or len(every) <= 256:
        return every
    ev = [b for b in range(w.batch) if cs.lengths[b] > w.budget]
    non = [b for b in range(w.batch) if cs.lengths[b] <= w.budget][:4]
    L = w.num_layers
    picks = [(l, ev[0], h) for l in (0, L // 2, L - 1) for h in range(w.num_kv_heads)]
    picks += [(0, b, 0) for b in non]
    rng = np.random.default_rng(7)
    while len(picks) < SAMPLE:
        t = (int(rng.integers(L)), int(ev[rng.integers(len(ev))]), int(rng.integers(w.num_kv_heads)))
        if t not in picks:
            picks.append(t)
    return picks


def refs_of(name, cs):
    """The oracle on every sampled slice (computed once per workload, one
    slice per task on a thread pool; the oracle itself is single-threaded)."""
    from concurrent.futures import ThreadPoolExecutor

    if name not in _refs:
        _refs.clear()
        sample = sample_of(name, cs)
        with ThreadPoolExecutor(16) as pool:
            out = list(pool.map(lambda t: _gpu.oracle_slice(cs, *t), sample))
        _refs[name] = dict(zip(sample, out))
    return _refs[name]


ALL = list(SMALL) + FULL


@pytest.mark.parametrize("name", ALL)
def test_score_parity(name):
    """I, counts and rbar of the GPU against the oracle; then the selection
    fed the GPU's own scores: its Z and R against the oracle's (rows whose
    counts sit on a tau-ambiguous pair excepted, like the counts)."""
    cs, dc = cache_of(name)
    w = cs.w
    imp, red, cnt = _gpu.gpu_score(dc)
    _, z, r = _gpu.gpu_select(dc, imp, red)
    band_rows = checked = 0
    for (l, b, h), ref in refs_of(name, cs).items():
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        if N <= w.budget:
            assert np.all(cnt[s] == -7), "non-evicting sequences must not be scored"
            continue
        what = f"{name} {(l, b, h)}"
        band_rows += _gpu.check_scores(ref, imp[s, s0:], red[s, s0:], cnt[s, s0:], what=what)
        _gpu.check_z_r(ref, z[s, s0:], r[s, s0:], w, N, what=what)
        checked += 1
    print(f"{name}: {checked} scored slices checked; rows with a pair in the tau band: {band_rows}")


@pytest.mark.parametrize("name", ALL)
def test_select_parity(name):
    """Selection fed with the oracle's own scores (as fp32)."""
    cs, dc = cache_of(name)
    w = cs.w
    n = cs.n_slots
    imp = np.zeros((w.slices, n), np.float32)
    red = np.zeros((w.slices, n), np.float32)
    refs = refs_of(name, cs)
    for (l, b, h), ref in refs.items():
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        if N > w.budget:
            imp[s, s0:] = ref.importance
            red[s, s0:] = ref.rbar
    keep, z, r = _gpu.gpu_select(dc, imp, red)
    ndiff = 0
    for (l, b, h), ref in refs.items():
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        row = keep[s]
        assert np.all(row[: w.budget - min(N, w.budget)] == -1)
        rel = _gpu.keep_rel_of(row, s0)
        if N > w.budget:
            nc = N - w.obs_window
            eps = _gpu.REL_TOL * (w.lam * ref.importance[:nc] + (1 - w.lam) * ref.R[:nc])
            assert np.all(np.abs(z[s, s0:s0 + nc] - ref.Z[:nc]) <= eps + 1e-12), f"{name} Z"
            assert np.all(np.abs(r[s, s0:s0 + nc] - ref.R[:nc]) <= _gpu.REL_TOL * ref.R[:nc]), f"{name} R"
            _gpu.check_self_topk(rel, z[s, s0:], w, N, what=f"{name} {(l, b, h)}")
        ndiff += _gpu.check_keep(rel, ref, w, N, what=f"{name} {(l, b, h)}")
    print(f"{name}: kept-set differences inside the band: {ndiff}")


def _random_keep(rng, B, n_slots, N):
    """A valid keep row: ascending sources, right-aligned, keep[j] >= j."""
    kept = min(N, B)
    s0 = n_slots - N
    if N <= B:
        src = s0 + np.arange(N)
    else:
        mode = rng.integers(0, 4)
        if mode == 0:  # drop a random subset
            src = s0 + np.sort(rng.choice(N, size=B, replace=False))
        elif mode == 1:  # drop only the oldest (every row moves by the same offset)
            src = s0 + np.arange(N - B, N)
        elif mode == 2:  # drop only the newest candidates (long stable prefix)
            src = s0 + np.concatenate([np.arange(B - 8), np.arange(N - 8, N)])
        else:  # drop one early token (every later row shifts by one)
            src = s0 + np.delete(np.arange(N), 3)[:B]
    row = np.full(B, -1, np.int32)
    row[B - kept:] = src
    return row


@pytest.mark.parametrize("name", ["small_ragged", "small_a4", "single_f32", "f32_chunks", "small_long", "llama8b_b1"])
def test_compact_bit_exact(name):
    """In-place compaction vs a plain gather of the pre-step bytes, adversarial keep patterns.
    The compaction moves rows in chunks (512 rows of bf16, 256 of fp32) with the next chunk's loads in
    flight during a chunk's stores: small_long spans 11 chunks, f32_chunks 3."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    cs, dc = cache_of(name)
    w = cs.w
    rng = np.random.default_rng(5)
    keep = np.stack([_random_keep(rng, w.budget, cs.n_slots, int(cs.lengths[b]))
                     for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)])
    tk = torch.from_numpy(keep.reshape(-1)).to(dev)
    rkv.rkv_compact(_gpu.params_of(w), dc.k_layers(), dc.v_layers(), tk, dc.seq_start, cs.n_slots)
    torch.cuda.synchronize()
    K1 = _gpu.to_host(dc.K, cs.K.dtype)
    V1 = _gpu.to_host(dc.V, cs.V.dtype)
    s_new = dc.seq_start.cpu().numpy()
    for l in range(w.num_layers):
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                row = keep[_gpu.slice_index(w, l, b, h)]
                exp_k = oracle.gather_rows(cs.K[l, b, h], row)
                exp_v = oracle.gather_rows(cs.V[l, b, h], row)
                m = row >= 0
                assert np.array_equal(K1[l, b, h, :w.budget][m].view(np.uint8), exp_k[m].view(np.uint8))
                assert np.array_equal(V1[l, b, h, :w.budget][m].view(np.uint8), exp_v[m].view(np.uint8))
                # padding destinations and rows past the budget are not written
                assert np.array_equal(K1[l, b, h, :w.budget][~m].view(np.uint8),
                                      cs.K[l, b, h, :w.budget][~m].view(np.uint8))
                assert np.array_equal(K1[l, b, h, w.budget:].view(np.uint8), cs.K[l, b, h, w.budget:].view(np.uint8))
            assert s_new[b] == w.budget - min(int(cs.lengths[b]), w.budget)


@pytest.mark.parametrize("name", ALL)
def test_evict_step(name):
    """The whole step: its compaction equals the gather of the pre-step bytes
    by the keep set that score + select produce (bit-exact, every slice), and
    that keep set matches the oracle's under the band rule (sampled slices)."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    cs, dc = cache_of(name)
    w = cs.w
    imp, red, _ = _gpu.gpu_score(dc)
    keep, z, _ = _gpu.gpu_select(dc, imp, red)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, ws, wsb)
    torch.cuda.synchronize()
    assert ns == w.budget
    s_new = dc.seq_start.cpu().numpy()
    K1 = _gpu.to_host(dc.K, cs.K.dtype)
    V1 = _gpu.to_host(dc.V, cs.V.dtype)
    del dc
    for l in range(w.num_layers):
        for b in range(w.batch):
            kept = min(int(cs.lengths[b]), w.budget)
            assert s_new[b] == w.budget - kept
            for h in range(w.num_kv_heads):
                row = keep[_gpu.slice_index(w, l, b, h)]
                src = row[w.budget - kept:]
                assert np.all(src >= 0) and np.all(row[: w.budget - kept] == -1)
                assert np.array_equal(K1[l, b, h, w.budget - kept:w.budget], cs.K[l, b, h][src])
                assert np.array_equal(V1[l, b, h, w.budget - kept:w.budget], cs.V[l, b, h][src])
                if w.capacity > w.n_slots:
                    assert np.array_equal(K1[l, b, h, w.n_slots:].view(np.uint8),
                                          cs.K[l, b, h, w.n_slots:].view(np.uint8))
    ndiff = 0
    refs = refs_of(name, cs)
    for (l, b, h), ref in refs.items():
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        rel = _gpu.keep_rel_of(keep[s], s0)
        if N > w.budget:
            _gpu.check_self_topk(rel, z[s, s0:], w, N, what=f"{name} {(l, b, h)}")
        ndiff += _gpu.check_keep(rel, ref, w, N, what=f"{name} {(l, b, h)}")
    print(f"{name}: {len(refs)} slices checked; kept-set differences inside the band: {ndiff}")


@pytest.mark.parametrize("name", ["small_ragged", "small_g5", "small_a4", "small_negtau", "max_capacity",
                                  "llama8b_b1"])
def test_fused_step_equals_staged(name):
    """rkv_evict_step scores, selects and compacts each slice in one launch
    (bf16 keys); rkv_evict_step_timed runs the same work as three kernels.
    Both leave bit-identical K and V caches, start slots and keep rows, for
    evicting and non-evicting sequences alike."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    cs, _ = cache_of(name)
    w = cs.w
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    out = []
    for staged in (False, True):
        dc = _gpu.DevCache.of(cs)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
        if staged:
            st, ns = rkv.rkv_evict_step_timed(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, ws,
                                              wsb, [0, 0, 0, 0])
        else:
            st, ns = rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, ws, wsb)
        torch.cuda.synchronize()
        assert ns == w.budget
        keep = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).cpu().numpy()
        out.append((_gpu.to_host(dc.K, cs.K.dtype).view(np.uint8), _gpu.to_host(dc.V, cs.V.dtype).view(np.uint8),
                    dc.seq_start.cpu().numpy(), keep))
        del dc
    for what, a, b in zip(("K", "V", "seq_start", "keep"), *out):
        assert np.array_equal(a, b), f"{name}: fused and staged steps differ in {what}"


def test_evict_step_degenerate():
    """One evicting batch with an empty sequence (N = 0), a one-token sequence
    and zero keys in an evicting sequence, one of them in the observation
    window. A zero key has no direction (unit key 0): no similarity with any
    key, row mean 0, logit 0. Scores against the oracle on every slice of the
    evicting sequence; the short sequences are not scored, keep everything
    and move right-aligned; compaction bit-exact; keep sets under the band
    rule."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = synth.small("degenerate", 151, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256)
    cs = synth.build_cache(w, seed=0)
    n = cs.n_slots
    cs.seq_start[0], cs.lengths[0] = n, 0
    cs.seq_start[1], cs.lengths[1] = n - 1, 1
    assert cs.lengths[2] == n > w.budget
    zero_rows = [5, 6, 100, n - 3]
    cs.K[:, 2, :, zero_rows] = 0
    dc = _gpu.DevCache.of(cs)
    imp, red, cnt = _gpu.gpu_score(dc)
    for l in range(w.num_layers):
        for h in range(w.num_kv_heads):
            for b in (0, 1):
                assert np.all(cnt[_gpu.slice_index(w, l, b, h)] == -7), "short sequences are not scored"
            s = _gpu.slice_index(w, l, 2, h)
            ref = _gpu.oracle_slice(cs, l, 2, h)
            assert np.all(ref.counts[zero_rows] == 0) and np.all(ref.rbar[zero_rows] == 0)
            _gpu.check_scores(ref, imp[s], red[s], cnt[s], what=f"degenerate {(l, 2, h)}")
            assert np.all(cnt[s][zero_rows] == 0) and np.all(red[s][zero_rows] == 0)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, n, ws, wsb)
    torch.cuda.synchronize()
    assert ns == w.budget
    keep = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).cpu().numpy().reshape(w.slices, w.budget)
    s_new = dc.seq_start.cpu().numpy()
    K1, V1 = _gpu.to_host(dc.K, cs.K.dtype), _gpu.to_host(dc.V, cs.V.dtype)
    for b in range(w.batch):
        N = int(cs.lengths[b])
        kept = min(N, w.budget)
        assert s_new[b] == w.budget - kept
        for l in range(w.num_layers):
            for h in range(w.num_kv_heads):
                s = _gpu.slice_index(w, l, b, h)
                row = keep[s]
                assert np.all(row[: w.budget - kept] == -1)
                src = row[w.budget - kept:]
                assert np.array_equal(K1[l, b, h, w.budget - kept:w.budget], cs.K[l, b, h][src])
                assert np.array_equal(V1[l, b, h, w.budget - kept:w.budget], cs.V[l, b, h][src])
                _gpu.check_keep(_gpu.keep_rel_of(row, int(cs.seq_start[b])), _gpu.oracle_slice(cs, l, b, h), w, N,
                                what=f"degenerate {(l, b, h)}")


def test_noop_below_trigger():
    """Below budget + buffer nothing is launched and the cache is bit-identical."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    cs, dc = cache_of("small_ragged")
    w = cs.w
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, w.n_slots - 1, ws, wsb)
    torch.cuda.synchronize()
    assert ns == w.n_slots - 1
    assert np.array_equal(_gpu.to_host(dc.K, cs.K.dtype).view(np.uint8), cs.K.view(np.uint8))
    assert np.array_equal(dc.seq_start.cpu().numpy(), cs.seq_start)


def test_deterministic():
    """Two steps on identical inputs give bit-identical caches and scores."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    cs, _ = cache_of("small_dup")
    w = cs.w
    outs = []
    for _ in range(2):
        dc = _gpu.DevCache.of(cs)
        imp, red, cnt = _gpu.gpu_score(dc)
        p = _gpu.params_of(w)
        wsb = rkv.rkv_workspace_bytes(p)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, ws, wsb)
        torch.cuda.synchronize()
        outs.append((imp, red, cnt, _gpu.to_host(dc.K, cs.K.dtype), _gpu.to_host(dc.V, cs.V.dtype)))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_stale_hip_error_does_not_fail_a_launch():
    """An error an earlier, unrelated HIP call left in the thread's last-error
    state (here hipSetDevice(-1), which changes nothing) must not be reported
    as a failure of the library's own launches: every launch returns its own
    status."""
    import ctypes

    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    hip = ctypes.CDLL("libamdhip64.so.7")
    cs, dc = cache_of("small_ragged")
    w = cs.w
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)  # no kernel launch: nothing clears the error below
    torch.cuda.synchronize()
    assert hip.hipSetDevice(-1) != 0
    st, ns = rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, ws, wsb,
                                check=False)
    torch.cuda.synchronize()
    hip.hipGetLastError()
    assert st == 0 and ns == w.budget, rkv.rkv_status_string(st)
