"""The hole-filling layout (order-free compaction with an order sidecar) on
the GPU against the oracle. The pages name copying the kept entries and
re-arranging the cache as costs of pruning (R-KV notes page, Q&A part 2,
causes 3 and 4); this layout moves only the kept tokens that arrived since
the last eviction.

- Compaction alone: random order permutations and keep lists, bit-exact
  against oracle.holefill_slice (K, V, order, seq_start).
- The whole step on a physically scrambled cache: the scores are computed
  on the virtual order, so the keep lists equal those of the
  order-preserving step on the unscrambled cache, and the result equals the
  oracle's hole-filling compaction of the scrambled bytes with those lists;
  sampled slices are also checked against the oracle's own selection.
- The long-generation sweep in this layout, lockstep with the oracle.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import replace

import numpy as np
import pytest

import _gpu
import oracle
import synth

pytestmark = pytest.mark.gpu

SMALL = {
    "small_ragged": synth.small("small_ragged", 101, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                                lengths=("uniform", 200, 384)),
    "small_a4": synth.small("small_a4", 103, num_layers=1, batch=2, num_kv_heads=2, group=3, budget=200, buffer=77,
                            obs_window=4, extra_capacity=40),
    "single_f32": synth.WORKLOADS["single_f32"],
    # the largest budget the hole-filling compaction takes (its LDS lists: 6 bytes per budget slot)
    "max_budget": synth.small("hf_max_budget", 141, num_layers=1, batch=1, num_kv_heads=1, group=2, budget=10000),
}


def scramble(cs, seed):
    """A random physical layout of the cache: per slice a permutation order of
    [0, budget) and the rows of virtual slot v < budget moved to order[v]."""
    w = cs.w
    rng = np.random.default_rng(seed)
    order = np.empty((w.num_layers, w.batch, w.num_kv_heads, w.budget), np.int32)
    K, V = cs.K.copy(), cs.V.copy()
    for l in range(w.num_layers):
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                o = rng.permutation(w.budget).astype(np.int32)
                order[l, b, h] = o
                K[l, b, h, o] = cs.K[l, b, h, :w.budget]
                V[l, b, h, o] = cs.V[l, b, h, :w.budget]
    return K, V, order


def dev_i32(a):
    torch, dev = _gpu.torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def oracle_holefill_all(w, K, V, order, keep, n_slots):
    """oracle.holefill_slice over every slice; returns (K', V', order', starts per sequence)."""
    K2, V2, O2 = K.copy(), V.copy(), order.copy()
    starts = np.zeros(w.batch, np.int32)
    for l in range(w.num_layers):
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                s = _gpu.slice_index(w, l, b, h)
                kk, vv, oo, lead = oracle.holefill_slice(K[l, b, h, :n_slots], V[l, b, h, :n_slots],
                                                         order[l, b, h], keep[s], w.budget)
                K2[l, b, h, :n_slots], V2[l, b, h, :n_slots], O2[l, b, h] = kk, vv, oo
                starts[b] = lead
    return K2, V2, O2, starts


@pytest.mark.parametrize("name", list(SMALL))
def test_compact_holefill_bit_exact(name):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = SMALL[name]
    cs = synth.build_cache(w, seed=0)
    K, V, order = scramble(cs, 11)
    rng = np.random.default_rng(3)
    n = cs.n_slots
    keep = np.full((w.slices, w.budget), -1, np.int32)
    for l in range(w.num_layers):
        for b in range(w.batch):
            N = int(cs.lengths[b])
            kept = min(N, w.budget)
            for h in range(w.num_kv_heads):
                s0 = n - N
                sel = np.sort(rng.choice(np.arange(s0, n), size=kept, replace=False))
                keep[_gpu.slice_index(w, l, b, h), w.budget - kept:] = sel
    Kd, Vd = _gpu.to_dev(K), _gpu.to_dev(V)
    Od, Sd = dev_i32(order), dev_i32(cs.seq_start)
    p = _gpu.params_of(w)
    rkv.rkv_compact_holefill(p, [Kd[l] for l in range(w.num_layers)], [Vd[l] for l in range(w.num_layers)],
                             dev_i32(keep), Sd, Od, n)
    torch.cuda.synchronize()
    K2, V2, O2, starts = oracle_holefill_all(w, K, V, order, keep, n)
    assert np.array_equal(Od.cpu().numpy(), O2)
    assert np.array_equal(Sd.cpu().numpy(), starts)
    assert np.array_equal(_gpu.to_host(Kd, K.dtype).view(np.uint8), K2.view(np.uint8))
    assert np.array_equal(_gpu.to_host(Vd, V.dtype).view(np.uint8), V2.view(np.uint8))


FULL_SAMPLE = [(0, 0, 0), (7, 0, 5), (31, 0, 7)]


@pytest.mark.parametrize("name", list(SMALL) + ["llama8b_b1"])
def test_evict_step_holefill(name):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = SMALL.get(name) or synth.WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    n = cs.n_slots

    def keep_of(ws):
        return ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).cpu().numpy().reshape(w.slices, w.budget)

    # the order-preserving step on the unscrambled cache
    dc = _gpu.DevCache.of(cs)
    ws0 = torch.empty(wsb, dtype=torch.uint8, device=dev)
    rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, n, ws0, wsb)
    torch.cuda.synchronize()
    keep_ref = keep_of(ws0)
    del dc
    # the hole-filling step on a scrambled copy
    K, V, order = scramble(cs, 5)
    Kd, Vd, Od, Sd = _gpu.to_dev(K), _gpu.to_dev(V), dev_i32(order), dev_i32(cs.seq_start)
    Qd = _gpu.to_dev(cs.Q)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step_holefill(p, [Kd[l] for l in range(w.num_layers)],
                                         [Vd[l] for l in range(w.num_layers)], Qd, Sd, Od, n, ws, wsb)
    torch.cuda.synchronize()
    assert ns == w.budget
    keep = keep_of(ws)
    assert np.array_equal(keep, keep_ref), "scores on the virtual order differ from the unscrambled step"
    K2, V2, O2, starts = oracle_holefill_all(w, K, V, order, keep, n)
    assert np.array_equal(Od.cpu().numpy(), O2)
    assert np.array_equal(Sd.cpu().numpy(), starts)
    assert np.array_equal(_gpu.to_host(Kd, K.dtype).view(np.uint8), K2.view(np.uint8))
    assert np.array_equal(_gpu.to_host(Vd, V.dtype).view(np.uint8), V2.view(np.uint8))
    # the selection against the oracle's own on sampled slices
    picks = FULL_SAMPLE if name == "llama8b_b1" else [
        (l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    for (l, b, h) in picks:
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        ref = _gpu.oracle_slice(cs, l, b, h)
        _gpu.check_keep(_gpu.keep_rel_of(keep[s], s0), ref, w, N, what=f"{name} {(l, b, h)}")


def test_sweep_holefill_lockstep():
    """125 rounds of the long-generation sweep in the hole-filling layout (a
    reduced shape at the 10 % budget): each round's new tokens go to the
    physical slots past the budget, the step scores the virtual order, and
    the oracle checks every slice in lockstep on the virtual pre-eviction
    rows: the kept set (band rule) and, bit-exactly, the compacted rows and
    the new order."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = replace(synth.WORKLOADS["llama8b_b16_sweep10pct"], name="sweep10pct_holefill", wid=112, num_layers=1,
                batch=2, num_kv_heads=2)
    sw = synth.Sweep(w, seed=0, threads=8)
    ds = synth.DeviceSweep(sw, order=True)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    keep_all = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).view(w.slices, w.budget)
    B, N, G = w.budget, w.budget + w.buffer, w.group
    slices = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    moved_total, ndiff = 0, 0
    with ThreadPoolExecutor(8) as pool:
        for r in range(synth.SweepRecipe().rounds):
            rnd = ds.next_round(r)
            Kp, Vp, Op = ds.host(ds.K), ds.host(ds.V), ds.order.cpu().numpy()
            st, ns = rkv.rkv_evict_step_holefill(p, ds.k_layers(), ds.v_layers(), ds.Q, ds.seq_start, ds.order,
                                                 ds.n_slots, ws, wsb)
            assert ns == B
            ds.n_slots = ns
            torch.cuda.synchronize()
            keep = keep_all.cpu().numpy()
            K1, V1, O1 = ds.host(ds.K), ds.host(ds.V), ds.order.cpu().numpy()

            def virt(l, b, h):
                rows = np.concatenate([Op[l, b, h], np.arange(B, N)])
                return Kp[l, b, h][rows]

            refs = list(pool.map(lambda t: oracle.slice_eval(
                virt(*t), rnd.Q[t[0], t[1], t[2] * G:(t[2] + 1) * G], budget=B, obs_window=w.obs_window,
                beta=w.beta, lam=w.lam, tau=w.tau, amb_eps=_gpu.TAU_BAND), slices))
            for (l, b, h), ref in zip(slices, refs):
                what = f"round {r} slice {(l, b, h)}"
                s = _gpu.slice_index(w, l, b, h)
                assert np.all(keep[s] >= 0), what
                ndiff += _gpu.check_keep(keep[s].astype(np.int64), ref, w, N, what=what)
                k2, v2, o2, lead = oracle.holefill_slice(Kp[l, b, h, :N], Vp[l, b, h, :N], Op[l, b, h], keep[s], B)
                assert lead == 0 and np.array_equal(O1[l, b, h], o2), what
                assert np.array_equal(K1[l, b, h, :N].view(np.uint8), k2.view(np.uint8)), what
                assert np.array_equal(V1[l, b, h, :N].view(np.uint8), v2.view(np.uint8)), what
                moved_total += int((keep[s] >= B).sum())
            assert not ds.seq_start.any()
    print(f"holefill sweep: band differences {ndiff}, rows moved per slice and round "
          f"{moved_total / (125 * len(slices)):.1f}")
