"""The long-generation sweep: successive eviction rounds of `buffer` new
tokens each on an evolving cache (R-KV notes page, summary table, row
"throughput": 16K generated tokens at a 10 % budget and at budget 1024, i.e.
125 rounds of 128 tokens). Every round the oracle runs on an exact copy of
the pre-eviction bytes the GPU holds (lockstep), so a kept-set difference
inside the tolerance band in one round cannot make later rounds diverge.
Each checked slice must keep the oracle's set up to the band rule and hold,
after compaction, exactly the pre-eviction rows of the keep lists the step
wrote (bit-exact K and V).
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import replace

import numpy as np
import pytest

import _gpu
import oracle
import synth

pytestmark = pytest.mark.gpu


def run_sweep(w, rounds, picks, threads=8):
    """Runs `rounds` eviction rounds of workload w on the device, checking
    the slices `picks` ([(l, b, h)]) every round. The host draws round r + 1
    while round r is evicted and checked. Returns (slices checked, kept-set
    differences inside the band)."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    sw = synth.Sweep(w, seed=0, threads=threads)
    ds = synth.DeviceSweep(sw)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    keep_all = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).view(w.slices, w.budget)
    B, N, G = w.budget, w.budget + w.buffer, w.group
    sl = [_gpu.slice_index(w, *t) for t in picks]
    ndiff = nchecked = 0
    with ThreadPoolExecutor(threads) as pool, ThreadPoolExecutor(1) as gen:
        nxt = gen.submit(sw.begin_round, 0)
        for r in range(rounds):
            rnd = ds.next_round(r, nxt.result())
            if r + 1 < rounds:
                nxt = gen.submit(sw.begin_round, r + 1)
            pre = [(ds.host(ds.K[l, b, h, :N]), ds.host(ds.V[l, b, h, :N])) for (l, b, h) in picks]
            st, ns = rkv.rkv_evict_step(p, ds.k_layers(), ds.v_layers(), ds.Q, ds.seq_start, ds.n_slots, ws, wsb)
            assert ns == B, f"round {r}: n_slots {ns}"
            ds.n_slots = ns
            torch.cuda.synchronize()
            assert not ds.seq_start.any(), f"round {r}: every sequence keeps budget tokens from slot 0"
            refs = pool.map(lambda i: oracle.slice_eval(
                pre[i][0], rnd.Q[picks[i][0], picks[i][1], picks[i][2] * G:(picks[i][2] + 1) * G], budget=B,
                obs_window=w.obs_window, beta=w.beta, lam=w.lam, tau=w.tau, amb_eps=_gpu.TAU_BAND),
                range(len(picks)))
            keeps = keep_all[sl].cpu().numpy()
            post = [(ds.host(ds.K[l, b, h, :B]), ds.host(ds.V[l, b, h, :B])) for (l, b, h) in picks]
            for (l, b, h), (k0, v0), ref, keep, (k1, v1) in zip(picks, pre, refs, keeps, post):
                what = f"round {r} slice {(l, b, h)}"
                assert np.all(keep >= 0), f"{what}: full sequences keep every destination slot"
                ndiff += _gpu.check_keep(keep.astype(np.int64), ref, w, N, what=what)
                assert np.array_equal(k1, k0[keep]), f"{what}: K rows"
                assert np.array_equal(v1, v0[keep]), f"{what}: V rows"
                nchecked += 1
    return nchecked, ndiff


REDUCED = {
    # the sweep's budgets and window at a reduced shape: every slice checked
    # in each of the 125 rounds
    "sweep10pct_reduced": replace(synth.WORKLOADS["llama8b_b16_sweep10pct"], name="sweep10pct_reduced", wid=110,
                                  num_layers=1, batch=2, num_kv_heads=2),
    "sweep1024_reduced": replace(synth.WORKLOADS["llama8b_b16_sweep1024"], name="sweep1024_reduced", wid=111,
                                 num_layers=1, batch=2, num_kv_heads=2),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_sweep_every_round_every_slice(name):
    w = REDUCED[name]
    every = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    n, ndiff = run_sweep(w, synth.SweepRecipe().rounds, every)
    print(f"{name}: {n} slice-rounds checked; kept-set differences inside the band: {ndiff}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama8b_b16_sweep10pct", "llama8b_b16_sweep1024"])
def test_sweep_full_shape(name):
    """The full 32-layer, batch-16 shape over all 125 rounds, the same 32
    slices checked in lockstep every round: layers 0, 15 and 31 x every KV
    head of sequence 0, plus seeded random slices."""
    w = synth.WORKLOADS[name]
    picks = synth.sweep_sample(w, 32)
    assert len(picks) == 32
    n, ndiff = run_sweep(w, synth.SweepRecipe().rounds, picks, threads=16)
    assert n == 32 * synth.SweepRecipe().rounds
    print(f"{name}: {n} slice-rounds checked (32 slices x 125 rounds); kept-set differences inside the band: "
          f"{ndiff}, outside: 0")
