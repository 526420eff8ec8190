"""Decode attention with importance capture on the GPU against the oracle.

R-KV's importance is the attention that the newest alpha queries pay each
cached token (R-KV notes page, summary table row "importance computation");
the decode steps compute those rows anyway, and the notes name fusing
attention, importance scoring and eviction as the way to cut compression's
cost (Q&A part 2, cause 4).

- Output of one decode step (the window's last query) against
  oracle.decode_attention, on bf16 and fp32 caches, group sizes 1 to 8,
  ragged batches (one with 8192 slices, which takes the 256-thread
  work-groups) and a slice long enough for more than 64 KiB of weights.
- Edge cases: a sequence with no valid slot (output 0, accumulator
  untouched) and one whose only key is its own (output = its value, exactly).
- The alpha window steps with capture: max over the group of the sums / alpha
  against the oracle's importance, and against the scoring kernel's own
  importance on every slice.
- The eviction step that reads the captured importance: keep sets by the
  band rule, compaction bit-exact.

Tolerance of the output: logits are fp32 sums of 128 exact bf16 products, so
their error is at most ~128 * 2^-24 * sum |q_d k_d| / sqrt(128), below 6e-5
for these N(0, 1) inputs; the weights' relative error is about as large, and
the output, a convex combination of values of magnitude below ~5, is within
3e-4 plus a few ulp of accumulation. 5e-4 absolute leaves headroom.
"""
import numpy as np
import pytest

import _gpu
import oracle
import synth

pytestmark = pytest.mark.gpu

OUT_TOL = 5e-4

WORKLOADS = {
    "small_ragged": synth.small("small_ragged", 101, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                                lengths=("uniform", 200, 384)),
    "small_g5": synth.small("small_g5", 102, num_layers=1, batch=1, num_kv_heads=3, group=5, budget=300, buffer=100),
    "small_a6": synth.small("small_a6", 105, num_layers=1, batch=2, num_kv_heads=2, group=3, budget=192, buffer=64,
                            obs_window=6),
    "small_g8": synth.small("small_g8", 121, num_layers=1, batch=2, num_kv_heads=1, group=8, budget=128, buffer=64),
    "small_a64": synth.small("small_a64", 107, num_layers=1, batch=1, num_kv_heads=2, group=1, budget=320, buffer=50,
                             obs_window=64),
    "single_f32": synth.WORKLOADS["single_f32"],
    "small_long": synth.small("small_long", 108, num_layers=1, batch=1, num_kv_heads=2, group=4, budget=5600),
    # the largest capacity (16384 slots); group 2 keeps the weights at 128 KiB of LDS
    "max_capacity_g2": synth.small("max_capacity_g2", 123, num_layers=1, batch=1, num_kv_heads=1, group=2,
                                   budget=16384 - 128),
    "llama8b_b1": synth.WORKLOADS["llama8b_b1"],
    # 8192 slices of at most 1152 slots: the 256-thread work-groups
    "llama8b_b32_ragged": synth.WORKLOADS["llama8b_b32_ragged"],
}
SAMPLED = {"llama8b_b1": [(0, 0, 0), (7, 0, 5), (19, 0, 2), (31, 0, 7)],
           "llama8b_b32_ragged": [(0, 0, 0), (5, 17, 3), (12, 3, 1), (31, 31, 7), (20, 9, 4)]}


def slices_of(w, name):
    return SAMPLED.get(name) or [(l, b, h) for l in range(w.num_layers) for b in range(w.batch)
                                 for h in range(w.num_kv_heads)]


def step_query(cs, t):
    """The decode queries of window step t, [L][b][Hq][D]."""
    return np.ascontiguousarray(cs.Q[:, :, :, t, :])


def run_decode(dc, q_host, n_slots, acc=None):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = dc.w
    out = torch.full((w.num_layers, w.batch, w.num_kv_heads * w.group, 128), -7.0, dtype=torch.float32, device=dev)
    rkv.rkv_decode_attention(_gpu.params_of(w), dc.k_layers(), dc.v_layers(), _gpu.to_dev(q_host), dc.seq_start,
                             n_slots, out, acc)
    return out


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_decode_attention_parity(name):
    torch, dev = _gpu.torch_dev()
    w = WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    dc = _gpu.DevCache.of(cs)
    q = step_query(cs, w.obs_window - 1)
    out = run_decode(dc, q, cs.n_slots)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G, worst = w.group, 0.0
    for (l, b, h) in slices_of(w, name):
        s0 = int(cs.seq_start[b])
        ref, _ = oracle.decode_attention(cs.K[l, b, h, s0:cs.n_slots], cs.V[l, b, h, s0:cs.n_slots],
                                         q[l, b, h * G:(h + 1) * G])
        err = np.max(np.abs(out[l, b, h * G:(h + 1) * G] - ref))
        worst = max(worst, float(err))
        assert err <= OUT_TOL, f"{name} {(l, b, h)}: output error {err:.3e}"
    print(f"{name}: worst output error {worst:.2e}")


def test_decode_attention_edges():
    """A sequence with no valid slot gets output 0 and leaves the accumulator
    alone; one whose only valid slot is the newest gets that slot's value
    exactly, with weight exactly 1."""
    torch, dev = _gpu.torch_dev()
    w = WORKLOADS["small_ragged"]
    cs = synth.build_cache(w, seed=0)
    dc = _gpu.DevCache.of(cs)
    n = cs.n_slots
    dc.seq_start[0] = n
    dc.seq_start[1] = n - 1
    acc = torch.zeros((w.num_layers, w.batch, w.num_kv_heads, w.group, w.capacity), dtype=torch.float32, device=dev)
    q = step_query(cs, 0)
    out = run_decode(dc, q, n, acc)
    torch.cuda.synchronize()
    out, acc = out.cpu().numpy(), acc.cpu().numpy()
    V = cs.V.view(np.uint16).astype(np.uint32) << 16
    V = V.view(np.float32)
    assert np.all(out[:, 0] == 0) and np.all(acc[:, 0] == 0)
    for l in range(w.num_layers):
        for h in range(w.num_kv_heads):
            for g in range(w.group):
                assert np.array_equal(out[l, 1, h * w.group + g], V[l, 1, h, n - 1])
            assert np.all(acc[l, 1, h, :, n - 1] == 1.0) and np.all(acc[l, 1, h, :, :n - 1] == 0)


def capture(dc, cs, acc):
    """The alpha window steps: the token at slot n_slots - alpha + t attends
    the slots up to itself, and its weights are added into acc."""
    w = cs.w
    for t in range(w.obs_window):
        run_decode(dc, step_query(cs, t), cs.n_slots - w.obs_window + 1 + t, acc)


@pytest.mark.parametrize("name", [n for n in WORKLOADS if n != "small_long"])
def test_captured_importance(name):
    torch, dev = _gpu.torch_dev()
    w = WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    dc = _gpu.DevCache.of(cs)
    acc = torch.zeros((w.num_layers, w.batch, w.num_kv_heads, w.group, w.capacity), dtype=torch.float32, device=dev)
    capture(dc, cs, acc)
    torch.cuda.synchronize()
    imp = (acc.amax(dim=3) / w.obs_window).cpu().numpy()  # [L][b][H][capacity]
    accn = acc.cpu().numpy()
    k3_imp, _, _ = _gpu.gpu_score(dc)
    for l in range(w.num_layers):
        for b in range(w.batch):
            s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
            assert np.all(accn[l, b, :, :, :s0] == 0) and np.all(accn[l, b, :, :, cs.n_slots:] == 0)
            if N <= w.budget:
                continue
            for h in range(w.num_kv_heads):
                s = _gpu.slice_index(w, l, b, h)
                mine, k3 = imp[l, b, h, s0:cs.n_slots], k3_imp[s, s0:cs.n_slots]
                rel = np.abs(mine - k3) / np.maximum(np.abs(k3), 1e-30)
                assert np.all(rel <= 2 * _gpu.REL_TOL), f"{name} {(l, b, h)} vs scoring kernel: worst {rel.max():.2e}"
    for (l, b, h) in slices_of(w, name):
        s0 = int(cs.seq_start[b])
        if int(cs.lengths[b]) <= w.budget:
            continue
        ref = _gpu.oracle_slice(cs, l, b, h)
        mine = imp[l, b, h, s0:cs.n_slots]
        rel = np.abs(mine - ref.importance) / np.maximum(np.abs(ref.importance), 1e-30)
        assert np.all(rel <= _gpu.REL_TOL), f"{name} {(l, b, h)}: captured importance worst rel {rel.max():.2e}"


@pytest.mark.parametrize("name", ["small_ragged", "small_a6", "single_f32", "llama8b_b1"])
def test_evict_step_captured(name):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    w = WORKLOADS[name]
    cs = synth.build_cache(w, seed=0)
    dc = _gpu.DevCache.of(cs)
    acc = torch.zeros((w.num_layers, w.batch, w.num_kv_heads, w.group, w.capacity), dtype=torch.float32, device=dev)
    capture(dc, cs, acc)
    p = _gpu.params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    koff = rkv.rkv_workspace_keep_offset(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step_captured(p, dc.k_layers(), dc.v_layers(), acc, dc.seq_start, cs.n_slots, ws, wsb)
    torch.cuda.synchronize()
    assert ns == w.budget
    keep = ws[koff:koff + w.slices * w.budget * 4].view(torch.int32).cpu().numpy().reshape(w.slices, w.budget)
    K1, V1 = _gpu.to_host(dc.K, cs.K.dtype), _gpu.to_host(dc.V, cs.V.dtype)
    s_new = dc.seq_start.cpu().numpy()
    ndiff = 0
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
    for (l, b, h) in slices_of(w, name):
        s = _gpu.slice_index(w, l, b, h)
        s0, N = int(cs.seq_start[b]), int(cs.lengths[b])
        ref = _gpu.oracle_slice(cs, l, b, h)
        ndiff += _gpu.check_keep(_gpu.keep_rel_of(keep[s], s0), ref, w, N, what=f"{name} {(l, b, h)}")
    print(f"{name}: kept-set differences inside the band: {ndiff}")
