"""The allocation-free eviction step (rkv_evict_step_noalloc, its workspace
built into the library) against the step with a caller workspace
(rkv_evict_step): the same results, bit for bit, on two calls in a row on
one GPU, the second with a smaller input than the first (the built-in array
keeps the first call's contents)."""
import numpy as np
import pytest

import _gpu
import synth

pytestmark = pytest.mark.gpu

FIRST = synth.small("noalloc_first", 125, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                    lengths=("uniform", 200, 384))
SECOND = synth.small("noalloc_second", 126, num_layers=1, batch=1, num_kv_heads=2, group=5, budget=192, buffer=72)


def _run(w, seed):
    import redundancy_aware_compression_amd as rkv

    torch, dev = _gpu.torch_dev()
    cs = synth.build_cache(w, seed=seed)
    p = _gpu.params_of(w)
    assert rkv.rkv_workspace_bytes(p) <= rkv.RKV_NOALLOC_WORKSPACE_BYTES
    ref, new = _gpu.DevCache.of(cs), _gpu.DevCache.of(cs)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _, ns_ref = rkv.rkv_evict_step(p, ref.k_layers(), ref.v_layers(), ref.Q, ref.seq_start, cs.n_slots, ws, wsb)
    _, ns_new = rkv.rkv_evict_step_noalloc(p, new.k_layers(), new.v_layers(), new.Q, new.seq_start, cs.n_slots)
    torch.cuda.synchronize()
    assert ns_ref == ns_new == w.budget
    for a, b, what in ((ref.K, new.K, "K"), (ref.V, new.V, "V"), (ref.seq_start, new.seq_start, "seq_start")):
        assert np.array_equal(a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8)), what
    # and the result is the step's: the kept rows are the pre-step rows of the oracle-checked keep sets
    # (covered by the parity tests of rkv_evict_step); here the two entry points must agree exactly


def test_noalloc_matches_step_twice_second_smaller():
    import redundancy_aware_compression_amd as rkv

    assert rkv.rkv_workspace_bytes(_gpu.params_of(SECOND)) < rkv.rkv_workspace_bytes(_gpu.params_of(FIRST))
    _run(FIRST, 0)
    _run(SECOND, 1)
