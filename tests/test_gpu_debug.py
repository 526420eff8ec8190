"""RKV_DEBUG: the device precondition checks (include/rkv.h, Debug checks).
Clean inputs pass and give the same bits as a step without the checks; each
violated precondition (a non-finite key, value or query element in a valid
slot, a seq_start past n_slots, an order table that is not a permutation)
returns RKV_ERR_PRECONDITION with the cache, the start slots and n_slots
untouched. The violations are planted in the inputs only: every kernel reads
within its buffers (seq_start is clamped, order entries are range-checked),
so nothing here can fault."""
import numpy as np
import pytest
import torch

import _gpu
import synth

pytestmark = pytest.mark.gpu

W = synth.small("debug_ragged", 130, num_layers=2, batch=3, num_kv_heads=2, group=4, budget=256,
                lengths=("uniform", 200, 384))
BF16_NAN = 0x7FC0


def _step(dc, cs, check=False):
    import redundancy_aware_compression_amd as rkv

    _, dev = _gpu.torch_dev()
    p = _gpu.params_of(cs.w)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step(p, dc.k_layers(), dc.v_layers(), dc.Q, dc.seq_start, cs.n_slots, ws, wsb,
                                check=check)
    torch.cuda.synchronize()
    return st, ns


def _code(name):
    import redundancy_aware_compression_amd as rkv

    return [k for k, v in rkv.STATUS.items() if v == name][0]


def _snapshot(dc, cs):
    return (_gpu.to_host(dc.K, cs.K.dtype).copy(), _gpu.to_host(dc.V, cs.V.dtype).copy(), dc.seq_start.cpu().numpy())


def _unchanged(dc, cs, snap):
    K, V, S = snap
    assert np.array_equal(_gpu.to_host(dc.K, cs.K.dtype).view(np.uint8), K.view(np.uint8))
    assert np.array_equal(_gpu.to_host(dc.V, cs.V.dtype).view(np.uint8), V.view(np.uint8))
    assert np.array_equal(dc.seq_start.cpu().numpy(), S)


def _bf16_nan_at(t, index):
    flat = t.view(-1)
    flat[np.ravel_multi_index(index, tuple(t.shape))] = BF16_NAN - 65536 if BF16_NAN > 32767 else BF16_NAN


def test_clean_inputs_pass_and_match(monkeypatch):
    cs = synth.build_cache(W, seed=0)
    plain = _gpu.DevCache.of(cs)
    monkeypatch.delenv("RKV_DEBUG", raising=False)
    assert _step(plain, cs) == (0, W.budget)
    checked = _gpu.DevCache.of(cs)
    monkeypatch.setenv("RKV_DEBUG", "1")
    assert _step(checked, cs) == (0, W.budget)
    for a, b in ((plain.K, checked.K), (plain.V, checked.V), (plain.seq_start, checked.seq_start)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("what", ["key", "value", "query"])
def test_non_finite_element_is_caught(monkeypatch, what):
    cs = synth.build_cache(W, seed=0)
    dc = _gpu.DevCache.of(cs)
    b = int(np.argmax(cs.lengths))  # an evicting sequence
    s0 = int(cs.seq_start[b])
    if what == "key":
        _bf16_nan_at(dc.K, (1, b, 1, s0 + 7, 33))
    elif what == "value":
        _bf16_nan_at(dc.V, (0, b, 0, cs.n_slots - 1, 127))
    else:
        _bf16_nan_at(dc.Q, (1, b, 5, 2, 64))
    snap = _snapshot(dc, cs)
    monkeypatch.setenv("RKV_DEBUG", "1")
    st, ns = _step(dc, cs)
    assert st == _code("RKV_ERR_PRECONDITION") and ns == cs.n_slots
    _unchanged(dc, cs, snap)


def test_padding_is_not_checked(monkeypatch):
    """NaN in the left padding and past n_slots is allowed: those slots are never read."""
    cs = synth.build_cache(W, seed=0)
    assert W.nan_padding
    dc = _gpu.DevCache.of(cs)
    b = int(np.argmin(cs.lengths))
    assert int(cs.seq_start[b]) > 0
    _bf16_nan_at(dc.K, (0, b, 0, 0, 0))
    monkeypatch.setenv("RKV_DEBUG", "1")
    assert _step(dc, cs) == (0, W.budget)


def test_seq_start_out_of_range_is_caught(monkeypatch):
    cs = synth.build_cache(W, seed=0)
    dc = _gpu.DevCache.of(cs)
    dc.seq_start[1] = cs.n_slots + 3
    snap = _snapshot(dc, cs)
    monkeypatch.setenv("RKV_DEBUG", "1")
    st, ns = _step(dc, cs)
    assert st == _code("RKV_ERR_PRECONDITION") and ns == cs.n_slots
    _unchanged(dc, cs, snap)


def test_score_checks_keys(monkeypatch):
    import redundancy_aware_compression_amd as rkv

    _, dev = _gpu.torch_dev()
    cs = synth.build_cache(W, seed=0)
    dc = _gpu.DevCache.of(cs)
    b = int(np.argmax(cs.lengths))
    _bf16_nan_at(dc.K, (0, b, 1, int(cs.seq_start[b]), 0))
    p = _gpu.params_of(W)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    n = cs.n_slots
    imp = torch.full((W.slices * n,), -5.0, dtype=torch.float32, device=dev)
    red = torch.full_like(imp, -5.0)
    monkeypatch.setenv("RKV_DEBUG", "1")
    st = rkv.rkv_score(p, dc.k_layers(), dc.Q, dc.seq_start, n, imp, red, None, ws, wsb, check=False)
    torch.cuda.synchronize()
    assert st == _code("RKV_ERR_PRECONDITION")
    assert bool((imp == -5.0).all()) and bool((red == -5.0).all())


def test_holefill_order_not_a_permutation_is_caught(monkeypatch):
    import redundancy_aware_compression_amd as rkv

    _, dev = _gpu.torch_dev()
    cs = synth.build_cache(W, seed=0)
    p = _gpu.params_of(W)
    wsb = rkv.rkv_workspace_bytes(p)
    order = np.tile(np.arange(W.budget, dtype=np.int32), (W.num_layers, W.batch, W.num_kv_heads, 1))
    Kd, Vd, Qd = _gpu.to_dev(cs.K), _gpu.to_dev(cs.V), _gpu.to_dev(cs.Q)
    Sd = torch.from_numpy(cs.seq_start.copy()).to(dev)
    monkeypatch.setenv("RKV_DEBUG", "1")
    for bad in ("duplicate", "range"):
        o = order.copy()
        if bad == "duplicate":
            o[1, 2, 0, 10] = o[1, 2, 0, 11]
        else:
            o[0, 0, 1, 3] = W.budget + 5
        Od = torch.from_numpy(o).to(dev)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        st, ns = rkv.rkv_evict_step_holefill(p, [Kd[l] for l in range(W.num_layers)],
                                             [Vd[l] for l in range(W.num_layers)], Qd, Sd, Od, cs.n_slots, ws, wsb,
                                             check=False)
        torch.cuda.synchronize()
        assert st == _code("RKV_ERR_PRECONDITION") and ns == cs.n_slots
        assert np.array_equal(Od.cpu().numpy(), o)
    # the identity order passes
    Od = torch.from_numpy(order).to(dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st, ns = rkv.rkv_evict_step_holefill(p, [Kd[l] for l in range(W.num_layers)],
                                         [Vd[l] for l in range(W.num_layers)], Qd, Sd, Od, cs.n_slots, ws, wsb,
                                         check=False)
    torch.cuda.synchronize()
    assert st == 0 and ns == W.budget
