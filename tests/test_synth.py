"""The seeded input generators (CPU): both the oracle and the GPU path are
fed from them, so their rounding, statistics, determinism and layout are
checked here against independent constructions rather than trusted."""
import math

import numpy as np
import pytest

import synth


def _rne_bf16_reference(f: np.ndarray) -> np.ndarray:
    """bf16 bits of float32 values by round-to-nearest-even, built from the
    two bf16 neighbours in float64 arithmetic (independent of the bit trick
    the generators use). Finite inputs only."""
    out = np.empty(f.shape, np.uint16)
    for i, x in enumerate(f.astype(np.float32)):
        u = int(np.float32(x).view(np.uint32))
        lo = u & 0xFFFF0000
        hi = lo + 0x10000  # next bf16 away from zero (may step into inf, which is what RNE gives there)
        vx = float(np.uint32(u).view(np.float32))
        vlo = float(np.uint32(lo).view(np.float32))
        vhi_bits = np.uint32(hi & 0xFFFFFFFF)
        vhi = float(vhi_bits.view(np.float32))
        if math.isinf(vhi):  # rounding past the largest finite value compares against 2^128
            vhi = math.copysign(2.0 ** 128, vhi)
        dlo, dhi = abs(vx - vlo), abs(vhi - vx)
        if dlo < dhi or (dlo == dhi and ((lo >> 16) & 1) == 0):
            out[i] = lo >> 16
        else:
            out[i] = (hi >> 16) & 0xFFFF
    return out


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(500) * 1e-39).astype(np.float32),  # subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, -3.0e38], np.float32),
        # exact ties: bit 15 set and the low 15 bits clear, with even and odd kept mantissas
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00018000], np.uint32).view(np.float32),
        # one below and one above a tie
        np.array([0x3F807FFF, 0x3F808001], np.uint32).view(np.float32),
        # the largest finite float rounds to infinity
        np.array([0x7F7FFFFF], np.uint32).view(np.float32),
    ])
    ref = _rne_bf16_reference(x)
    assert np.array_equal(synth.bf16_bits(x), ref)
    L = synth.lib()
    c = np.array([L.synth_bf16_from_f32(float(v)) for v in x], np.uint16)
    assert np.array_equal(c, ref)
    assert synth.bf16_bits(np.array([np.nan], np.float32))[0] == synth.BF16_NAN


def _normals(key, n, code=synth.F32):
    a = np.empty(n, np.float32 if code == synth.F32 else np.uint16)
    synth.lib().synth_fill_normal(key, 0.0, 1.0, code, a.ctypes.data, n)
    return a


def test_normal_moments_and_tails():
    x = _normals(synth.stream_key(0, 1, 0, 0, 0, 0), 400_000).astype(np.float64)
    assert abs(x.mean()) < 0.006
    assert abs(x.var() - 1.0) < 0.01
    assert abs(np.mean(x ** 3)) < 0.02  # symmetric
    assert abs(np.mean(x ** 4) - 3.0) < 0.06  # Gaussian kurtosis
    # two-sided tail mass beyond 2 and 3 standard deviations
    assert abs(np.mean(np.abs(x) > 2.0) - math.erfc(2 / math.sqrt(2))) < 0.002
    assert abs(np.mean(np.abs(x) > 3.0) - math.erfc(3 / math.sqrt(2))) < 0.0006
    # the bf16 stream is the fp32 stream rounded to nearest even
    key = synth.stream_key(3, 2, 1, 4, 5, 6)
    assert np.array_equal(_normals(key, 5000, synth.BF16), synth.bf16_bits(_normals(key, 5000)))


def test_uniforms_are_strictly_inside_the_unit_interval():
    n = 200_000
    u = np.empty(n, np.float32)
    synth.lib().synth_fill_uniform_open(synth.stream_key(0, 5, 6, 0, 0, 0), u.ctypes.data, n)
    assert u.min() > 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.003
    assert abs(u.var() - 1.0 / 12.0) < 0.002


def test_streams_are_deterministic_and_independent():
    k1 = synth.stream_key(0, 2, synth.T_KEYS, 3, 0, 5)
    assert k1 == synth.stream_key(0, 2, synth.T_KEYS, 3, 0, 5)
    keys = {synth.stream_key(s, wl, t, l, b, h) for s in (0, 1) for wl in (2, 3) for t in (0, 1)
            for l in (0, 1) for b in (0, 1) for h in (0, 1)}
    assert len(keys) == 64  # every coordinate changes the key
    a, b = _normals(k1, 20000), _normals(synth.stream_key(0, 2, synth.T_KEYS, 3, 0, 6), 20000)
    assert np.array_equal(a, _normals(k1, 20000))
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.03


def test_cache_layout_padding_canary_and_lengths():
    w = synth.small("synth_layout", 130, num_layers=2, batch=4, num_kv_heads=2, group=3, budget=192, buffer=64,
                    lengths=("uniform", 100, 256), extra_capacity=16)
    cs = synth.build_cache(w, seed=0)
    assert np.array_equal(cs.seq_start, w.n_slots - cs.lengths)
    assert np.all((cs.lengths >= 100) & (cs.lengths <= 256))
    again = synth.build_cache(w, seed=0)
    assert np.array_equal(cs.K, again.K) and np.array_equal(cs.V, again.V) and np.array_equal(cs.Q, again.Q)
    other = synth.build_cache(w, seed=1)
    assert not np.array_equal(cs.K, other.K)
    for b in range(w.batch):
        s0 = int(cs.seq_start[b])
        pad = cs.K[:, b, :, :s0]
        assert np.all(pad == synth.BF16_NAN)  # padding is NaN, so a masking leak cannot hide
        assert np.all(cs.K[:, b, :, w.n_slots:] == synth.BF16_CANARY)
        valid = synth.to_float(cs.K[:, b, :, s0:w.n_slots], "bf16")
        assert np.all(np.isfinite(valid))


def test_repeated_spans_are_noisy_copies_of_earlier_windows():
    """The key recipe: the stated number of 32-token spans are copies of an
    earlier window plus N(0, 0.05^2) noise, cosine about 1 / sqrt(1 + 0.05^2)
    with their source; other spans have no such partner."""
    w = synth.small("synth_spans", 131, num_layers=1, batch=1, num_kv_heads=1, group=1, budget=1024)
    cs = synth.build_cache(w, seed=0)
    K = synth.to_float(cs.K[0, 0, 0, : w.n_slots], "bf16")
    Kh = K / np.linalg.norm(K, axis=1, keepdims=True)
    S = Kh @ Kh.T
    L = w.span_len
    nsp = w.n_slots // L
    copies = 0
    for sp in range(1, nsp):
        blk = S[sp * L:(sp + 1) * L, : sp * L]
        # a copy: each row's best earlier partner is near 0.9988, and the partners form one window
        best = blk.max(axis=1)
        if np.all(best > 0.99):
            arg = blk.argmax(axis=1)
            assert np.all(np.diff(arg) == 1), "a copied span comes from one contiguous window"
            assert np.all(np.abs(best - 1 / math.sqrt(1 + w.noise_sigma ** 2)) < 0.01)
            copies += 1
        else:
            assert best.max() < 0.5  # independent Gaussian keys in 128 dims
    first, last, cnt = synth.n_copies_for(w, w.n_slots)
    assert copies == cnt


def test_sentences_cover_the_valid_slots():
    w = synth.small("synth_sent", 132, num_layers=2, batch=3, num_kv_heads=2, group=2, budget=256,
                    lengths=("uniform", 150, 384))
    cs = synth.build_cache(w, seed=0)
    se = synth.sentences(cs, dim=64, repeat_p=0.3, noise=0.2)
    for b in range(w.batch):
        s0 = int(cs.seq_start[b])
        ids = se.sent_id[0, b, 0]
        assert np.all(ids[:s0] == -1) and np.all(ids[w.n_slots:] == -1)
        run = ids[s0:w.n_slots]
        assert run[0] == 0 and np.all(np.diff(run) >= 0) and np.all(np.diff(run) <= 1)
        lens = np.bincount(run)
        assert np.all((lens[:-1] >= 8) & (lens[:-1] <= 40)) and 1 <= lens[-1] <= 40
        assert int(se.n_sent[b]) == len(lens)
        for l in range(w.num_layers):  # every layer and head carries the same map at generation time
            for h in range(w.num_kv_heads):
                assert np.array_equal(se.sent_id[l, b, h], ids)
        v = se.vectors[b, : se.n_sent[b]].astype(np.float64)
        vh = v / np.linalg.norm(v, axis=1, keepdims=True)
        c = vh @ vh.T
        np.fill_diagonal(c, 0)
        # repeats (noisy copies, sigma 0.2) sit near 1 / sqrt(1.04); unrelated vectors near 0
        high = c[c > 0.5]
        assert np.all(high > 0.9) and np.all(np.abs(c[c <= 0.5]) < 0.6)
