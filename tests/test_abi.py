"""The C-ABI library without a GPU: it loads, exports every entry point that
include/rkv.h declares, and rejects bad arguments on the host before any
launch (so no call here touches device memory)."""
import ctypes
import os
import re

import pytest

import redundancy_aware_compression_amd as rkv
from redundancy_aware_compression_amd._binding import load_hip_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")

# Fake device pointers: never dereferenced, because every call below fails
# validation or takes a documented no-launch path.
FAKE = 0x10000
FAKE_WS = 0x100000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["rkv_workspace_bytes", "rkv_score", "rkv_select", "rkv_compact", "rkv_evict_step",
              "rkv_status_string", "rkv_last_hip_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = load_hip_library(rkv.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"librkv.so does not export {name}"


def P(**kw):
    base = dict(num_layers=2, batch=2, num_kv_heads=2, group=4, capacity=384, budget=256)
    base.update(kw)
    return rkv.make_params(**base)


def layers(n=2, ptr=FAKE):
    return [ptr + 4096 * i for i in range(n)]


def test_status_strings():
    for code, name in rkv.STATUS.items():
        assert rkv.rkv_status_string(code) == name
    assert rkv.rkv_last_hip_error() == 0


def test_workspace_bytes():
    p = P()
    n = rkv.rkv_workspace_bytes(p)
    slices = 2 * 2 * 2
    # row means, counts and importance per slot, kept slots per budget entry
    assert n >= slices * 384 * 4 * 3 + slices * 256 * 4
    assert n % 256 == 0
    assert rkv.rkv_workspace_bytes(P(budget=8, obs_window=8)) == 0
    assert rkv.rkv_workspace_bytes(P(capacity=100)) == 0


def test_workspace_keep_offset():
    """The keep lists sit inside the workspace, 256-byte aligned, with room
    for [slices][budget] int32 entries; invalid params are rejected."""
    for kw in [dict(), dict(budget=300, capacity=500), dict(num_layers=3, batch=5)]:
        p = P(**kw)
        off, n = rkv.rkv_workspace_keep_offset(p), rkv.rkv_workspace_bytes(p)
        slices = p.num_layers * p.batch * p.num_kv_heads
        assert off % 256 == 0 and off + slices * p.budget * 4 <= n
        # it follows the three per-slot score regions
        assert off >= slices * p.capacity * 4 * 3
    with pytest.raises(rkv.RkvError):
        rkv.rkv_workspace_keep_offset(P(capacity=100))


BAD_PARAMS = [
    (dict(lam=1.5), "RKV_ERR_BAD_PARAM"),
    (dict(lam=-0.1), "RKV_ERR_BAD_PARAM"),
    (dict(lam=float("nan")), "RKV_ERR_BAD_PARAM"),
    (dict(tau=1.5), "RKV_ERR_BAD_PARAM"),
    (dict(beta=-1), "RKV_ERR_BAD_PARAM"),
    (dict(dtype=7), "RKV_ERR_BAD_PARAM"),
    (dict(num_layers=0), "RKV_ERR_BAD_SHAPE"),
    (dict(num_layers=129), "RKV_ERR_BAD_SHAPE"),
    (dict(batch=0), "RKV_ERR_BAD_SHAPE"),
    (dict(num_kv_heads=0), "RKV_ERR_BAD_SHAPE"),
    (dict(group=0), "RKV_ERR_BAD_SHAPE"),
    (dict(obs_window=0), "RKV_ERR_BAD_SHAPE"),
    (dict(budget=8), "RKV_ERR_BAD_SHAPE"),  # budget must exceed the window
    (dict(buffer=0), "RKV_ERR_BAD_SHAPE"),
    (dict(capacity=383), "RKV_ERR_BAD_SHAPE"),  # < budget + buffer
    (dict(head_dim=64), "RKV_ERR_UNSUPPORTED"),
    (dict(capacity=20000), "RKV_ERR_UNSUPPORTED"),
    (dict(group=9), "RKV_ERR_UNSUPPORTED"),  # 9 * 8 query rows > 64
]


@pytest.mark.parametrize("kw,expect", BAD_PARAMS, ids=[str(b[0]) for b in BAD_PARAMS])
def test_bad_params_rejected_by_every_entry_point(kw, expect):
    p = P(**kw)
    code = [k for k, v in rkv.STATUS.items() if v == expect][0]
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, 300, FAKE, FAKE, None, FAKE_WS, 1 << 40, stream=0,
                         check=False) == code
    assert rkv.rkv_select(p, FAKE, FAKE, FAKE, 300, FAKE, stream=0, check=False) == code
    assert rkv.rkv_compact(p, layers(), layers(), FAKE, FAKE, 300, stream=0, check=False) == code
    st, ns = rkv.rkv_evict_step(p, layers(), layers(), FAKE, FAKE, 384, FAKE_WS, 1 << 40, stream=0, check=False)
    assert st == code and ns == 384
    st, ns = rkv.rkv_evict_step_holefill(p, layers(), layers(), FAKE, FAKE, FAKE, 384, FAKE_WS, 1 << 40, stream=0,
                                         check=False)
    assert st == code and ns == 384
    assert rkv.rkv_compact_holefill(p, layers(), layers(), FAKE, FAKE, FAKE, 300, stream=0, check=False) == code
    assert rkv.rkv_decode_attention(p, layers(), layers(), FAKE, FAKE, 300, FAKE, None, stream=0, check=False) == code
    st, ns = rkv.rkv_evict_step_captured(p, layers(), layers(), FAKE, FAKE, 384, FAKE_WS, 1 << 40, stream=0,
                                         check=False)
    assert st == code and ns == 384


def test_sampled_argument_errors():
    """The sampled selection: keep_newest, top_k and temperature ranges, NULL
    inputs, and the step's no-op below the trigger."""
    p = P()
    need = rkv.rkv_workspace_bytes(p)
    BADP, NULL = st_of("RKV_ERR_BAD_PARAM"), st_of("RKV_ERR_NULL_ARG")
    for kn, tk, temp in ((-1, 10, 1.0), (256, 10, 1.0), (8, -1, 1.0), (8, 10, 0.0), (8, 10, float("inf")),
                         (8, 10, float("nan"))):
        assert rkv.rkv_select_sampled(p, FAKE, FAKE, FAKE, 300, kn, tk, temp, FAKE, stream=0, check=False) == BADP
        st, _ = rkv.rkv_evict_step_sampled(p, layers(), layers(), FAKE, FAKE, FAKE, 384, kn, tk, temp, FAKE_WS, need,
                                           stream=0, check=False)
        assert st == BADP
    assert rkv.rkv_select_sampled(p, 0, FAKE, FAKE, 300, 8, 10, 1.0, FAKE, stream=0, check=False) == NULL
    assert rkv.rkv_select_sampled(p, FAKE, 0, FAKE, 300, 8, 10, 1.0, FAKE, stream=0, check=False) == NULL
    assert rkv.rkv_select_sampled(p, FAKE, FAKE, FAKE, 255, 8, 10, 1.0, FAKE, stream=0,
                                  check=False) == st_of("RKV_ERR_BAD_SHAPE")
    for ns in (0, 255, 383):
        st, out = rkv.rkv_evict_step_sampled(p, layers(), layers(), FAKE, FAKE, FAKE, ns, 8, 10, 1.0, FAKE_WS, need,
                                             stream=0, check=False)
        assert st == 0 and out == ns


def test_sentence_argument_errors():
    p = P()
    need = rkv.rkv_workspace_bytes(p)
    NULL, MIS, SHAPE, BADP = (st_of(x) for x in ("RKV_ERR_NULL_ARG", "RKV_ERR_MISALIGNED", "RKV_ERR_BAD_SHAPE",
                                                   "RKV_ERR_BAD_PARAM"))
    assert rkv.rkv_sentence_penalty(p, 0, FAKE, 16, 64, 0.8, FAKE, stream=0, check=False) == NULL
    assert rkv.rkv_sentence_penalty(p, FAKE + 8, FAKE, 16, 64, 0.8, FAKE, stream=0, check=False) == MIS
    for s_max, dim in ((0, 64), (16, 2), (16, 66), (16, 8196)):
        assert rkv.rkv_sentence_penalty(p, FAKE, FAKE, s_max, dim, 0.8, FAKE, stream=0, check=False) == SHAPE
    assert rkv.rkv_sentence_penalty(p, FAKE, FAKE, 16, 64, 1.5, FAKE, stream=0, check=False) == BADP
    st, _ = rkv.rkv_evict_step_sentences(p, layers(), layers(), FAKE, FAKE, 384, 0, FAKE, FAKE, 16, 64, 0.8, FAKE,
                                         FAKE_WS, need, stream=0, check=False)
    assert st == NULL
    st, _ = rkv.rkv_evict_step_sentences(p, layers(), layers(), FAKE, FAKE, 384, FAKE + 2, FAKE, FAKE, 16, 64, 0.8,
                                         FAKE, FAKE_WS, need, stream=0, check=False)
    assert st == MIS
    for ns in (0, 383):  # below the trigger: nothing launched
        st, out = rkv.rkv_evict_step_sentences(p, layers(), layers(), FAKE, FAKE, ns, FAKE, FAKE, FAKE, 16, 64, 0.8,
                                               FAKE, FAKE_WS, need, stream=0, check=False)
        assert st == 0 and out == ns


def test_decode_argument_errors():
    """Decode attention and the captured step: NULL and misaligned pointers,
    the slot range, the group and LDS limits (nothing launched), and the
    captured step's no-op below the trigger."""
    p = P()
    need = rkv.rkv_workspace_bytes(p)
    NULL, MIS, SHAPE, UNS = (st_of(x) for x in ("RKV_ERR_NULL_ARG", "RKV_ERR_MISALIGNED", "RKV_ERR_BAD_SHAPE",
                                                "RKV_ERR_UNSUPPORTED"))
    dec = rkv.rkv_decode_attention
    assert dec(p, layers(), layers(), 0, FAKE, 300, FAKE, None, stream=0, check=False) == NULL
    assert dec(p, layers(), layers(), FAKE, 0, 300, FAKE, None, stream=0, check=False) == NULL
    assert dec(p, layers(), layers(), FAKE, FAKE, 300, 0, None, stream=0, check=False) == NULL
    assert dec(p, layers(), [FAKE, 0], FAKE, FAKE, 300, FAKE, None, stream=0, check=False) == NULL
    assert dec(p, layers(), layers(), FAKE + 4, FAKE, 300, FAKE, None, stream=0, check=False) == MIS
    assert dec(p, layers(), layers(), FAKE, FAKE, 300, FAKE + 2, None, stream=0, check=False) == MIS
    assert dec(p, layers(), layers(), FAKE, FAKE, 300, FAKE, FAKE + 1, stream=0, check=False) == MIS
    for ns in (0, -1, 385):
        assert dec(p, layers(), layers(), FAKE, FAKE, ns, FAKE, None, stream=0, check=False) == SHAPE
    # more than 8 query heads per KV head (with a 1-token window, so the params are valid)
    assert dec(P(group=16, obs_window=1, budget=256), layers(), layers(), FAKE, FAKE, 300, FAKE, None, stream=0,
               check=False) == UNS
    # the weights of 8 heads over 6000 slots (192 KB) exceed the work-group's LDS
    big = P(group=8, capacity=8000, budget=7000)
    assert dec(big, layers(), layers(), FAKE, FAKE, 6000, FAKE, None, stream=0, check=False) == UNS
    st, _ = rkv.rkv_evict_step_captured(p, layers(), layers(), 0, FAKE, 384, FAKE_WS, need, stream=0, check=False)
    assert st == NULL
    st, _ = rkv.rkv_evict_step_captured(p, layers(), layers(), FAKE + 2, FAKE, 384, FAKE_WS, need, stream=0,
                                        check=False)
    assert st == MIS
    for ns in (0, 383):  # below the trigger: nothing launched
        st, out = rkv.rkv_evict_step_captured(p, layers(), layers(), FAKE, FAKE, ns, FAKE_WS, need, stream=0,
                                              check=False)
        assert st == 0 and out == ns


def test_holefill_argument_errors():
    """The hole-filling entry points: NULL or misaligned order, slot range,
    and the no-op below the trigger (nothing launched, fake pointers untouched)."""
    p = P()
    need = rkv.rkv_workspace_bytes(p)
    NULL, MIS, SHAPE = st_of("RKV_ERR_NULL_ARG"), st_of("RKV_ERR_MISALIGNED"), st_of("RKV_ERR_BAD_SHAPE")
    st, _ = rkv.rkv_evict_step_holefill(p, layers(), layers(), FAKE, FAKE, 0, 384, FAKE_WS, need, stream=0,
                                        check=False)
    assert st == NULL
    st, _ = rkv.rkv_evict_step_holefill(p, layers(), layers(), FAKE, FAKE, FAKE + 2, 384, FAKE_WS, need, stream=0,
                                        check=False)
    assert st == MIS
    assert rkv.rkv_compact_holefill(p, layers(), layers(), FAKE, FAKE, 0, 300, stream=0, check=False) == NULL
    assert rkv.rkv_compact_holefill(p, layers(), layers(), FAKE, FAKE, FAKE + 1, 300, stream=0, check=False) == MIS
    assert rkv.rkv_compact_holefill(p, layers(), layers(), FAKE, FAKE, FAKE, 255, stream=0, check=False) == SHAPE
    big = P(budget=12000, capacity=12200)
    st, _ = rkv.rkv_evict_step_holefill(big, layers(), layers(), FAKE, FAKE, FAKE, 12200, FAKE_WS, 1 << 40,
                                        stream=0, check=False)
    assert st == st_of("RKV_ERR_UNSUPPORTED")
    for ns in (0, 255, 383):
        st, out = rkv.rkv_evict_step_holefill(p, layers(), layers(), FAKE, FAKE, FAKE, ns, FAKE_WS, need, stream=0,
                                              check=False)
        assert st == 0 and out == ns


def st_of(name):
    return [k for k, v in rkv.STATUS.items() if v == name][0]


def test_null_and_alignment_errors():
    p = P()
    big = 1 << 40
    NULL, MIS = st_of("RKV_ERR_NULL_ARG"), st_of("RKV_ERR_MISALIGNED")
    assert rkv.rkv_score(p, [FAKE, 0], FAKE, FAKE, 300, FAKE, FAKE, None, FAKE_WS, big, stream=0, check=False) == NULL
    assert rkv.rkv_score(p, layers(), 0, FAKE, 300, FAKE, FAKE, None, FAKE_WS, big, stream=0, check=False) == NULL
    assert rkv.rkv_score(p, layers(), FAKE, 0, 300, FAKE, FAKE, None, FAKE_WS, big, stream=0, check=False) == NULL
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, 300, 0, FAKE, None, FAKE_WS, big, stream=0, check=False) == NULL
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, 300, FAKE, FAKE, None, 0, big, stream=0, check=False) == NULL
    assert rkv.rkv_score(p, [FAKE + 8, FAKE], FAKE, FAKE, 300, FAKE, FAKE, None, FAKE_WS, big, stream=0,
                         check=False) == MIS
    assert rkv.rkv_score(p, layers(), FAKE + 4, FAKE, 300, FAKE, FAKE, None, FAKE_WS, big, stream=0,
                         check=False) == MIS
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, 300, FAKE, FAKE, None, FAKE_WS + 16, big, stream=0,
                         check=False) == MIS
    assert rkv.rkv_select(p, 0, FAKE, FAKE, 300, FAKE, stream=0, check=False) == NULL
    assert rkv.rkv_select(p, FAKE, FAKE, FAKE, 300, 0, stream=0, check=False) == NULL
    assert rkv.rkv_compact(p, layers(), [0, FAKE], FAKE, FAKE, 300, stream=0, check=False) == NULL
    assert rkv.rkv_compact(p, layers(), layers(), 0, FAKE, 300, stream=0, check=False) == NULL
    assert rkv.rkv_compact(p, layers(), [FAKE, FAKE + 2], FAKE, FAKE, 300, stream=0, check=False) == MIS
    st, _ = rkv.rkv_evict_step(p, layers(), layers(), FAKE, 0, 384, FAKE_WS, big, stream=0, check=False)
    assert st == NULL
    st, _ = rkv.rkv_evict_step(p, layers(), layers(), FAKE, FAKE, 384, 0, big, stream=0, check=False)
    assert st == NULL


def test_slot_range_and_workspace_errors():
    p = P()
    SHAPE, WS = st_of("RKV_ERR_BAD_SHAPE"), st_of("RKV_ERR_WORKSPACE_TOO_SMALL")
    need = rkv.rkv_workspace_bytes(p)
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, 385, FAKE, FAKE, None, FAKE_WS, need, stream=0,
                         check=False) == SHAPE
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, -1, FAKE, FAKE, None, FAKE_WS, need, stream=0,
                         check=False) == SHAPE
    assert rkv.rkv_score(p, layers(), FAKE, FAKE, 300, FAKE, FAKE, None, FAKE_WS, need - 1, stream=0,
                         check=False) == WS
    assert rkv.rkv_select(p, FAKE, FAKE, FAKE, 255, FAKE, stream=0, check=False) == SHAPE  # below budget
    assert rkv.rkv_select(p, FAKE, FAKE, FAKE, 385, FAKE, stream=0, check=False) == SHAPE
    assert rkv.rkv_compact(p, layers(), layers(), FAKE, FAKE, 255, stream=0, check=False) == SHAPE
    st, ns = rkv.rkv_evict_step(p, layers(), layers(), FAKE, FAKE, 385, FAKE_WS, need, stream=0, check=False)
    assert st == SHAPE and ns == 385
    st, ns = rkv.rkv_evict_step(p, layers(), layers(), FAKE, FAKE, 384, FAKE_WS, need - 256, stream=0, check=False)
    assert st == WS and ns == 384


def test_no_launch_paths_return_ok():
    """Below the trigger the step launches nothing; scoring with n_slots <= budget
    has nothing to score. Both succeed without touching the fake pointers."""
    p = P()
    need = rkv.rkv_workspace_bytes(p)
    for ns in (0, 1, 255, 256, 383):
        st, out = rkv.rkv_evict_step(p, layers(), layers(), FAKE, FAKE, ns, FAKE_WS, need, stream=0, check=False)
        assert st == 0 and out == ns
    for ns in (0, 100, 256):
        assert rkv.rkv_score(p, layers(), FAKE, FAKE, ns, FAKE, FAKE, None, FAKE_WS, need, stream=0,
                             check=False) == 0


def test_python_raises_on_error():
    with pytest.raises(rkv.RkvError, match="RKV_ERR_BAD_PARAM"):
        rkv.rkv_select(P(lam=2.0), FAKE, FAKE, FAKE, 300, FAKE, stream=0)


def test_peaks_library_exports_its_header():
    """librkv_peaks.so (the peak microbenchmarks) exports what include/rkv_peaks.h
    declares; its argument checks run on the host (nothing is launched)."""
    from redundancy_aware_compression_amd import build as rkv_build

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "rkv_peaks.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(rkv_peak_[a-z_0-9]+)\s*\(", text)))
    assert {"rkv_peak_mfma_bf16", "rkv_peak_mfma_bf16_random", "rkv_peak_hbm_read", "rkv_peak_hbm_copy"} <= set(names)
    lib = load_hip_library(rkv_build.PEAKS_LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    lib.rkv_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.rkv_peak_hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                      ctypes.c_void_p]
    lib.rkv_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.rkv_peak_hbm_read(FAKE, 100, 4, FAKE, None) != 0  # not a multiple of 16
    assert lib.rkv_peak_hbm_copy(FAKE + 8, FAKE, 4096, 4, None) != 0  # misaligned
    assert lib.rkv_peak_mfma_bf16(0, 10, FAKE, None) != 0  # no work-groups
    lib.rkv_peak_mfma_bf16_random.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.rkv_peak_mfma_bf16_random(4, 0, FAKE, None) != 0  # no rounds
    assert lib.rkv_peak_threads_per_block() == 256


def test_binding_checks_layer_lists():
    """The binding refuses a per-layer pointer list whose length is not
    num_layers (the library would read past it) and tensors that are not
    exactly one contiguous layer of the cache's element type; nothing is
    called in either case."""
    import torch

    p = P()
    with pytest.raises(ValueError):
        rkv.rkv_compact(p, layers(1), layers(), FAKE, FAKE, 300, stream=0)
    with pytest.raises(ValueError):
        rkv.rkv_evict_step(p, layers(), layers(3), FAKE, FAKE, 384, FAKE_WS, 1 << 40, stream=0)
    one = p.batch * p.num_kv_heads * p.capacity * p.head_dim
    good = [torch.empty(one, dtype=torch.bfloat16) for _ in range(2)]
    for bad in ([torch.empty(one - 1, dtype=torch.bfloat16)] * 2, [torch.empty(one, dtype=torch.float32)] * 2,
                [torch.empty(2 * one, dtype=torch.bfloat16)[::2]] * 2):
        with pytest.raises(ValueError):
            rkv.rkv_score(p, bad, FAKE, FAKE, 300, FAKE, FAKE, None, FAKE_WS, 1 << 40, stream=0)
    # the right tensors pass the binding; the library then rejects the NULL queries
    assert rkv.rkv_score(p, good, 0, FAKE, 300, FAKE, FAKE, None, FAKE_WS, 1 << 40, stream=0,
                         check=False) == st_of("RKV_ERR_NULL_ARG")


def test_noalloc_limits_and_noop():
    """The allocation-free step rejects parameters whose workspace exceeds its
    built-in array, and takes the no-op path below the trigger, both before
    touching any device."""
    big = P(num_layers=32, batch=32, num_kv_heads=8, capacity=1152, budget=1024)
    assert rkv.rkv_workspace_bytes(big) > rkv.RKV_NOALLOC_WORKSPACE_BYTES
    st, ns = rkv.rkv_evict_step_noalloc(big, layers(32), layers(32), FAKE, FAKE, 1152, stream=0, check=False)
    assert st == st_of("RKV_ERR_WORKSPACE_TOO_SMALL") and ns == 1152
    p = P()
    assert rkv.rkv_workspace_bytes(p) <= rkv.RKV_NOALLOC_WORKSPACE_BYTES
    st, ns = rkv.rkv_evict_step_noalloc(p, layers(), layers(), FAKE, FAKE, 383, stream=0, check=False)
    assert st == 0 and ns == 383
    st, _ = rkv.rkv_evict_step_noalloc(p, layers(), layers(), 0, FAKE, 384, stream=0, check=False)
    assert st == st_of("RKV_ERR_NULL_ARG")
    st, _ = rkv.rkv_evict_step_noalloc(p, layers(), layers(), FAKE + 4, FAKE, 384, stream=0, check=False)
    assert st == st_of("RKV_ERR_MISALIGNED")


def test_one_hip_runtime_whatever_the_import_order():
    """Loading librkv before torch is imported must not map a second HIP
    runtime beside the one torch brings (librkv's launches would then go
    through a runtime that cannot use the device torch has opened)."""
    import subprocess
    import sys
    import textwrap

    code = textwrap.dedent('''
        import redundancy_aware_compression_amd as rkv
        rkv.rkv_workspace_bytes(rkv.make_params(2, 2, 2, 4, 384, 256))  # loads librkv
        import torch
        from redundancy_aware_compression_amd._binding import hip_runtimes_mapped
        m = hip_runtimes_mapped()
        assert len(m) == 1, m
        print("one runtime:", m.pop())
    ''')
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
