"""Seeded synthetic workloads for the R-KV eviction step.

This package is the one module that both sides of every comparison use: the
CPU oracle under ``oracle/`` and the HIP library. It draws numbers, rounds
them to the storage type and lays them out; it holds none of the eviction
method's arithmetic. Its C half (``rkv_synth.c``) is built with gcc into
``librkv_synth.so`` next to this file.

Workloads stand in for the reasoning traces of DeepSeek-R1-Distill models
that the R-KV pages evaluate on (MATH-500 / AIME 2024 generations); those
traces, datasets and weights are not used. Repetition is injected as noisy
copies of earlier token spans, standing in for the repeated reasoning text
the R-KV page describes in its summary table (row "core observation").
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rkv_synth.c")
_LIB_PATH = os.path.join(_HERE, "librkv_synth.so")

BF16 = 0
F32 = 1

# tensor ids of the per-slice streams
T_KEYS, T_VALUES, T_QUERIES, T_LENGTHS, T_MIX = 0, 1, 2, 3, 4

BF16_NAN = 0x7FC0
BF16_CANARY = 0x7F81  # a signalling-NaN pattern no generator or copy produces


def build(force: bool = False) -> str:
    """Compiles rkv_synth.c with gcc (always when force, else when missing/stale)."""
    stale = (not os.path.exists(_LIB_PATH)) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        L.synth_stream_key.restype = u64
        L.synth_stream_key.argtypes = [u64, i64, i64, i64, i64, i64]
        L.synth_fill_normal.restype = None
        L.synth_fill_normal.argtypes = [u64, dbl, dbl, i32, vp, i64]
        L.synth_slice_keys.restype = i32
        L.synth_slice_keys.argtypes = [u64, i32, i32, i32, i32, i32, i32, dbl, i32, vp, vp]
        L.synth_mixture_means.restype = None
        L.synth_mixture_means.argtypes = [u64, i32, i32, dbl, vp]
        L.synth_mixture_drift.restype = None
        L.synth_mixture_drift.argtypes = [u64, i32, i32, dbl, vp]
        L.synth_mixture_tokens.restype = None
        L.synth_mixture_tokens.argtypes = [u64, i32, i32, i32, vp, i32, vp]
        L.synth_inject_repeats.restype = i32
        L.synth_inject_repeats.argtypes = [u64, i32, i32, i32, dbl, dbl, vp, i32, i32, vp]
        L.synth_bf16_from_f32.restype = ctypes.c_uint16
        L.synth_bf16_from_f32.argtypes = [ctypes.c_float]
        _lib = L
    return _lib


def stream_key(seed: int, workload: int, tensor: int, layer: int, seq: int, head: int) -> int:
    return lib().synth_stream_key(seed, workload, tensor, layer, seq, head)


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


@dataclass(frozen=True)
class Workload:
    """Shape, method parameters and input recipe of one eviction workload."""

    name: str
    wid: int  # workload id folded into every stream key
    num_layers: int
    batch: int
    num_kv_heads: int
    group: int
    head_dim: int
    budget: int
    buffer: int = 128
    obs_window: int = 8
    beta: int = 2
    lam: float = 0.1
    tau: float = 0.5
    dtype: str = "bf16"
    span_len: int = 32
    copy_frac: float = 0.3  # fraction of spans overwritten by copies (rounded)
    n_copies: Optional[int] = None  # fixed copy count instead of copy_frac
    spans_in_candidates: bool = False  # destination spans restricted to the candidate range
    noise_sigma: float = 0.05
    lengths: tuple = ("full",)  # ("full",) or ("uniform", lo, hi)
    nan_padding: bool = True
    extra_capacity: int = 0  # slots past budget+buffer (filled with a canary)

    @property
    def n_slots(self) -> int:
        return self.budget + self.buffer

    @property
    def capacity(self) -> int:
        return self.n_slots + self.extra_capacity

    @property
    def q_heads(self) -> int:
        return self.num_kv_heads * self.group

    @property
    def slices(self) -> int:
        return self.num_layers * self.batch * self.num_kv_heads

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    @property
    def code(self) -> int:
        return BF16 if self.dtype == "bf16" else F32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


# The workloads the eviction step is measured and checked on. Model shapes:
# Llama-8B-like GQA (32 layers, 8 KV heads, group 4, head_dim 128) and
# Qwen-14B-like GQA (48 layers, 8 KV heads, group 5). Budgets: R-KV's 10 %
# and fixed-1024 settings (R-KV page, summary table, row "throughput").
WORKLOADS = {
    "single_f32": Workload("single_f32", 1, 1, 1, 1, 1, 128, 256, dtype="f32", span_len=16, n_copies=4,
                           spans_in_candidates=True),
    "llama8b_b1": Workload("llama8b_b1", 2, 32, 1, 8, 4, 128, 1024),
    "llama8b_b32_ragged": Workload("llama8b_b32_ragged", 3, 32, 32, 8, 4, 128, 1024, lengths=("uniform", 600, 1152)),
    "qwen14b_b8": Workload("qwen14b_b8", 4, 48, 8, 8, 5, 128, 4096, copy_frac=0.4),
    "llama8b_b16_sweep10pct": Workload("llama8b_b16_sweep10pct", 5, 32, 16, 8, 4, 128, 1638),
    "llama8b_b16_sweep1024": Workload("llama8b_b16_sweep1024", 6, 32, 16, 8, 4, 128, 1024),
}


def small(name: str = "small", wid: int = 100, **kw) -> Workload:
    """A reduced workload for tests (same recipe, smaller shape)."""
    base = dict(num_layers=2, batch=1, num_kv_heads=2, group=4, head_dim=128, budget=256)
    base.update(kw)
    return Workload(name, wid, **base)


def seq_lengths(w: Workload, seed: int) -> np.ndarray:
    """Valid-token count N_b of each sequence at the trigger (n_slots = budget + buffer)."""
    if w.lengths[0] == "full":
        return np.full(w.batch, w.n_slots, dtype=np.int32)
    _, lo, hi = w.lengths
    out = np.empty(w.batch, dtype=np.int32)
    for b in range(w.batch):
        # one uniform integer per sequence: the top 53 bits of its stream key
        # scaled to [lo, hi] in exact integer arithmetic
        k = stream_key(seed, w.wid, T_LENGTHS, 0, b, 0)
        out[b] = lo + ((k >> 11) * (hi - lo + 1) >> 53)
    return out


def n_copies_for(w: Workload, n_valid: int) -> tuple:
    """(first_span, last_span, n_copies) of the repeated-span recipe for n_valid tokens."""
    nsp = n_valid // w.span_len
    if w.spans_in_candidates:
        last = (n_valid - w.obs_window) // w.span_len - 1
    else:
        last = nsp - 1
    if w.n_copies is not None:
        cnt = w.n_copies
    else:
        cnt = int(math.floor(w.copy_frac * nsp + 0.5))
    return 1, last, max(0, min(cnt, last))


@dataclass
class CacheSet:
    """One batch of per-layer caches plus observation queries, host memory."""

    w: Workload
    seed: int
    K: np.ndarray  # [L][b][H][C][D] uint16 (bf16 bits) or float32
    V: np.ndarray
    Q: np.ndarray  # [L][b][H*G][alpha][D]
    seq_start: np.ndarray  # [b] int32
    n_slots: int
    lengths: np.ndarray  # [b] int32


def _fill_pad(arr: np.ndarray, w: Workload):
    if w.dtype == "bf16":
        arr.fill(BF16_NAN)
    else:
        arr.fill(np.float32("nan"))


def _canary(w: Workload):
    return BF16_CANARY if w.dtype == "bf16" else np.uint32(0x7F800001).view(np.float32)


def build_cache(w: Workload, seed: int = 0, threads: Optional[int] = None) -> CacheSet:
    """Generates K, V, Q, seq_start for workload w.

    Sequence b holds N_b valid tokens in slots [n_slots - N_b, n_slots)
    (left padding). Padding slots are filled with NaN when w.nan_padding, so a
    masking leak shows up as a non-finite score; slots past n_slots carry a
    canary pattern.
    """
    L = lib()
    lens = seq_lengths(w, seed)
    C, D = w.capacity, w.head_dim
    K = np.empty((w.num_layers, w.batch, w.num_kv_heads, C, D), dtype=w.np_dtype)
    V = np.empty_like(K)
    Q = np.empty((w.num_layers, w.batch, w.q_heads, w.obs_window, D), dtype=w.np_dtype)
    seq_start = (w.n_slots - lens).astype(np.int32)

    def one(task):
        l, b, h = task
        n = int(lens[b])
        s0 = int(seq_start[b])
        kslc = K[l, b, h]
        vslc = V[l, b, h]
        if s0 > 0:
            if w.nan_padding:
                _fill_pad(kslc[:s0], w)
                _fill_pad(vslc[:s0], w)
            else:
                kslc[:s0] = 0
                vslc[:s0] = 0
        if C > w.n_slots:
            kslc[w.n_slots:] = _canary(w)
            vslc[w.n_slots:] = _canary(w)
        krows = np.empty((n, D), dtype=w.np_dtype)
        first, last, cnt = n_copies_for(w, n)
        L.synth_slice_keys(stream_key(seed, w.wid, T_KEYS, l, b, h), n, D, w.span_len, first, last, cnt,
                           w.noise_sigma, w.code, _ptr(krows), None)
        kslc[s0:s0 + n] = krows
        vrows = np.empty((n, D), dtype=w.np_dtype)
        L.synth_fill_normal(stream_key(seed, w.wid, T_VALUES, l, b, h), 0.0, 1.0, w.code, _ptr(vrows), n * D)
        vslc[s0:s0 + n] = vrows
        qblk = np.empty((w.group, w.obs_window, D), dtype=w.np_dtype)
        L.synth_fill_normal(stream_key(seed, w.wid, T_QUERIES, l, b, h), 0.0, 1.0, w.code, _ptr(qblk),
                            qblk.size)
        Q[l, b, h * w.group:(h + 1) * w.group] = qblk

    tasks = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads <= 1 or len(tasks) < 4:
        for t in tasks:
            one(t)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, tasks))
    return CacheSet(w, seed, K, V, Q, seq_start, w.n_slots, lens)


def to_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64 (bf16 bits or float32)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 bits (round-to-nearest-even) via the C generator's rule."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(f)] = BF16_NAN
    return r
