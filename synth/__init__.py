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
T_KEYS, T_VALUES, T_QUERIES, T_LENGTHS, T_MIX, T_SCORES, T_UNIFORMS, T_SENT = 0, 1, 2, 3, 4, 5, 6, 7

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
        L.synth_repeat_plan.restype = i32
        L.synth_repeat_plan.argtypes = [u64, i32, i32, dbl, i32, vp]
        L.synth_repeat_apply.restype = None
        L.synth_repeat_apply.argtypes = [u64, i32, i32, i32, vp, dbl, vp, i32, vp]
        L.synth_fill_uniform_open.restype = None
        L.synth_fill_uniform_open.argtypes = [u64, vp, i64]
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


# ---------------------------------------------------------------------------
# Long-generation sweep: 16K generated tokens as successive eviction rounds of
# `buffer` new tokens (R-KV page, summary table, row "throughput": 16K
# generation at a 10 % budget and at budget 1024).

# stream tensor ids of round r: SWEEP_T0 + 8 (r + 1) + kind (r = -1: the
# initial cache)
SWEEP_T0 = 16
K_DRIFT, K_TOKENS, K_PLAN, K_NOISE, K_VALUES, K_QUERIES = range(6)


@dataclass(frozen=True)
class SweepRecipe:
    """Token recipe of the sweep: a drifting Gaussian mixture per slice
    (same-component cosine about 0.2, below tau) with noisy repeats of
    windows of the retained cache."""

    n_comp: int = 16
    mean_sigma: float = 0.5
    drift_sigma: float = 0.05
    repeat_p: float = 0.3
    block_len: int = 32
    noise_sigma: float = 0.05
    rounds: int = 125


@dataclass
class SweepRound:
    """Host inputs of one round before the repeats are applied."""

    r: int
    K: np.ndarray  # [L][b][H][buffer][D] new keys (mixture tokens)
    V: np.ndarray  # [L][b][H][buffer][D] new values, N(0, 1)
    Q: np.ndarray  # [L][b][H*G][alpha][D] observation queries, N(0, 1)
    src: np.ndarray  # [L][b][H][buffer / block_len] window start in the retained cache, -1 = none

    def window_rows(self, w: Workload) -> np.ndarray:
        """Flat cache-row indices ((slice * capacity) + slot) of every
        replaced block's source window, in slice-major, block order."""
        blk = self.src.reshape(w.slices, -1)
        sl, bi = np.nonzero(blk >= 0)
        starts = sl.astype(np.int64) * w.capacity + blk[sl, bi]
        bl = self.K.shape[3] // blk.shape[1]
        return (starts[:, None] + np.arange(bl)[None, :]).reshape(-1)


class Sweep:
    """Seeded inputs of the long-generation sweep for a workload with
    batch-uniform lengths: an initial cache of `budget` tokens per slice
    (the steady state), then per round `buffer` new tokens appended after
    them and fresh observation queries. The repeats of a round copy windows
    of the cache retained by the previous eviction, which the caller fetches
    (SweepRound.window_rows) from wherever that cache lives."""

    def __init__(self, w: Workload, seed: int = 0, recipe: SweepRecipe = SweepRecipe(),
                 threads: Optional[int] = None):
        assert w.lengths == ("full",) and w.buffer % recipe.block_len == 0
        self.w, self.seed, self.rc = w, seed, recipe
        self.threads = threads or min(16, os.cpu_count() or 1)
        self.tasks = [(l, b, h) for l in range(w.num_layers) for b in range(w.batch) for h in range(w.num_kv_heads)]
        self.means = np.empty((w.slices, recipe.n_comp, w.head_dim), dtype=np.float64)
        L = lib()

        def init(i):
            l, b, h = self.tasks[i]
            L.synth_mixture_means(stream_key(seed, w.wid, T_MIX, l, b, h), recipe.n_comp, w.head_dim,
                                  recipe.mean_sigma, _ptr(self.means[i]))

        self._map(init)

    def _map(self, fn):
        """fn(i) for every slice i, over contiguous chunks of slices per thread."""
        n = len(self.tasks)
        if self.threads <= 1 or n < 4:
            for i in range(n):
                fn(i)
            return
        nch = min(n, 4 * self.threads)
        bounds = [n * c // nch for c in range(nch + 1)]

        def run(c):
            for i in range(bounds[c], bounds[c + 1]):
                fn(i)

        with ThreadPoolExecutor(self.threads) as ex:
            list(ex.map(run, range(nch)))

    def _key(self, r, kind, l, b, h):
        return stream_key(self.seed, self.w.wid, SWEEP_T0 + 8 * (r + 1) + kind, l, b, h)

    def initial(self) -> CacheSet:
        """Round-0 state: slots [0, budget) of every slice hold mixture tokens
        with repeats copied from the slice's own (pre-repeat) tokens; slots
        past the budget hold zeros; n_slots = budget."""
        w, rc, L = self.w, self.rc, lib()
        C, D, B = w.capacity, w.head_dim, w.budget
        K = np.zeros((w.num_layers, w.batch, w.num_kv_heads, C, D), dtype=w.np_dtype)
        V = np.zeros_like(K)
        Q = np.zeros((w.num_layers, w.batch, w.q_heads, w.obs_window, D), dtype=w.np_dtype)
        nblk = B // rc.block_len

        def one(i):
            l, b, h = self.tasks[i]
            rows = K[l, b, h, :B]
            L.synth_mixture_tokens(self._key(-1, K_TOKENS, l, b, h), B, D, rc.n_comp, _ptr(self.means[i]), w.code,
                                   _ptr(rows))
            src = np.empty(nblk, dtype=np.int32)
            nrep = L.synth_repeat_plan(self._key(-1, K_PLAN, l, b, h), B, rc.block_len, rc.repeat_p, B, _ptr(src))
            if nrep:
                win = np.ascontiguousarray(
                    np.concatenate([rows[s:s + rc.block_len] for s in src if s >= 0]))
                L.synth_repeat_apply(self._key(-1, K_NOISE, l, b, h), B, D, rc.block_len, _ptr(src),
                                     rc.noise_sigma, _ptr(win), w.code, _ptr(rows))
            L.synth_fill_normal(self._key(-1, K_VALUES, l, b, h), 0.0, 1.0, w.code, _ptr(V[l, b, h, :B]), B * D)

        self._map(one)
        seq_start = np.zeros(w.batch, dtype=np.int32)
        return CacheSet(w, self.seed, K, V, Q, seq_start, B, np.full(w.batch, B, dtype=np.int32))

    def begin_round(self, r: int) -> SweepRound:
        """Drifts the mixture and draws round r's new tokens, values, queries
        and repeat plan (everything that does not read the retained cache)."""
        w, rc, L = self.w, self.rc, lib()
        n, D = w.buffer, w.head_dim
        K = np.empty((w.num_layers, w.batch, w.num_kv_heads, n, D), dtype=w.np_dtype)
        V = np.empty_like(K)
        Q = np.empty((w.num_layers, w.batch, w.q_heads, w.obs_window, D), dtype=w.np_dtype)
        src = np.empty((w.num_layers, w.batch, w.num_kv_heads, n // rc.block_len), dtype=np.int32)

        def one(i):
            l, b, h = self.tasks[i]
            m = self.means[i]
            L.synth_mixture_drift(self._key(r, K_DRIFT, l, b, h), rc.n_comp, D, rc.drift_sigma, _ptr(m))
            L.synth_mixture_tokens(self._key(r, K_TOKENS, l, b, h), n, D, rc.n_comp, _ptr(m), w.code,
                                   _ptr(K[l, b, h]))
            L.synth_repeat_plan(self._key(r, K_PLAN, l, b, h), n, rc.block_len, rc.repeat_p, w.budget,
                                _ptr(src[l, b, h]))
            L.synth_fill_normal(self._key(r, K_VALUES, l, b, h), 0.0, 1.0, w.code, _ptr(V[l, b, h]), n * D)
            qb = Q[l, b, h * w.group:(h + 1) * w.group]
            L.synth_fill_normal(self._key(r, K_QUERIES, l, b, h), 0.0, 1.0, w.code, _ptr(qb), qb.size)

        self._map(one)
        return SweepRound(r, K, V, Q, src)

    def finish_round(self, rnd: SweepRound, windows: np.ndarray) -> None:
        """Applies the repeats: windows holds the rows of rnd.window_rows()
        ([rows][D], storage dtype) read from the retained cache."""
        w, rc, L = self.w, self.rc, lib()
        D, bl = w.head_dim, rc.block_len
        blk = rnd.src.reshape(w.slices, -1)
        nrep = (blk >= 0).sum(axis=1)
        first = np.concatenate([[0], np.cumsum(nrep)]) * bl
        assert windows.shape == (int(first[-1]), D) and windows.dtype == w.np_dtype
        Kf = rnd.K.reshape(w.slices, w.buffer, D)

        def one(i):
            if nrep[i] == 0:
                return
            l, b, h = self.tasks[i]
            win = np.ascontiguousarray(windows[first[i]:first[i + 1]])
            L.synth_repeat_apply(self._key(rnd.r, K_NOISE, l, b, h), w.buffer, D, bl, _ptr(np.ascontiguousarray(blk[i])),
                                 rc.noise_sigma, _ptr(win), w.code, _ptr(Kf[i]))

        self._map(one)


def sweep_sample(w: Workload, n: int = 32, seed: int = 11) -> list:
    """The fixed set of (layer, sequence, KV head) slices a sweep is checked
    on in every round: the first, a middle (L / 2 - 1) and the last layer x
    every KV head of sequence 0, then seeded random slices up to n."""
    L, H = w.num_layers, w.num_kv_heads
    picks = []
    for l in (0, L // 2 - 1, L - 1):
        for h in range(H):
            if (l, 0, h) not in picks:
                picks.append((l, 0, h))
    rng = np.random.default_rng(seed)
    while len(picks) < min(n, w.slices):
        t = (int(rng.integers(L)), int(rng.integers(w.batch)), int(rng.integers(H)))
        if t not in picks:
            picks.append(t)
    return picks[:n]


class DeviceSweep:
    """The sweep's cache resident on a torch device: K and V
    [L][b][H][capacity][D] and the observation queries, as the eviction step
    reads them. next_round(r) appends round r's tokens after the retained
    `budget` slots (the repeats' windows are read from the device cache) and
    leaves n_slots = budget + buffer with every sequence starting at slot 0.
    The caller then runs the eviction step, which must bring n_slots back to
    `budget`. With order=True the cache is kept in the hole-filling layout:
    `order` [L][b][H][budget] int32 (identity at first) maps the retained
    virtual slots to physical rows, and the repeats read their windows
    through it."""

    def __init__(self, sweep: Sweep, device="cuda", order: bool = False):
        import torch

        self.torch, self.sweep, self.w = torch, sweep, sweep.w
        w = self.w
        cs = sweep.initial()
        self.dev = torch.device(device)
        self.K = self._up(cs.K)
        self.V = self._up(cs.V)
        self.Q = self._up(cs.Q)
        del cs
        self.seq_start = torch.zeros(w.batch, dtype=torch.int32, device=self.dev)
        self.n_slots = w.budget
        self.order = None
        if order:
            ident = torch.arange(w.budget, dtype=torch.int32, device=self.dev)
            self.order = ident.repeat(w.slices).view(w.num_layers, w.batch, w.num_kv_heads, w.budget).contiguous()

    def _up(self, a: np.ndarray):
        t = self.torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        return t.to(self.dev)

    def host(self, t) -> np.ndarray:
        a = t.detach().cpu().numpy()
        return a.view(np.uint16) if self.w.dtype == "bf16" else a

    def k_layers(self):
        return [self.K[l] for l in range(self.w.num_layers)]

    def v_layers(self):
        return [self.V[l] for l in range(self.w.num_layers)]

    def next_round(self, r: int, rnd: Optional[SweepRound] = None) -> SweepRound:
        """Appends round r; rnd, when given, is self.sweep.begin_round(r)
        drawn ahead of time (it reads nothing the eviction changes, so a
        caller may draw round r + 1 while round r is evicted and checked)."""
        torch, w = self.torch, self.w
        assert self.n_slots == w.budget, "the previous round was not evicted"
        if rnd is None:
            rnd = self.sweep.begin_round(r)
        assert rnd.r == r
        rows = torch.from_numpy(rnd.window_rows(w)).to(self.dev)
        if self.order is not None:  # virtual retained slots -> physical rows
            sl, v = rows // w.capacity, rows % w.capacity
            rows = sl * w.capacity + self.order.view(-1, w.budget)[sl, v].long()
        win = self.host(self.K.view(-1, w.head_dim).index_select(0, rows))
        self.sweep.finish_round(rnd, win)
        B, n = w.budget, w.buffer
        self.K[:, :, :, B:B + n].copy_(torch.from_numpy(rnd.K.view(np.int16) if w.dtype == "bf16" else rnd.K))
        self.V[:, :, :, B:B + n].copy_(torch.from_numpy(rnd.V.view(np.int16) if w.dtype == "bf16" else rnd.V))
        self.Q.copy_(torch.from_numpy(rnd.Q.view(np.int16) if w.dtype == "bf16" else rnd.Q))
        self.seq_start.zero_()
        self.n_slots = B + n
        return rnd



def sampled_inputs(w: Workload, seed: int = 0):
    """Per-slot scores (N(0, 1), float32) and uniforms (strictly inside (0, 1),
    float32) of every slice, [L][b][H][n_slots]: the caller-side inputs of the
    sampled selection (a learned scorer's outputs and the draw's randomness)."""
    L = lib()
    shape = (w.num_layers, w.batch, w.num_kv_heads, w.n_slots)
    sc = np.empty(shape, np.float32)
    un = np.empty(shape, np.float32)
    for l in range(w.num_layers):
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                L.synth_fill_normal(stream_key(seed, w.wid, T_SCORES, l, b, h), 0.0, 1.0, F32, _ptr(sc[l, b, h]),
                                    w.n_slots)
                L.synth_fill_uniform_open(stream_key(seed, w.wid, T_UNIFORMS, l, b, h), _ptr(un[l, b, h]), w.n_slots)
    return sc, un



@dataclass
class Sentences:
    """Synthetic sentence structure of a cache (SkipKV's inputs): sequence b's
    valid tokens split into n_sent[b] sentences of 8..40 tokens in generation
    order; vectors[b][i] stands for the mean of sentence i's last-layer hidden
    states; sent_id[l][b][h][slot] is the sentence of the slot's token (-1 for
    padding and unused slots)."""

    vectors: np.ndarray  # [batch][s_max][dim] float32
    n_sent: np.ndarray  # [batch] int32
    sent_id: np.ndarray  # [L][b][H][capacity] int32


def sentences(cs: CacheSet, dim: int = 1024, repeat_p: float = 0.25, noise: float = 0.2, seed: int = 0) -> Sentences:
    """Sentence boundaries, vectors and the per-slot sentence sidecar for a
    cache. Vectors are N(0, 1); with probability repeat_p a sentence's vector
    is instead a noisy copy (noise sigma per element) of a uniformly chosen
    earlier sentence's, so that earlier sentence becomes redundant (cosine
    about 1 / sqrt(1 + noise^2))."""
    w = cs.w
    rng = np.random.default_rng(np.uint64(stream_key(seed, w.wid, T_SENT, 0, 0, 0)))
    bounds = []
    for b in range(w.batch):
        n, t, ids = int(cs.lengths[b]), 0, []
        k = 0
        while t < n:
            ln = int(rng.integers(8, 41))
            ids.extend([k] * min(ln, n - t))
            t += ln
            k += 1
        bounds.append(np.asarray(ids, np.int32))
    n_sent = np.array([int(x.max()) + 1 if len(x) else 0 for x in bounds], np.int32)
    s_max = max(1, int(n_sent.max()))
    vec = np.zeros((w.batch, s_max, dim), np.float32)
    for b in range(w.batch):
        for i in range(n_sent[b]):
            if i > 0 and rng.random() < repeat_p:
                src = int(rng.integers(0, i))
                vec[b, i] = vec[b, src] + noise * rng.standard_normal(dim).astype(np.float32)
            else:
                vec[b, i] = rng.standard_normal(dim).astype(np.float32)
    sid = np.full((w.num_layers, w.batch, w.num_kv_heads, w.capacity), -1, np.int32)
    for b in range(w.batch):
        s0 = int(cs.seq_start[b])
        sid[:, b, :, s0:s0 + len(bounds[b])] = bounds[b]
    return Sentences(vec, n_sent, sid)
