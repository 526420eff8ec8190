"""CPU oracle of the R-KV eviction step — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never uses it.

``rkv_oracle.cpp`` is plain single-threaded C++ in double precision, built
with g++ into ``librkv_oracle.so`` next to this file; this module is only its
ctypes marshalling. Every function is pinned by the ``-m "not gpu"`` tests
(hand-derived closed forms, textbook special cases, invariants, brute force).
Parity unpinned by the pages themselves: they print no example, so the
readings they leave open (the exact combination formula and protection rule,
which the R-KV page does not print; the sentence penalty's form; the sampled
draw's parameters; the free-row order of the hole-filling layout) are pinned
to those readings, stated in the source, not to values the pages give.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rkv_oracle.cpp")
_HDR = os.path.join(_HERE, "rkv_oracle.h")
_LIB_PATH = os.path.join(_HERE, "librkv_oracle.so")

ORC_BF16 = 0
ORC_F32 = 1


def build(force: bool = False) -> str:
    """Compiles the oracle with g++ -O2 (no fast-math, no OpenMP, no SIMD intrinsics)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _SliceParams(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("group", ctypes.c_int32),
                ("obs_window", ctypes.c_int32), ("budget", ctypes.c_int32), ("beta", ctypes.c_int32),
                ("lam", ctypes.c_double), ("tau", ctypes.c_double), ("amb_eps", ctypes.c_double)]


class _SliceOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("importance", "rowmean", "counts", "rbar", "R", "Z", "ambiguous", "keep")]


class _StepParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_layers", "batch", "num_kv_heads", "group", "head_dim", "capacity", "budget", "buffer",
                 "obs_window", "beta")] + [("lam", ctypes.c_double), ("tau", ctypes.c_double)]


_lib = None


def load_library(path: str):
    """Loads an oracle shared library built from rkv_oracle.cpp and declares its C signatures."""
    L = ctypes.CDLL(path)
    L.orc_slice.restype = ctypes.c_int32
    L.orc_slice.argtypes = [ctypes.POINTER(_SliceParams), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.POINTER(_SliceOut)]
    L.orc_evict_step.restype = ctypes.c_int32
    L.orc_evict_step.argtypes = [ctypes.POINTER(_StepParams), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.orc_gather_rows.restype = None
    L.orc_gather_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p]
    L.orc_slice_penalized.restype = ctypes.c_int32
    L.orc_slice_penalized.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    L.orc_sentence_penalty.restype = None
    L.orc_sentence_penalty.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double,
                                       ctypes.c_void_p]
    L.orc_select_sampled.restype = ctypes.c_int32
    L.orc_select_sampled.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.orc_decode_attention.restype = ctypes.c_int32
    L.orc_decode_attention.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    L.orc_holefill_slice.restype = ctypes.c_int32
    L.orc_holefill_slice.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return ORC_BF16
    if a.dtype == np.float32:
        return ORC_F32
    raise TypeError(f"oracle inputs are bf16 bits (uint16) or float32, got {a.dtype}")


@dataclass
class SliceResult:
    kept: int
    keep: np.ndarray  # positions within the slice, ascending
    importance: Optional[np.ndarray] = None
    rowmean: Optional[np.ndarray] = None
    counts: Optional[np.ndarray] = None
    rbar: Optional[np.ndarray] = None
    R: Optional[np.ndarray] = None
    Z: Optional[np.ndarray] = None
    ambiguous: Optional[np.ndarray] = None


def slice_eval(keys: np.ndarray, queries: np.ndarray, budget: int, obs_window: int = 8, beta: int = 2,
               lam: float = 0.1, tau: float = 0.5, amb_eps: float = 0.0,
               token_penalty: Optional[np.ndarray] = None) -> SliceResult:
    """Scores and selects one slice.

    keys: [N, D]; queries: [G, alpha, D] (or [G*alpha, D]); both bf16 bits
    (uint16) or float32. Scores are returned only when N > budget.
    """
    keys = np.ascontiguousarray(keys)
    queries = np.ascontiguousarray(queries)
    code = _dtype_code(keys)
    assert _dtype_code(queries) == code
    N, D = keys.shape
    G = queries.size // (obs_window * D)
    assert G * obs_window * D == queries.size
    p = _SliceParams(N, D, G, obs_window, budget, beta, lam, tau, amb_eps)
    nk = min(N, budget)
    keep = np.zeros(max(nk, 1), dtype=np.int32)
    res = SliceResult(kept=0, keep=keep)
    out = _SliceOut()
    out.keep = keep.ctypes.data
    if N > budget:
        res.importance = np.zeros(N)
        res.rowmean = np.zeros(N)
        res.counts = np.zeros(N, dtype=np.int32)
        res.rbar = np.zeros(N)
        res.R = np.zeros(N)
        res.Z = np.zeros(N)
        res.ambiguous = np.zeros(N, dtype=np.int32)
        for name in ("importance", "rowmean", "counts", "rbar", "R", "Z", "ambiguous"):
            setattr(out, name, getattr(res, name).ctypes.data)
    if token_penalty is None:
        kept = lib().orc_slice(ctypes.byref(p), code, keys.ctypes.data, queries.ctypes.data, ctypes.byref(out))
    else:
        pen = np.ascontiguousarray(token_penalty, dtype=np.float64)
        assert pen.shape == (N,)
        kept = lib().orc_slice_penalized(ctypes.byref(p), code, keys.ctypes.data, queries.ctypes.data,
                                         pen.ctypes.data, ctypes.byref(out))
    if kept < 0:
        raise ValueError("oracle rejected the slice parameters")
    res.kept = kept
    res.keep = keep[:kept].copy()
    return res


def evict_step(K: np.ndarray, V: np.ndarray, Q: np.ndarray, seq_start: np.ndarray, n_slots: int, budget: int,
               buffer: int = 128, obs_window: int = 8, beta: int = 2, lam: float = 0.1, tau: float = 0.5):
    """One eviction step in place on host arrays K, V: [L][b][H][C][D].

    Returns (evicted: bool, n_slots_after, keep [L][b][H][B] source slots or -1).
    seq_start is updated in place.
    """
    assert K.shape == V.shape and K.dtype == V.dtype
    assert K.flags["C_CONTIGUOUS"] and V.flags["C_CONTIGUOUS"] and seq_start.dtype == np.int32
    Q = np.ascontiguousarray(Q)
    code = _dtype_code(K)
    L_, Bt, H, C, D = K.shape
    G = Q.shape[2] // H
    p = _StepParams(L_, Bt, H, G, D, C, budget, buffer, obs_window, beta, lam, tau)
    kptrs = (ctypes.c_void_p * L_)(*[K[l].ctypes.data for l in range(L_)])
    vptrs = (ctypes.c_void_p * L_)(*[V[l].ctypes.data for l in range(L_)])
    ns = ctypes.c_int32(n_slots)
    keep = np.full((L_, Bt, H, budget), -1, dtype=np.int32)
    rc = lib().orc_evict_step(ctypes.byref(p), code, ctypes.cast(kptrs, ctypes.c_void_p),
                              ctypes.cast(vptrs, ctypes.c_void_p), Q.ctypes.data, seq_start.ctypes.data,
                              ctypes.addressof(ns), keep.ctypes.data)
    if rc < 0:
        raise ValueError("oracle rejected the step parameters")
    return rc == 1, ns.value, keep


def gather_rows(src: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """dst[j] = src[keep[j]] for keep[j] >= 0; dst rows with keep[j] < 0 are zero."""
    src = np.ascontiguousarray(src)
    keep = np.ascontiguousarray(keep, dtype=np.int32)
    dst = np.zeros((keep.shape[0],) + src.shape[1:], dtype=src.dtype)
    row_bytes = src.strides[0]
    lib().orc_gather_rows(src.ctypes.data, keep.ctypes.data, keep.shape[0], row_bytes, dst.ctypes.data)
    return dst


def holefill_slice(K: np.ndarray, V: np.ndarray, order: np.ndarray, keep: np.ndarray, budget: int):
    """Hole-filling compaction of one slice (orc_holefill_slice) on copies:
    K, V are the slice's physical rows [n_slots][D], order its budget
    entries, keep the selection's budget entries. Returns (K', V', order',
    new start)."""
    K2, V2 = np.array(K, copy=True, order="C"), np.array(V, copy=True, order="C")
    o2 = np.array(order, dtype=np.int32, copy=True)
    kp = np.ascontiguousarray(keep, dtype=np.int32)
    assert K2.shape == V2.shape and kp.shape[0] == budget and o2.shape[0] == budget
    lead = lib().orc_holefill_slice(K2.ctypes.data, V2.ctypes.data, K2.strides[0], budget, K2.shape[0],
                                    kp.ctypes.data, o2.ctypes.data)
    if lead < 0:
        raise ValueError("order is not a permutation of [0, budget) or keep is malformed")
    return K2, V2, o2, int(lead)


def select_sampled(scores: np.ndarray, uniforms: np.ndarray, budget: int, keep_newest: int, top_k: int,
                   temperature: float = 1.0) -> np.ndarray:
    """orc_select_sampled on one slice: kept positions, ascending."""
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    un = np.ascontiguousarray(uniforms, dtype=np.float32)
    assert sc.shape == un.shape and sc.ndim == 1
    out = np.empty(max(budget, sc.shape[0]), np.int32)
    n = lib().orc_select_sampled(sc.shape[0], budget, keep_newest, top_k, temperature, sc.ctypes.data,
                                 un.ctypes.data, out.ctypes.data)
    if n < 0:
        raise ValueError("invalid sampled-selection parameters")
    return out[:n].copy()


def sentence_penalty(vectors: np.ndarray, tau_s: float) -> np.ndarray:
    """orc_sentence_penalty: vectors [n_sent][dim] float32 -> penalties [n_sent] (double)."""
    v = np.ascontiguousarray(vectors, dtype=np.float32)
    out = np.zeros(v.shape[0])
    lib().orc_sentence_penalty(v.shape[0], v.shape[1], v.ctypes.data, tau_s, out.ctypes.data)
    return out


def decode_attention(keys: np.ndarray, values: np.ndarray, queries: np.ndarray):
    """Decode attention of one slice: keys, values [n][D] and the newest
    token's queries [G][D] (bf16 as uint16, or float32). Returns (out [G][D],
    weights [G][n]) in float64."""
    keys, values, queries = (np.ascontiguousarray(a) for a in (keys, values, queries))
    dt = _dtype_code(keys)
    if _dtype_code(values) != dt or _dtype_code(queries) != dt:
        raise ValueError("keys, values and queries must share a dtype")
    n, D = keys.shape
    G = queries.shape[0]
    if values.shape != (n, D) or queries.shape != (G, D):
        raise ValueError("shape mismatch")
    out = np.zeros((G, D), np.float64)
    w = np.zeros((G, n), np.float64)
    rc = lib().orc_decode_attention(n, D, G, dt, keys.ctypes.data, values.ctypes.data, queries.ctypes.data,
                                    out.ctypes.data, w.ctypes.data)
    if rc != 0:
        raise ValueError("orc_decode_attention rejected its arguments")
    return out, w


# The acceptance rule of a GPU result against the oracle on the same bytes.
# |S_ij - tau| below TAU_BAND can flip the similarity decision between fp32
# accumulation and double: 128 exact products summed in fp32 carry a relative
# error of at most ~128 * 2^-24 of sum |k_i[d] k_j[d]| <= |k_i||k_j|, plus
# ~1e-7 from each norm, i.e. below 1.6e-5 in S; 3e-5 leaves headroom. Scores
# are compared to REL_TOL relative.
TAU_BAND = 3e-5
REL_TOL = 1e-3


def band_exceptions(ref: SliceResult, N: int, budget: int, obs_window: int, lam: float, rel_tol: float) -> np.ndarray:
    """The acceptance rule's exceptions among a slice's candidates: those whose
    oracle Z lies within eps_i + eps_k of the k-th largest Z (eps_i =
    rel_tol (lam |I_i| + (1 - lam) |R_i|), k = budget - obs_window, ties by
    the later slot), and those on a tau-ambiguous pair. Boolean [N - obs_window]."""
    nc, k = N - obs_window, budget - obs_window
    Z, I, R = ref.Z[:nc], ref.importance[:nc], ref.R[:nc]
    eps = rel_tol * (lam * np.abs(I) + (1 - lam) * np.abs(R))
    order = sorted(range(nc), key=lambda i: (-Z[i], -i))
    kth = order[k - 1]
    ex = np.abs(Z - Z[kth]) <= eps + eps[kth]
    return ex | ref.ambiguous[:nc].astype(bool)


def compare_keep(keep_rel: np.ndarray, ref: SliceResult, N: int, budget: int, obs_window: int, lam: float,
                 rel_tol: float):
    """A kept set (positions within the slice, ascending) against the oracle's
    under the acceptance rule. Returns (problems, n_diff, outside): problems
    lists structural violations (size, order, window), n_diff the candidates
    in one set only, outside those of them not excepted by band_exceptions."""
    problems = []
    keep_rel = np.asarray(keep_rel)
    if len(keep_rel) != min(N, budget):
        problems.append(f"kept {len(keep_rel)} != {min(N, budget)}")
        return problems, 0, []
    if np.any(np.diff(keep_rel) <= 0):
        problems.append("keep not strictly ascending")
    if N <= budget:
        if not np.array_equal(keep_rel, np.arange(N)):
            problems.append("a short sequence must keep every token")
        return problems, 0, []
    if not set(range(N - obs_window, N)) <= set(keep_rel.tolist()):
        problems.append("observation window not kept")
    g = set(int(x) for x in keep_rel if x < N - obs_window)
    r = set(int(x) for x in ref.keep if x < N - obs_window)
    diff = g ^ r
    outside = []
    if diff:
        ex = band_exceptions(ref, N, budget, obs_window, lam, rel_tol)
        outside = sorted(i for i in diff if not ex[i])
    return problems, len(diff), outside
