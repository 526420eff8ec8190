"""ctypes marshalling for librkv.so; names and argument order follow include/rkv.h."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "librkv.so")

RKV_BF16 = 0
RKV_F32 = 1
RKV_MAX_LAYERS = 128
RKV_MAX_CAPACITY = 16384
RKV_MAX_QROWS = 64
RKV_NOALLOC_WORKSPACE_BYTES = 32 << 20

STATUS = {
    0: "RKV_OK",
    1: "RKV_ERR_NULL_ARG",
    2: "RKV_ERR_BAD_SHAPE",
    3: "RKV_ERR_BAD_PARAM",
    4: "RKV_ERR_WORKSPACE_TOO_SMALL",
    5: "RKV_ERR_MISALIGNED",
    6: "RKV_ERR_UNSUPPORTED",
    7: "RKV_ERR_HIP",
    8: "RKV_ERR_PRECONDITION",
}


class RkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        if status == 7:
            msg += f" (hipError {_lib().rkv_last_hip_error()})"
        super().__init__(msg)


class RkvParams(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("budget", ctypes.c_int32),
        ("buffer", ctypes.c_int32),
        ("obs_window", ctypes.c_int32),
        ("beta", ctypes.c_int32),
        ("lambda_", ctypes.c_float),
        ("sim_threshold", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


def make_params(num_layers: int, batch: int, num_kv_heads: int, group: int, capacity: int, budget: int,
                buffer: int = 128, obs_window: int = 8, beta: int = 2, lam: float = 0.1, tau: float = 0.5,
                dtype: str = "bf16", head_dim: int = 128) -> RkvParams:
    code = {"bf16": RKV_BF16, "f32": RKV_F32}[dtype] if isinstance(dtype, str) else int(dtype)
    return RkvParams(num_layers, batch, num_kv_heads, group, head_dim, capacity, budget, buffer, obs_window, beta,
                     lam, tau, code)


_handle = None


def library_path() -> str:
    return _LIB


def hip_runtimes_mapped() -> set:
    """Paths of the HIP runtime libraries mapped into this process."""
    with open("/proc/self/maps") as f:
        return {line.split()[-1] for line in f if "libamdhip64" in line.split()[-1]}


def load_hip_library(path: str) -> ctypes.CDLL:
    """Loads a HIP library built here (librkv, the peak microbenchmarks).
    They need the HIP runtime by soname. torch ships its own copy; if such a
    library were loaded first, the system copy would be mapped and torch
    would map its own beside it: two runtimes in one process, the library's
    launches going through one that cannot use the device torch has opened.
    Mapping torch's first makes the library bind to it; loading refuses when
    more than one runtime is mapped all the same."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(path)
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime is mapped into this process: {sorted(runtimes)}; load "
                          "this package's libraries after torch, or without torch in the process")
    return L


def _lib():
    global _handle
    if _handle is None:
        if not os.path.exists(_LIB):
            raise ImportError(f"librkv.so is not built at {_LIB}; run `python -m redundancy_aware_compression_amd.build`")
        L = load_hip_library(_LIB)
        P = ctypes.POINTER(RkvParams)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.rkv_workspace_bytes.restype = sz
        L.rkv_workspace_bytes.argtypes = [P]
        L.rkv_workspace_keep_offset.restype = sz
        L.rkv_workspace_keep_offset.argtypes = [P]
        L.rkv_score.restype = ctypes.c_int
        L.rkv_score.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        L.rkv_select.restype = ctypes.c_int
        L.rkv_select.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp]
        L.rkv_compact.restype = ctypes.c_int
        L.rkv_compact.argtypes = [P, vp, vp, vp, vp, i32, vp]
        L.rkv_evict_step.restype = ctypes.c_int
        L.rkv_evict_step.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(i32), vp, sz, vp]
        L.rkv_evict_step_timed.restype = ctypes.c_int
        L.rkv_evict_step_timed.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(i32), vp, sz, vp, vp]
        L.rkv_evict_step_holefill.restype = ctypes.c_int
        L.rkv_evict_step_holefill.argtypes = [P, vp, vp, vp, vp, vp, ctypes.POINTER(i32), vp, sz, vp]
        L.rkv_evict_step_holefill_timed.restype = ctypes.c_int
        L.rkv_evict_step_holefill_timed.argtypes = [P, vp, vp, vp, vp, vp, ctypes.POINTER(i32), vp, sz, vp, vp]
        L.rkv_compact_holefill.restype = ctypes.c_int
        L.rkv_compact_holefill.argtypes = [P, vp, vp, vp, vp, vp, i32, vp]
        f32 = ctypes.c_float
        L.rkv_select_sampled.restype = ctypes.c_int
        L.rkv_select_sampled.argtypes = [P, vp, vp, vp, i32, i32, i32, f32, vp, vp]
        L.rkv_evict_step_sampled.restype = ctypes.c_int
        L.rkv_evict_step_sampled.argtypes = [P, vp, vp, vp, vp, vp, ctypes.POINTER(i32), i32, i32, f32, vp, sz, vp]
        L.rkv_sentence_penalty.restype = ctypes.c_int
        L.rkv_sentence_penalty.argtypes = [P, vp, vp, i32, i32, f32, vp, vp]
        L.rkv_evict_step_sentences.restype = ctypes.c_int
        L.rkv_evict_step_sentences.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(i32), vp, vp, vp, i32, i32, f32, vp,
                                               vp, sz, vp]
        L.rkv_decode_attention.restype = ctypes.c_int
        L.rkv_decode_attention.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp]
        L.rkv_evict_step_noalloc.restype = ctypes.c_int
        L.rkv_evict_step_noalloc.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(i32), vp]
        L.rkv_evict_step_captured.restype = ctypes.c_int
        L.rkv_evict_step_captured.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(i32), vp, sz, vp]
        L.rkv_status_string.restype = ctypes.c_char_p
        L.rkv_status_string.argtypes = [ctypes.c_int]
        L.rkv_last_hip_error.restype = ctypes.c_int
        L.rkv_last_hip_error.argtypes = []
        _handle = L
    return _handle


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _ptr_array(xs: Sequence) -> ctypes.Array:
    return (ctypes.c_void_p * len(xs))(*[_ptr(x) for x in xs])


def _layers(p: RkvParams, xs: Sequence, what: str):
    """The HOST array of per-layer cache pointers, as a void pointer. The
    library reads exactly p.num_layers entries, so a shorter list would hand
    it arbitrary memory as device pointers: the count is checked here, and a
    tensor entry must hold exactly one layer [batch][num_kv_heads][capacity]
    [head_dim] of the cache's element type, contiguous."""
    if 1 <= p.num_layers <= RKV_MAX_LAYERS and len(xs) != p.num_layers:
        # (an out-of-range num_layers is the library's RKV_ERR_BAD_SHAPE, returned before it reads the array)
        raise ValueError(f"{what}: {len(xs)} layer pointers for num_layers = {p.num_layers}")
    elem = 4 if p.dtype == RKV_F32 else 2
    need = p.batch * p.num_kv_heads * p.capacity * p.head_dim
    for l, x in enumerate(xs):
        if x is None:
            raise ValueError(f"{what}[{l}] is None")
        if isinstance(x, int) or not hasattr(x, "numel"):
            continue
        if x.element_size() != elem or x.numel() != need or not x.is_contiguous():
            raise ValueError(f"{what}[{l}]: {x.numel()} contiguous elements of {elem} bytes expected "
                             f"({need}); got {x.numel()} of {x.element_size()} bytes, contiguous={x.is_contiguous()}")
    return ctypes.cast(_ptr_array(xs), ctypes.c_void_p)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return int(torch.cuda.current_stream().cuda_stream) if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(st: int, where: str) -> int:
    if st != 0:
        raise RkvError(st, where)
    return st


def rkv_workspace_bytes(p: RkvParams) -> int:
    return int(_lib().rkv_workspace_bytes(ctypes.byref(p)))


def rkv_workspace_keep_offset(p: RkvParams) -> int:
    """Byte offset of rkv_evict_step's keep lists in the workspace; raises on invalid params."""
    off = int(_lib().rkv_workspace_keep_offset(ctypes.byref(p)))
    if off == ctypes.c_size_t(-1).value:
        raise RkvError(3, "rkv_workspace_keep_offset")
    return off


def rkv_status_string(st: int) -> str:
    return _lib().rkv_status_string(st).decode()


def rkv_last_hip_error() -> int:
    return int(_lib().rkv_last_hip_error())


def rkv_score(p: RkvParams, k_layers: Sequence, obs_q, seq_start, n_slots: int, importance, redundancy,
              counts=None, ws=None, ws_bytes: int = 0, stream=None, check: bool = True) -> int:
    st = _lib().rkv_score(ctypes.byref(p), _layers(p, k_layers, "k_layers"), _ptr(obs_q),
                          _ptr(seq_start), n_slots, _ptr(importance), _ptr(redundancy), _ptr(counts), _ptr(ws),
                          ws_bytes, _stream(stream))
    return _check(st, "rkv_score") if check else st


def rkv_select(p: RkvParams, importance, redundancy, seq_start, n_slots: int, keep, z_out=None, r_out=None,
               stream=None, check: bool = True) -> int:
    st = _lib().rkv_select(ctypes.byref(p), _ptr(importance), _ptr(redundancy), _ptr(seq_start), n_slots, _ptr(keep),
                           _ptr(z_out), _ptr(r_out), _stream(stream))
    return _check(st, "rkv_select") if check else st


def rkv_compact(p: RkvParams, k_layers: Sequence, v_layers: Sequence, keep, seq_start, n_slots: int, stream=None,
                check: bool = True) -> int:
    st = _lib().rkv_compact(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                            _layers(p, v_layers, "v_layers"), _ptr(keep), _ptr(seq_start), n_slots,
                            _stream(stream))
    return _check(st, "rkv_compact") if check else st


def rkv_evict_step(p: RkvParams, k_layers: Sequence, v_layers: Sequence, obs_q, seq_start, n_slots: int, ws,
                   ws_bytes: int, stream=None, check: bool = True):
    """Returns (status, n_slots after the step)."""
    ns = ctypes.c_int32(n_slots)
    st = _lib().rkv_evict_step(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                               _layers(p, v_layers, "v_layers"), _ptr(obs_q), _ptr(seq_start),
                               ctypes.byref(ns), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "rkv_evict_step")
    return st, ns.value


def rkv_evict_step_timed(p: RkvParams, k_layers: Sequence, v_layers: Sequence, obs_q, seq_start, n_slots: int, ws,
                         ws_bytes: int, stage_events: Sequence[int], stream=None, check: bool = True):
    """rkv_evict_step recording 4 caller-created hipEvent_t handles between its stages."""
    ns = ctypes.c_int32(n_slots)
    if len(stage_events) != 4:
        raise ValueError("rkv_evict_step_timed takes 4 events")
    ev = (ctypes.c_void_p * 4)(*stage_events)
    st = _lib().rkv_evict_step_timed(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                     _layers(p, v_layers, "v_layers"), _ptr(obs_q),
                                     _ptr(seq_start), ctypes.byref(ns), _ptr(ws), ws_bytes, _stream(stream),
                                     ctypes.cast(ev, ctypes.c_void_p))
    if check:
        _check(st, "rkv_evict_step_timed")
    return st, ns.value


def rkv_evict_step_holefill(p: RkvParams, k_layers: Sequence, v_layers: Sequence, obs_q, seq_start, order,
                            n_slots: int, ws, ws_bytes: int, stream=None, check: bool = True):
    """The eviction step in the hole-filling layout; returns (status, n_slots after the step)."""
    ns = ctypes.c_int32(n_slots)
    st = _lib().rkv_evict_step_holefill(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                        _layers(p, v_layers, "v_layers"), _ptr(obs_q),
                                        _ptr(seq_start), _ptr(order), ctypes.byref(ns), _ptr(ws), ws_bytes,
                                        _stream(stream))
    if check:
        _check(st, "rkv_evict_step_holefill")
    return st, ns.value


def rkv_evict_step_holefill_timed(p: RkvParams, k_layers: Sequence, v_layers: Sequence, obs_q, seq_start, order,
                                  n_slots: int, ws, ws_bytes: int, stage_events: Sequence[int], stream=None,
                                  check: bool = True):
    """rkv_evict_step_holefill recording 4 caller-created hipEvent_t handles between its stages."""
    ns = ctypes.c_int32(n_slots)
    if len(stage_events) != 4:
        raise ValueError("rkv_evict_step_holefill_timed takes 4 events")
    ev = (ctypes.c_void_p * 4)(*stage_events)
    st = _lib().rkv_evict_step_holefill_timed(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                              _layers(p, v_layers, "v_layers"), _ptr(obs_q),
                                              _ptr(seq_start), _ptr(order), ctypes.byref(ns), _ptr(ws), ws_bytes,
                                              _stream(stream), ctypes.cast(ev, ctypes.c_void_p))
    if check:
        _check(st, "rkv_evict_step_holefill_timed")
    return st, ns.value


def rkv_compact_holefill(p: RkvParams, k_layers: Sequence, v_layers: Sequence, keep, seq_start, order,
                         n_slots: int, stream=None, check: bool = True) -> int:
    st = _lib().rkv_compact_holefill(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                     _layers(p, v_layers, "v_layers"), _ptr(keep),
                                     _ptr(seq_start), _ptr(order), n_slots, _stream(stream))
    return _check(st, "rkv_compact_holefill") if check else st


def rkv_select_sampled(p: RkvParams, scores, uniforms, seq_start, n_slots: int, keep_newest: int, top_k: int,
                       temperature: float, keep, stream=None, check: bool = True) -> int:
    st = _lib().rkv_select_sampled(ctypes.byref(p), _ptr(scores), _ptr(uniforms), _ptr(seq_start), n_slots,
                                   keep_newest, top_k, temperature, _ptr(keep), _stream(stream))
    return _check(st, "rkv_select_sampled") if check else st


def rkv_evict_step_sampled(p: RkvParams, k_layers: Sequence, v_layers: Sequence, scores, uniforms, seq_start,
                           n_slots: int, keep_newest: int, top_k: int, temperature: float, ws, ws_bytes: int,
                           stream=None, check: bool = True):
    """The eviction step with the sampled selection; returns (status, n_slots after the step)."""
    ns = ctypes.c_int32(n_slots)
    st = _lib().rkv_evict_step_sampled(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                       _layers(p, v_layers, "v_layers"), _ptr(scores),
                                       _ptr(uniforms), _ptr(seq_start), ctypes.byref(ns), keep_newest, top_k,
                                       temperature, _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "rkv_evict_step_sampled")
    return st, ns.value


def rkv_sentence_penalty(p: RkvParams, vectors, n_sent, s_max: int, dim: int, tau_s: float, penalty, stream=None,
                         check: bool = True) -> int:
    st = _lib().rkv_sentence_penalty(ctypes.byref(p), _ptr(vectors), _ptr(n_sent), s_max, dim, tau_s, _ptr(penalty),
                                     _stream(stream))
    return _check(st, "rkv_sentence_penalty") if check else st


def rkv_evict_step_sentences(p: RkvParams, k_layers: Sequence, v_layers: Sequence, obs_q, seq_start, n_slots: int,
                             sent_id, vectors, n_sent, s_max: int, dim: int, tau_s: float, penalty, ws, ws_bytes: int,
                             stream=None, check: bool = True):
    """The eviction step with SkipKV's sentence deduction; returns (status, n_slots after the step)."""
    ns = ctypes.c_int32(n_slots)
    st = _lib().rkv_evict_step_sentences(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                         _layers(p, v_layers, "v_layers"), _ptr(obs_q),
                                         _ptr(seq_start), ctypes.byref(ns), _ptr(sent_id), _ptr(vectors),
                                         _ptr(n_sent), s_max, dim, tau_s, _ptr(penalty), _ptr(ws), ws_bytes,
                                         _stream(stream))
    if check:
        _check(st, "rkv_evict_step_sentences")
    return st, ns.value


def rkv_decode_attention(p: RkvParams, k_layers: Sequence, v_layers: Sequence, q, seq_start, n_slots: int, out,
                         imp_acc=None, stream=None, check: bool = True) -> int:
    """Decode attention of the newest token; with imp_acc the weights are added into it."""
    st = _lib().rkv_decode_attention(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                     _layers(p, v_layers, "v_layers"), _ptr(q), _ptr(seq_start),
                                     n_slots, _ptr(out), _ptr(imp_acc) if imp_acc is not None else None,
                                     _stream(stream))
    return _check(st, "rkv_decode_attention") if check else st


def rkv_evict_step_captured(p: RkvParams, k_layers: Sequence, v_layers: Sequence, imp_acc, seq_start, n_slots: int,
                            ws, ws_bytes: int, stream=None, check: bool = True):
    """The eviction step with the importance captured by decode attention; returns
    (status, n_slots after the step)."""
    ns = ctypes.c_int32(n_slots)
    st = _lib().rkv_evict_step_captured(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                        _layers(p, v_layers, "v_layers"), _ptr(imp_acc),
                                        _ptr(seq_start), ctypes.byref(ns), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "rkv_evict_step_captured")
    return st, ns.value


def rkv_evict_step_noalloc(p: RkvParams, k_layers: Sequence, v_layers: Sequence, obs_q, seq_start, n_slots: int,
                           stream=None, check: bool = True):
    """rkv_evict_step on the library's built-in workspace (no allocation);
    returns (status, n_slots after the step)."""
    ns = ctypes.c_int32(n_slots)
    st = _lib().rkv_evict_step_noalloc(ctypes.byref(p), _layers(p, k_layers, "k_layers"),
                                       _layers(p, v_layers, "v_layers"), _ptr(obs_q), _ptr(seq_start),
                                       ctypes.byref(ns), _stream(stream))
    if check:
        _check(st, "rkv_evict_step_noalloc")
    return st, ns.value
