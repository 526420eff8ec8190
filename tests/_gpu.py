"""GPU-side helpers of the parity tests: device copies of synthetic caches,
calls through the C ABI, and the acceptance rule against the oracle."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle
import synth

# the acceptance rule's tolerances (defined, with their derivation, beside the
# rule itself in the oracle package)
TAU_BAND = oracle.TAU_BAND
REL_TOL = oracle.REL_TOL
# rbar is checked to REL_TOL relative, plus this absolute floor for row means
# that cancel to near 0: the fp32 error of khat_i . s / (N - 1), s the sum of
# unit keys, is about 128 * 2^-24 * |s| / (N - 1), which for the ~sqrt(N)-sized
# |s| of mostly unrelated keys lies far below 1e-6.
RBAR_FLOOR = 1e-6


def torch_dev():
    import torch

    return torch, torch.device("cuda")


def to_dev(arr: np.ndarray):
    torch, dev = torch_dev()
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def to_host(t, like_dtype) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if like_dtype == np.uint16:
        return a.view(np.uint16)
    return a


def params_of(w: synth.Workload):
    import redundancy_aware_compression_amd as rkv

    return rkv.make_params(w.num_layers, w.batch, w.num_kv_heads, w.group, w.capacity, w.budget, w.buffer,
                           w.obs_window, w.beta, w.lam, w.tau, w.dtype)


@dataclass
class DevCache:
    cs: synth.CacheSet
    K: object
    V: object
    Q: object
    seq_start: object

    @classmethod
    def of(cls, cs: synth.CacheSet) -> "DevCache":
        torch, dev = torch_dev()
        return cls(cs, to_dev(cs.K), to_dev(cs.V), to_dev(cs.Q), torch.from_numpy(cs.seq_start.copy()).to(dev))

    @property
    def w(self):
        return self.cs.w

    def k_layers(self):
        return [self.K[l] for l in range(self.w.num_layers)]

    def v_layers(self):
        return [self.V[l] for l in range(self.w.num_layers)]


def slice_index(w, l, b, h):
    return (l * w.batch + b) * w.num_kv_heads + h


def gpu_score(dc: DevCache, n_slots=None):
    """rkv_score on the device copy; returns host (importance, redundancy, counts), each [slices][n_slots]."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = torch_dev()
    w = dc.w
    n = n_slots if n_slots is not None else dc.cs.n_slots
    p = params_of(w)
    wsb = rkv.rkv_workspace_bytes(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    imp = torch.zeros(w.slices * n, dtype=torch.float32, device=dev)
    red = torch.zeros_like(imp)
    cnt = torch.full((w.slices * n,), -7, dtype=torch.int32, device=dev)
    rkv.rkv_score(p, dc.k_layers(), dc.Q, dc.seq_start, n, imp, red, cnt, ws, wsb)
    torch.cuda.synchronize()
    return (imp.cpu().numpy().reshape(w.slices, n), red.cpu().numpy().reshape(w.slices, n),
            cnt.cpu().numpy().reshape(w.slices, n))


def gpu_select(dc: DevCache, imp: np.ndarray, red: np.ndarray, n_slots=None):
    """rkv_select from host score arrays; returns (keep [slices][B], z [slices][n], r [slices][n])."""
    import redundancy_aware_compression_amd as rkv

    torch, dev = torch_dev()
    w = dc.w
    n = n_slots if n_slots is not None else dc.cs.n_slots
    p = params_of(w)
    ti = torch.from_numpy(np.ascontiguousarray(imp, dtype=np.float32).reshape(-1)).to(dev)
    tr = torch.from_numpy(np.ascontiguousarray(red, dtype=np.float32).reshape(-1)).to(dev)
    keep = torch.full((w.slices * w.budget,), -9, dtype=torch.int32, device=dev)
    z = torch.zeros(w.slices * n, dtype=torch.float32, device=dev)
    r = torch.zeros_like(z)
    rkv.rkv_select(p, ti, tr, dc.seq_start, n, keep, z, r)
    torch.cuda.synchronize()
    return (keep.cpu().numpy().reshape(w.slices, w.budget), z.cpu().numpy().reshape(w.slices, n),
            r.cpu().numpy().reshape(w.slices, n))


def oracle_slice(cs: synth.CacheSet, l, b, h):
    w = cs.w
    s0 = int(cs.seq_start[b])
    return oracle.slice_eval(cs.K[l, b, h, s0:cs.n_slots], cs.Q[l, b, h * w.group:(h + 1) * w.group],
                             budget=w.budget, obs_window=w.obs_window, beta=w.beta, lam=w.lam, tau=w.tau,
                             amb_eps=TAU_BAND)


def check_scores(ref, imp, red, cnt, what=""):
    """Importance to REL_TOL relative; counts exact and redundancy to REL_TOL
    relative (plus RBAR_FLOOR) except rows with a pair inside the tau band.
    Returns #band rows."""
    N = ref.importance.shape[0]
    r_i = ref.importance
    bad = np.abs(imp[:N] - r_i) > REL_TOL * np.abs(r_i) + 1e-30
    assert not bad.any(), f"{what} importance: {bad.sum()} bad, worst rel " \
                          f"{np.max(np.abs(imp[:N] - r_i) / np.maximum(np.abs(r_i), 1e-30)):.3e}"
    amb = ref.ambiguous.astype(bool)
    cbad = (cnt[:N] != ref.counts) & ~amb
    assert not cbad.any(), f"{what} counts differ at {np.nonzero(cbad)[0][:10]}: gpu {cnt[:N][cbad][:10]} " \
                           f"ref {ref.counts[cbad][:10]}"
    rbad = (np.abs(red[:N] - ref.rbar) > REL_TOL * np.abs(ref.rbar) + RBAR_FLOOR) & ~amb
    assert not rbad.any(), f"{what} redundancy: {rbad.sum()} bad, worst {np.max(np.abs(red[:N] - ref.rbar)):.3e}"
    return int(amb.sum())


def check_z_r(ref, z, r, w, N, what=""):
    """Z and R of the selection fed the GPU's scores against the oracle's:
    R to REL_TOL relative, Z within eps_i = REL_TOL (lam I_i + (1 - lam) R_i)
    (the bound the relative errors of I and R give). Rows on a tau-ambiguous
    pair are excepted: their counts, hence rbar and R, may legitimately differ."""
    nc = N - w.obs_window
    amb = ref.ambiguous[:nc].astype(bool)
    I, R, Z = ref.importance[:nc], ref.R[:nc], ref.Z[:nc]
    rb = (np.abs(r[:nc] - R) > REL_TOL * R) & ~amb
    assert not rb.any(), f"{what} R from GPU scores: {rb.sum()} bad"
    eps = REL_TOL * (w.lam * np.abs(I) + (1 - w.lam) * np.abs(R))
    zb = (np.abs(z[:nc] - Z) > eps + 1e-12) & ~amb
    assert not zb.any(), f"{what} Z from GPU scores: {zb.sum()} bad, worst {np.max(np.abs(z[:nc] - Z) - eps):.3e}"


def band_exceptions(ref, w, N):
    """Candidates whose oracle Z lies within tolerance of the k-th largest."""
    return oracle.band_exceptions(ref, N, w.budget, w.obs_window, w.lam, REL_TOL)


def check_keep(keep_rel: np.ndarray, ref, w, N, what=""):
    """GPU keep (positions within the slice) vs the oracle's under the band rule.
    Returns the number of differing candidates (all inside the band)."""
    problems, ndiff, outside = oracle.compare_keep(keep_rel, ref, N, w.budget, w.obs_window, w.lam, REL_TOL)
    assert not problems, f"{what}: {problems}"
    assert not outside, f"{what} keep differs outside the tolerance band at {outside[:10]}"
    return ndiff


def check_self_topk(keep_rel: np.ndarray, z: np.ndarray, w, N, what=""):
    """The GPU's keep is exactly the top-k of the GPU's own Z (ties: later wins)."""
    nc, k = N - w.obs_window, w.budget - w.obs_window
    zz = z[:nc].astype(np.float32)
    zz = np.where(zz == 0, np.float32(0), zz)  # -0 == +0
    order = sorted(range(nc), key=lambda i: (-float(zz[i]), -i))
    exp = sorted(order[:k] + list(range(nc, N)))
    assert np.array_equal(keep_rel, np.asarray(exp)), f"{what} keep is not the top-k of its own scores"


def keep_rel_of(keep_row: np.ndarray, s0: int) -> np.ndarray:
    v = keep_row[keep_row >= 0]
    return (v - s0).astype(np.int64)
