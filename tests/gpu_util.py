"""Helpers of the GPU parity tests: move seeded inputs to the device, and
compare the HIP path's results with the oracle's."""
import numpy as np
import torch

import sparse_mixture_experts_04_amd as moe

TIE_MARGIN = 1e-6     # top-k margin (float64 probability gap) below which ids may legally differ
WEIGHT_TOL = 1e-5     # routing weights, absolute, fp32
BF16_REL_TOL = 2e-2   # layer outputs, per-token relative L2, bf16 inputs with fp32 accumulation
F32_REL_TOL = 1e-4    # same for the all-fp32 path (fp32 rounding over d*F products)


def rel_tol(dtype):
    return BF16_REL_TOL if dtype == "bf16" else F32_REL_TOL


def to_dev(a, dtype, device="cuda"):
    """numpy input (bf16 bit patterns or float32) -> device tensor of the layer dtype."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def round_to(a64, dtype):
    """Round float64 values to the layer dtype (what a device buffer of that dtype holds)."""
    t = torch.from_numpy(np.ascontiguousarray(a64))
    return t.to(torch.bfloat16).to(torch.float64).numpy() if dtype == "bf16" else t.to(torch.float32).to(
        torch.float64).numpy()


def cfg_of(inp, T=None):
    w = inp.workload
    return moe.config(T if T is not None else inp.X.shape[0], w.d, w.F, w.E, w.k, inp.expert_capacity, w.dtype)


def row_rel_err(got, ref):
    """Per-row relative L2 error; rows whose reference is all zero must be exactly zero."""
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return out


def check_routing(ids_gpu, w_gpu, r, report=None):
    """ids bit-exact except tokens whose oracle margin is below TIE_MARGIN;
    weights within WEIGHT_TOL wherever the ids agree.  Returns the mask of
    tokens whose ids differ."""
    ids_gpu = np.asarray(ids_gpu)
    diff = (ids_gpu != r.ids).any(axis=1)
    flagged = r.margin < TIE_MARGIN
    bad = diff & ~flagged
    assert not bad.any(), f"ids differ on {int(bad.sum())} unflagged tokens, first {np.nonzero(bad)[0][:8]}"
    same = ~diff
    err = np.abs(np.asarray(w_gpu, dtype=np.float64)[same] - r.weights[same])
    assert err.size == 0 or err.max() <= WEIGHT_TOL, f"routing weight error {err.max():.3g}"
    if report is not None:
        report["flagged_tokens"] = int(flagged.sum())
        report["id_mismatch_tokens"] = int(diff.sum())
        report["max_weight_err"] = float(err.max()) if err.size else 0.0
    return diff


def check_dispatch_exact(counts, offsets, perm, inv_perm, disp, Tk):
    counts = np.asarray(counts)
    offsets = np.asarray(offsets)
    perm = np.asarray(perm)
    inv_perm = np.asarray(inv_perm)
    assert np.array_equal(counts, disp.counts), "expert_counts differ"
    assert np.array_equal(offsets, disp.offsets), "expert_offsets differ"
    N = int(disp.offsets[-1])
    assert np.array_equal(perm[:N], disp.perm), "perm differs"
    assert (perm[N:Tk] == -1).all(), "perm rows past N must be -1"
    assert np.array_equal(inv_perm, disp.inv_perm), "inv_perm differs"


def check_dispatch_valid(ids_gpu, counts, offsets, perm, inv_perm, E, capacity):
    """Properties any correct dispatch of the given ids has (used where a
    near-tie flipped ids, so the oracle's own dispatch is not comparable)."""
    ids_gpu = np.asarray(ids_gpu)
    T, k = ids_gpu.shape
    counts, offsets, perm, inv_perm = map(np.asarray, (counts, offsets, perm, inv_perm))
    assert np.array_equal(counts, np.bincount(ids_gpu.reshape(-1), minlength=E))
    kept = np.diff(offsets)
    if capacity >= 0:
        assert (kept == np.minimum(counts, capacity)).all()
    else:
        assert (kept == counts).all()
    N = int(offsets[-1])
    assert offsets[0] == 0 and (perm[N:] == -1).all()
    assert (inv_perm[perm[:N]] == np.arange(N)).all()
    assert int((inv_perm >= 0).sum()) == N
    t = perm[:N] // k
    s = perm[:N] % k
    e = ids_gpu[t, s]
    assert (np.diff(e.astype(np.int64) * T + t) > 0).all()
