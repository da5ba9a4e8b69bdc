"""Shared helpers for the GPU parity tests (marshalling and tolerance checks only)."""
import math

import numpy as np
import torch

# Acceptance bar for floating-point outputs: max |d out| <= 2e-2 * max |ref| (per query row) and
# |d lse| <= 1e-3, with -inf matched exactly for rows that select nothing.
OUT_REL_TOL = 2e-2
LSE_ABS_TOL = 1e-3


def to_dev(w, device="cuda"):
    d = {"q": torch.from_numpy(w["q_bits"].view(np.int16)).view(torch.bfloat16).to(device),
         "k_cache": torch.from_numpy(w["k_cache"]).to(device),
         "indices": torch.from_numpy(w["indices"]).to(device)}
    if w["extra_k_cache"] is not None:
        d["extra_k_cache"] = torch.from_numpy(w["extra_k_cache"]).to(device)
        d["extra_indices"] = torch.from_numpy(w["extra_indices"]).to(device)
    return d


def check_rows(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    """out_gpu bf16 [..., H, 512], lse_gpu fp32 [..., H]; refs float64 of the same leading shape."""
    o = out_gpu.float().cpu().double().numpy().reshape(-1, *out_gpu.shape[-2:])
    l = lse_gpu.cpu().double().numpy().reshape(-1, lse_gpu.shape[-1])
    ro = np.asarray(out_ref).reshape(o.shape)
    rl = np.asarray(lse_ref).reshape(l.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    for r in range(o.shape[0]):
        ninf = np.isneginf(rl[r])
        assert np.array_equal(np.isneginf(l[r]), ninf), f"{what}: row {r} -inf pattern differs"
        if ninf.all():
            assert np.all(o[r] == 0), f"{what}: row {r} selects nothing but output is not zero"
            continue
        d_lse = np.abs(l[r][~ninf] - rl[r][~ninf]).max()
        assert d_lse <= LSE_ABS_TOL, f"{what}: row {r} |d lse| = {d_lse:.3e}"
        scale = np.abs(ro[r]).max()
        d_out = np.abs(o[r] - ro[r]).max()
        assert d_out <= OUT_REL_TOL * scale, f"{what}: row {r} |d out| = {d_out:.3e} > 2e-2 * {scale:.3e}"


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even, subnormals kept)."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    e = np.floor(np.log2(np.abs(x[fin])))
    q = np.exp2(np.maximum(e, -126) - 7)
    v = np.round(x[fin] / q) * q
    v = np.where(np.abs(v) >= 2.0 ** 128, np.copysign(np.inf, v), v)
    out[fin] = v
    return out


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().double().numpy()


def cuda_available():
    return torch.cuda.is_available()
