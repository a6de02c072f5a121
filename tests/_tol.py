"""Parity bars for comparing the HIP path with the fp64 oracle.

* f32 path:  max_i |g_i - r_i| / max(|r_i|, rms(r)) <= 1e-4
* bf16 path: ||g - r||_F / ||r||_F <= 1e-2  and  max_i |g_i - r_i| <= 3e-2 * rms(r)

When the result itself is stored in bf16 (``stored_bf16=True``), storing it
costs up to half a bf16 ulp, 2^-8 * |r_i|, on top of the arithmetic; the
max-abs bar then reads |g_i - r_i| <= 3e-2 * rms(r) + 2^-8 * |r_i|.
"""
import numpy as np
import torch

F32_MAX_REL = 1e-4
BF16_FRO = 1e-2
BF16_MAX_ABS_RMS = 3e-2


def as_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def errors(g, r):
    g, r = as_np(g), as_np(r)
    assert g.shape == r.shape, (g.shape, r.shape)
    d = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r)))
    fro = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    max_rel = float(np.max(d / np.maximum(np.abs(r), rms))) if r.size else 0.0
    max_abs = float(d.max()) if r.size else 0.0
    return {"fro": fro, "max_rel": max_rel, "max_abs": max_abs, "rms": rms,
            "finite": bool(np.isfinite(g).all())}


def assert_f32(g, r, bar=F32_MAX_REL):
    e = errors(g, r)
    assert e["finite"] and e["max_rel"] <= bar, e
    return e


def assert_bf16(g, r, fro=BF16_FRO, max_abs_rms=BF16_MAX_ABS_RMS, stored_bf16=False):
    e = errors(g, r)
    assert e["finite"], e
    assert e["fro"] <= fro, e
    if stored_bf16:
        g, r = as_np(g), as_np(r)
        excess = np.abs(g - r) - (max_abs_rms * e["rms"] + 2.0 ** -8 * np.abs(r))
        e["max_excess"] = float(excess.max())
        assert e["max_excess"] <= 0, e
    else:
        assert e["max_abs"] <= max_abs_rms * e["rms"], e
    return e
