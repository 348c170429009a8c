"""Helpers for the GPU parity tests (comparison rules, device buffers)."""
import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
NEAR_TIE = 1e-6   # decisions whose oracle margin is below this are reported, not failed


def close(g, o, rel=1e-3):
    """|g - o| <= rel * max(|o|, 1e-3 * rms(o)) element-wise (finite entries);
    non-finite entries must agree exactly."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    fin = np.isfinite(o)
    assert np.array_equal(fin, np.isfinite(g)), "finite pattern differs"
    assert np.array_equal(g[~fin], o[~fin]), "non-finite entries differ"
    if not fin.any():
        return 0.0
    rms = np.sqrt(np.mean(o[fin] ** 2))
    bound = rel * np.maximum(np.abs(o[fin]), 1e-3 * rms)
    err = np.abs(g[fin] - o[fin])
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"max error / bound = {worst:.3g}"
    return worst


def bf16_ulp_close(g_bf16: torch.Tensor, o_f32: np.ndarray, ulps: int = 1, floor_rel: float = 1e-6):
    """bf16 output against the float oracle: within `ulps` bf16 steps (at the
    oracle's magnitude) plus the absolute floor floor_rel * rms(o).  The floor
    is the fp32 tolerance's rms floor (1e-3 * 1e-3 rms): outputs that cancel to
    far below the typical magnitude have bf16 steps far smaller than the fp32
    accumulation error, so a bare step count cannot hold there.  Returns the
    largest error in bf16 steps (for the report)."""
    o = np.asarray(o_f32, np.float64)
    g = g_bf16.detach().float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(o ** 2)) if o.size else 0.0
    mag = np.maximum(np.abs(o), np.finfo(np.float32).tiny)
    step = np.exp2(np.floor(np.log2(mag)) - 7)          # bf16 spacing at |o|
    err = np.abs(g - o)
    assert np.all(err <= ulps * step + floor_rel * rms), \
        f"max error / bound = {float(np.max(err / (ulps * step + floor_rel * rms))):.3g}"
    return float(np.max(err / step))


def dev(x):
    return x.to(DEV) if isinstance(x, torch.Tensor) else torch.as_tensor(x).to(DEV)


def ws(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)


def report(name, **kv):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)
