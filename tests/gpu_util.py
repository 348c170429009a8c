"""Helpers for the GPU parity tests (comparison rules, device buffers)."""
import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
NEAR_TIE = 1e-6   # decisions whose oracle margin is below this are reported, not failed


def close(g, o, rel=1e-3, floor=1e-3):
    """|g - o| <= rel * max(|o|, floor * rms(o)) element-wise (finite
    entries); non-finite entries must agree exactly."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    fin = np.isfinite(o)
    assert np.array_equal(fin, np.isfinite(g)), "finite pattern differs"
    assert np.array_equal(g[~fin], o[~fin]), "non-finite entries differ"
    if not fin.any():
        return 0.0
    rms = np.sqrt(np.mean(o[fin] ** 2))
    bound = rel * np.maximum(np.abs(o[fin]), floor * rms)
    err = np.abs(g[fin] - o[fin])
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"max error / bound = {worst:.3g}"
    return worst


U32 = 2.0 ** -24   # unit roundoff of fp32 (round to nearest)


def conv_error_bound(x, x_prev, w, base=None, group: int = 16) -> np.ndarray:
    """Element-wise bound on |y_fp32 - y_exact| for the two-tap dynamic
    convolution y_t = (base0 + c_t[g]) x_t + (base1 + c_t[G+g]) x_{t-1},
    c_t = W x_t, derived from the fp32 arithmetic alone:
      * each tap c = sum_i w_i x_i has bf16 factors, so every product is exact
        in fp32 and the sum, in any order or blocking, is within
        gamma_d * sum_i |w_i x_i|, gamma_d = d u / (1 - d u) (the standard
        forward bound of a floating-point sum, Higham, Accuracy and Stability
        of Numerical Algorithms, Thm. 3.1);
      * the base add, the two products, their sum, the final rounding and the
        oracle's own rounding to fp32 add at most 5 u (|k0 x_t| + |k1 x_{t-1}|).
    Bug-sized errors stay far outside it: a dropped 64-wide K block moves a
    tap by ~sqrt(64/d) |c|, about 7x the bound at d = 5120, and a wrong
    channel-to-group map or sign moves it by ~|c|."""
    xf = np.asarray(x.float().numpy() if hasattr(x, "float") else x, np.float64)
    wf = np.asarray(w.float().numpy() if hasattr(w, "float") else w, np.float64)
    B, L, d = xf.shape
    G = d // group
    if x_prev is None:
        pf = np.zeros((B, d))
    else:
        pf = np.asarray(x_prev.float().numpy() if hasattr(x_prev, "float") else x_prev, np.float64)
    xm1 = np.concatenate([pf[:, None, :], xf[:, :-1, :]], axis=1)
    c = xf @ wf.T                                 # [B, L, 2G]
    s = np.abs(xf) @ np.abs(wf).T                 # sum |w_i x_i|
    gam = d * U32 / (1 - d * U32)
    ch = np.arange(d) // group
    c0, c1 = c[..., ch], c[..., G + ch]
    dc0, dc1 = gam * s[..., ch], gam * s[..., G + ch]
    if base is not None:
        bf = np.asarray(base.numpy() if hasattr(base, "numpy") else base, np.float64)
        c0 = c0 + bf[0]
        c1 = c1 + bf[1]
    t0, t1 = np.abs(c0 * xf), np.abs(c1 * xm1)
    return dc0 * np.abs(xf) + dc1 * np.abs(xm1) + 5 * U32 * (t0 + t1)


def gemm_error_bound(x, w) -> np.ndarray:
    """Element-wise bound on |fp32 (x w^T) - exact| for bf16 x [n, d] and w
    [m, d]: every product of two bf16 values is exact in fp32, so a sum of d
    of them, in any order or blocking, is within gamma_d * sum_i |x_i w_i|,
    gamma_d = d u / (1 - d u) (Higham, Accuracy and Stability of Numerical
    Algorithms, Thm. 3.1)."""
    xf = np.asarray(x.float().numpy() if hasattr(x, "float") else x, np.float64)
    wf = np.asarray(w.float().numpy() if hasattr(w, "float") else w, np.float64)
    d = xf.shape[-1]
    return d * U32 / (1 - d * U32) * (np.abs(xf) @ np.abs(wf).T)


def conv_close(g, o, bound) -> float:
    """fp32 conv output within the arithmetic bound of conv_error_bound."""
    g = np.asarray(g, np.float64)
    err = np.abs(g - np.asarray(o, np.float64))
    worst = float(np.max(err / np.maximum(bound, np.finfo(np.float64).tiny)))
    assert worst <= 1.0, f"max error / bound = {worst:.3g}"
    return worst


def bf16_ulp_close(g_bf16: torch.Tensor, o_f32: np.ndarray, bound: np.ndarray, ulps: int = 1):
    """bf16 output against the float oracle: within `ulps` bf16 steps (at the
    oracle's magnitude) plus the fp32 arithmetic bound `bound` (the bf16 value
    is the round-to-nearest of an fp32 result that is itself within `bound`).
    Returns the largest error in bf16 steps (for the report)."""
    o = np.asarray(o_f32, np.float64)
    g = g_bf16.detach().float().cpu().numpy().astype(np.float64)
    mag = np.maximum(np.abs(o), np.finfo(np.float32).tiny)
    step = np.exp2(np.floor(np.log2(mag)) - 7)          # bf16 spacing at |o|
    err = np.abs(g - o)
    assert np.all(err <= ulps * step + bound), \
        f"max error / bound = {float(np.max(err / (ulps * step + bound))):.3g}"
    return float(np.max(err / step))


def _f64(a):
    return np.asarray(a.float().numpy() if hasattr(a, "float") else a, np.float64)


def conv_term_scale(x, x_prev, w, base=None, group: int = 16, tap_floor: float = 1e-2) -> np.ndarray:
    """Per-element magnitude of the two terms of the two-tap convolution
    ("DFlash 2: Keep Drafting Parallel", section "A lightweight local
    convolution", eq. Conv_k: y_t = k0 (.) x_t + k1 (.) x_{t-1}), from the
    exact (float64) taps k0 = base0 + c_t[g], k1 = base1 + c_t[G+g],
    c_t = W x_t:   max(|k0|, f0) |x_t| + max(|k1|, f1) |x_{t-1}|.
    The 1e-3 relative tolerance of the conv outputs is taken against this
    sum, not against |y|: the two terms may cancel, and no fp32 evaluation
    can then hold 1e-3 of |y|.  A tap is itself a sum of d products and can
    cancel to near zero, where no fp32 sum holds 1e-3 of it either; its
    magnitude is floored at f = tap_floor x the rms of that tap over the
    site (f0 for k0, f1 for k1): a tap under 1 % of the typical tap is held
    to 1e-5 of the typical tap in absolute terms.  A plain fp32 split-K sum
    of the exact bf16 products (any order; its tap errors reach ~1.5e-6 at
    d = 5120, rms tap 1.4) stays under 0.05 of this allowance on a
    batch-4, block-16, d = 5120 site; taps built from bf16-rounded partial
    sums fail it on about half the elements, by up to ~370-fold
    (tests/test_parity_rules.py)."""
    xf, wf = _f64(x), _f64(w)
    B, L, d = xf.shape
    G = d // group
    pf = np.zeros((B, d)) if x_prev is None else _f64(x_prev)
    xm1 = np.concatenate([pf[:, None, :], xf[:, :-1, :]], axis=1)
    c = xf @ wf.T                                  # [B, L, 2G]
    ch = np.arange(d) // group
    k0, k1 = c[..., ch], c[..., G + ch]
    if base is not None:
        bf = _f64(base.numpy() if hasattr(base, "numpy") else base)
        k0 = k0 + bf[0]
        k1 = k1 + bf[1]
    f0 = tap_floor * np.sqrt(np.mean(k0 ** 2))
    f1 = tap_floor * np.sqrt(np.mean(k1 ** 2))
    return np.maximum(np.abs(k0), f0) * np.abs(xf) + np.maximum(np.abs(k1), f1) * np.abs(xm1)


def conv_rel_close(g, o, scale, rel: float = 1e-3) -> float:
    """fp32 conv output: |g - o| <= rel * scale element-wise (scale from
    conv_term_scale).  Returns the largest error / allowance."""
    err = np.abs(np.asarray(g, np.float64) - np.asarray(o, np.float64))
    worst = float(np.max(err / (rel * scale)))
    assert worst <= 1.0, f"max error / (1e-3 x term magnitude) = {worst:.3g}"
    return worst


def conv_rel_close_bf16(g_bf16, o_f32, scale, rel: float = 1e-3, ulps: int = 1) -> float:
    """bf16 conv output: within `ulps` bf16 steps (at the oracle's magnitude)
    of the oracle, plus the fp32 allowance rel * scale (the bf16 value is the
    round-to-nearest of an fp32 result that must meet that allowance).
    Returns the largest error in bf16 steps."""
    o = np.asarray(o_f32, np.float64)
    g = g_bf16.detach().float().cpu().numpy().astype(np.float64) if hasattr(g_bf16, "detach") \
        else np.asarray(g_bf16, np.float64)
    mag = np.maximum(np.abs(o), np.finfo(np.float32).tiny)
    step = np.exp2(np.floor(np.log2(mag)) - 7)          # bf16 spacing at |o|
    err = np.abs(g - o)
    allow = ulps * step + rel * scale
    assert np.all(err <= allow), f"max error / allowance = {float(np.max(err / allow)):.3g}"
    return float(np.max(err / step))


def dev(x):
    return x.to(DEV) if isinstance(x, torch.Tensor) else torch.as_tensor(x).to(DEV)


def ws(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)


def report(name, **kv):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)
