"""Test helpers: host/device conversions and the floating-point acceptance rules.

Acceptance for bf16 GEMM outputs (the workloads' stated bar): against the
oracle's unrounded float64 value, max |gpu - ref| <= 2e-2 and
||gpu - ref||_2 / ||ref||_2 <= 1e-2.  A tighter per-element bound derived from
the arithmetic is checked as well:

    |gpu - ref| <= half_ulp(out dtype, |ref|) + 1.2 * gamma_K * S + 1e-5 (1 + |ref|)

where S = sum_k |x_k w_k| (+ |b|) and gamma_K = K u / (1 - K u) with u = 2^-24
bounds fp32 accumulation in any order, 1.2 covers the GELU slope (|g'| < 1.13),
and the last term covers fp32 evaluation of the bias add and GELU.
"""
import numpy as np
import torch

U32 = 2.0 ** -24
MAX_ABS = 2e-2
MAX_REL_L2 = 1e-2


def bits_to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 GPU tensor (same bits)."""
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 / fp32 GPU tensor to float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def gamma(n, u=U32):
    return n * u / (1 - n * u)


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 8), 2.0 ** -134)


def half_ulp_f32(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 24), 2.0 ** -150)


def abs_dot(xbits: np.ndarray, wbits: np.ndarray, bias_bits=None) -> np.ndarray:
    """S = |x| @ |w|^T (+ |b|) in float64, for the accumulation-error bound."""
    import oracle
    s = np.abs(oracle.bf16_widen(xbits)) @ np.abs(oracle.bf16_widen(wbits)).T
    if bias_bits is not None:
        s = s + np.abs(oracle.bf16_widen(bias_bits))[None, :]
    return s


def check_close(gpu: np.ndarray, ref: np.ndarray, k: int, out_bf16: bool, S=None, what=""):
    """Apply the stated bar (max-abs, rel-L2) and, when S is given, the tight bound."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what
    err = np.abs(gpu - ref)
    max_abs = float(err.max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(gpu - ref)) / nref if nref > 0 else float(np.linalg.norm(gpu - ref))
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs} > {MAX_ABS}"
    assert rel <= MAX_REL_L2, f"{what}: rel L2 error {rel} > {MAX_REL_L2}"
    if S is not None:
        mag = np.maximum(np.abs(ref), np.abs(gpu))
        hu = half_ulp_bf16(mag) if out_bf16 else half_ulp_f32(mag)
        bound = hu + 1.2 * gamma(k + 2) * S + 1e-5 * (1 + np.abs(ref))
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the derived bound; "
                               f"worst excess {float((err - bound).max())}")
    return max_abs, rel


def sample_rows(m: int, n_random: int, seed: int, tile: int = 256) -> np.ndarray:
    """Rows 0, 1, m-1, every tile-boundary pair (t-1, t) and seeded random rows."""
    rows = {0, 1, m - 1}
    for t in range(tile, m, tile):
        rows.update((t - 1, t))
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, m, size=n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < m), dtype=np.int64)


def check_swiglu(gpu, x_bits, w_bits, b_bits, out_bf16, rows=None, what=""):
    """SwiGLU output against the oracle.

    The pre-rounding error E of each element is bounded by propagating the two halves'
    accumulation errors E_g, E_u (as in check_close): 1.1 E_g (|u| + E_u) + |silu(g)| E_u,
    since |silu'| <= 1.1, plus the fp32 evaluation of silu and of the product (a few ulp).
    The stated bar is then applied to the reference mirror-rounded to the output dtype:
    with bf16 output, wherever no bf16 rounding boundary lies within E of the reference,
    the GPU's value must round to the same bf16 value (|gpu - bf16(ref)| = 0).  Where one
    does (a reference next to a rounding boundary, or a tiny one whose E spans several
    output steps), more than one output value is correct, and the element is held to
    |gpu - ref| <= E + half an output ulp, which every element must satisfy.  rel-L2 is
    taken against the unrounded reference."""
    import oracle
    n = w_bits.shape[0] // 2
    xs = x_bits if rows is None else x_bits[rows]
    k = x_bits.shape[1]
    bg = bu = None
    if b_bits is not None:
        bg, bu = b_bits[:n], b_bits[n:]
    ref = oracle.colwise_swiglu(x_bits, w_bits, b_bits, rows=rows)
    g = oracle.linear(x_bits, np.ascontiguousarray(w_bits[:n]), bg, rows=rows)
    u = oracle.linear(x_bits, np.ascontiguousarray(w_bits[n:]), bu, rows=rows)
    e_g = 1.2 * gamma(k + 2) * abs_dot(xs, w_bits[:n], bg) + 1e-6
    e_u = 1.2 * gamma(k + 2) * abs_dot(xs, w_bits[n:], bu) + 1e-6
    with np.errstate(over="ignore"):
        sg = np.abs(g / (1.0 + np.exp(-g)))
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape and np.all(np.isfinite(gpu)), what
    err = np.abs(gpu - ref)
    mag = np.maximum(np.abs(ref), np.abs(gpu))
    hu = half_ulp_bf16(mag) if out_bf16 else half_ulp_f32(mag)
    e_pre = 1.1 * e_g * (np.abs(u) + e_u) + sg * e_u + 8 * U32 * mag + 1e-7
    if out_bf16:
        ref_r = oracle.bf16_widen(oracle.bf16_round(ref))
        decided = (oracle.bf16_widen(oracle.bf16_round(ref - e_pre)) == ref_r) & \
                  (oracle.bf16_widen(oracle.bf16_round(ref + e_pre)) == ref_r)
        err_r = np.abs(gpu - ref_r)
        wrong = decided & (err_r != 0)
        assert not wrong.any(), (f"{what}: {int(wrong.sum())} outputs rounded differently from the "
                                 f"mirror-rounded reference, worst {float(err_r[wrong].max())}")
    else:
        max_abs = float(err.max()) if err.size else 0.0
        assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs} > {MAX_ABS}"
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(gpu - ref)) / nref if nref > 0 else float(np.linalg.norm(gpu - ref))
    assert rel <= MAX_REL_L2, f"{what}: rel L2 error {rel} > {MAX_REL_L2}"
    bad = err > hu + e_pre
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the derived SwiGLU bound; "
                           f"worst excess {float((err - hu - e_pre).max())}")
