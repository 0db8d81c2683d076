"""Shared helpers of the GPU parity tests: device upload of stored bits and
the tolerance gates. No method arithmetic here."""

import numpy as np

# Gates (stated with the workloads): fp32 inputs -> 1e-4 relative; bf16 / fp8
# inputs -> O max-abs 2e-2 and LSE max-abs 1e-3, against the float64 oracle on
# the same stored bits.
F32_REL = 1e-4
LP_O_ABS = 2e-2
LP_LSE_ABS = 1e-3
# bf16 / fp8 inputs, in addition: per output row (all heads of one query),
# max|dO| <= 1e-2 * max|O_ref|. Long-context outputs are small (about
# 1/sqrt(keys)), so the absolute gate alone would pass an all-zero O. The
# kernels round each probability to bf16 before the PV product (relative
# error <= 2^-9, independent across keys) and a bf16 output once more
# (<= 2^-9 of the element): the row's largest error stays a few times
# 2^-9 / sqrt(3) of its largest element, about 1e-3 to 3e-3 measured;
# 1e-2 leaves that margin and fails any missing term or wrong row.
LP_O_ROW_REL = 1e-2


def row_rel_err(o, o_ref):
    """max over rows (first axis) of max|o - o_ref| / max|o_ref| on that row;
    a row whose reference is all zeros must be all zeros."""
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    if o.size == 0:
        return 0.0
    d = np.abs(o - o_ref).reshape(o.shape[0], -1).max(axis=1)
    r = np.abs(o_ref).reshape(o.shape[0], -1).max(axis=1)
    zero = r == 0
    if np.any(zero & (d > 0)):
        return float("inf")
    return float(np.max(np.where(zero, 0.0, d / np.where(zero, 1.0, r))))


def dev():
    import torch
    return torch.device("cuda:0")


def bf16_tensor(bits, device=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device or dev())


def f32_tensor(x, device=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device or dev())


def u8_tensor(x, device=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(device or dev())


def i32_tensor(x, device=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device or dev())


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def check_f32(o, lse, o_ref, lse_ref, what=""):
    """fp32 gate: max|dO| / max|O_ref| <= 1e-4; |dLSE| <= 1e-4 * max(1, |LSE|);
    -inf LSE must match exactly."""
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), what
    fin = np.isfinite(lse_ref)
    err_o = np.max(np.abs(o - o_ref)) / max(np.max(np.abs(o_ref)), 1e-30)
    err_l = np.max(np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))) if fin.any() else 0.0
    assert not np.any(np.isnan(o)), what
    assert not np.any(np.isnan(lse)), what
    assert row_rel_err(o, o_ref) <= 10 * F32_REL, what
    assert err_o <= F32_REL, f"{what}: O rel err {err_o:.3g}"
    assert err_l <= F32_REL, f"{what}: LSE rel err {err_l:.3g}"
    return err_o, err_l


def check_lowp(o, lse, o_ref, lse_ref, what=""):
    """bf16/fp8 gate: O max-abs <= 2e-2, LSE max-abs <= 1e-3, and per row
    max|dO| <= 1e-2 * max|O_ref| (LP_O_ROW_REL). Returns (O max-abs, LSE
    max-abs, largest row-relative O error)."""
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), what
    fin = np.isfinite(lse_ref)
    assert not np.any(np.isnan(o)), what
    assert not np.any(np.isnan(lse)), what
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    rel = row_rel_err(o, o_ref)
    assert err_o <= LP_O_ABS, f"{what}: O max-abs {err_o:.3g}"
    assert err_l <= LP_LSE_ABS, f"{what}: LSE max-abs {err_l:.3g}"
    assert rel <= LP_O_ROW_REL, f"{what}: O row-relative error {rel:.3g}"
    return err_o, err_l, rel


def check_lowp_scaled(o, lse, o_ref, lse_ref, what=""):
    """For extra cases whose values are not N(0,1)-sized (planted large keys,
    where in MLA the value is the key): the bf16 rounding of P is relative, so
    the O bound scales with max|O|: max-abs <= 2e-2 * max(1, max|O_ref|);
    LSE max-abs <= 1e-3 * max(1, max|LSE_ref|)."""
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), what
    assert not np.any(np.isnan(o)), what
    assert not np.any(np.isnan(lse)), what
    so = max(1.0, float(np.max(np.abs(o_ref))))
    sl = max(1.0, float(np.max(np.abs(lse_ref[fin])))) if fin.any() else 1.0
    err_o = float(np.max(np.abs(o - o_ref)))
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    rel = row_rel_err(o, o_ref)
    assert err_o <= LP_O_ABS * so, f"{what}: O max-abs {err_o:.3g} (scale {so:.3g})"
    assert err_l <= LP_LSE_ABS * sl, f"{what}: LSE max-abs {err_l:.3g} (scale {sl:.3g})"
    assert rel <= LP_O_ROW_REL, f"{what}: O row-relative error {rel:.3g}"
    return err_o, err_l
