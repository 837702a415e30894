"""Shared helpers for the GPU parity tests: numpy <-> device tensors and the comparison rules."""
import numpy as np

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> device torch.bfloat16."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def host(t):
    """Device tensor -> numpy (uint16 view for int16 / bfloat16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_codes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


REL_TOL = 1e-5  # fp32 accumulation against the exact dyadic products (sum |a b| scale, and normwise)


def assert_gemm_close(got, ref, absbound, what):
    """Per element |got - ref| <= 1e-5 * sum_k |a_k b_k| and normwise ||got - ref|| <= 1e-5 ||ref||."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    lim = REL_TOL * np.asarray(absbound, np.float64) + 1e-300
    bad = np.argwhere(err > lim)
    assert bad.size == 0, f"{what}: {len(bad)} entries outside 1e-5*sum|ab|, first {bad[:3].tolist()} err {err[tuple(bad[0])]} lim {lim[tuple(bad[0])]}"
    nref = np.linalg.norm(ref)
    if nref > 0:
        assert np.linalg.norm(got - ref) <= REL_TOL * nref, what


def assert_bf16_matches(got_bits, ref, absbound, what):
    """bf16 output equals the RNE rounding of the exact value, except where the exact value lies
    within the fp32 accumulation bound of a bf16 rounding boundary (then either neighbour is fine)."""
    got = bf16_to_f64(got_bits)
    ref = np.asarray(ref, np.float64)
    slack = REL_TOL * np.asarray(absbound, np.float64)
    lo = _round_bf16(ref - slack)
    hi = _round_bf16(ref + slack)
    ok = (got >= np.minimum(lo, hi)) & (got <= np.maximum(lo, hi))
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{what}: {len(bad)} bf16 mismatches, first {bad[:3].tolist()} got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"


def _round_bf16(v):
    v = np.asarray(v, np.float64)
    f, e = np.frexp(v)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)
