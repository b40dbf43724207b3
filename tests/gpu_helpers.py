"""Shared helpers for the GPU parity tests (marshalling and comparisons only)."""
import sys

import numpy as np

# Tolerances (the bar the HIP path is held to against the oracle):
#  - int32 accumulators from identical int8 codes: bit-exact;
#  - bf16 outputs from identical codes and scales: bit-exact (same formula,
#    same fp32 operation order, RNE);
#  - int8 codes produced by the GPU's fp32 fast Walsh-Hadamard transform and
#    fp32 quotient vs the oracle's exact fp64 rotation and fp64 quotient:
#    identical except at most 1 LSB on at most 0.01 % of the elements (the
#    fp32 roundings can move a value across a rounding boundary);
#  - on small structured rows, where 0.01 % is less than one element: codes
#    identical except where the oracle's exact quotient lies within 2^-12 of
#    a rounding boundary n + 1/2 (there they may differ by one);
#  - int4 clip choice: the oracle's error at the GPU's candidate within a
#    near-tie bound of the oracle's minimum (see assert_clip_choice);
#  - fp32 scales: within 4 ulp (absmax can differ by the same rounding);
#  - bf16 end-to-end outputs: relative L2 <= 1e-3.
CODE_MISMATCH_MAX_FRAC = 1e-4
NEAR_TIE = 2.0 ** -12
SCALE_RTOL = 4 * 2.0 ** -23
REL_L2_MAX = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def to_dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_to_dev(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(t.bfloat16)


def bf16_from_dev(x):
    t = torch()
    return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def code_mismatch(q_gpu, q_ref):
    d = q_gpu.astype(np.int16) - q_ref.astype(np.int16)
    return (int(np.abs(d).max()) if d.size else 0), (np.count_nonzero(d) / max(d.size, 1))


def assert_codes_close(q_gpu, q_ref, what="codes", q_exact=None):
    """At most 1 LSB apart, on at most 0.01 % of the elements (counted as at
    most max(1, 1e-4 n), so that a single rounding tie in a small test does
    not fail it); with the oracle's exact quotients at hand, every differing
    code must also sit at a rounding boundary (assert_codes_off_ties)."""
    assert q_gpu.shape == q_ref.shape, (q_gpu.shape, q_ref.shape)
    mx, frac = code_mismatch(q_gpu, q_ref)
    assert mx <= 1, f"{what}: max code difference {mx}"
    n_diff = int(round(frac * q_gpu.size))
    assert n_diff <= max(1, CODE_MISMATCH_MAX_FRAC * q_gpu.size), f"{what}: {frac:.3e} of codes differ ({n_diff})"
    if q_exact is not None:
        assert_codes_off_ties(q_gpu, q_ref, q_exact, what)
    return frac


def assert_scales_close(s_gpu, s_ref, what="scales"):
    s_gpu = s_gpu.astype(np.float64)
    s_ref = s_ref.astype(np.float64)
    zero = s_ref == 0
    assert np.all(s_gpu[zero] == 0), f"{what}: zero rows must get scale 0"
    rel = np.abs(s_gpu[~zero] - s_ref[~zero]) / s_ref[~zero]
    assert rel.size == 0 or rel.max() <= SCALE_RTOL, f"{what}: max rel diff {rel.max():.3e}"


def rel_l2(y_gpu_bits, y_ref_bits):
    a = bf16_bits_to_f64(y_gpu_bits)
    b = bf16_bits_to_f64(y_ref_bits)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def assert_rel_l2(y_gpu_bits, y_ref_bits, what="y"):
    r = rel_l2(y_gpu_bits, y_ref_bits)
    assert r <= REL_L2_MAX, f"{what}: relative L2 {r:.3e}"
    return r


def exact_quotients(x_f64, scales, group):
    """The oracle's exact rotated rows (fp64 dense product) divided by the
    stored fp32 scales, in fp64: the values the oracle's codes round."""
    import oracle
    rot = oracle.rotate_rows(np.asarray(x_f64, dtype=np.float64), group)
    s = np.asarray(scales, dtype=np.float64)
    return rot / np.where(s == 0, 1.0, s)[:, None]


def assert_codes_off_ties(q_gpu, q_ref, q_exact, what="codes"):
    """Codes equal the oracle's except where the exact quotient lies within
    NEAR_TIE of a rounding boundary n + 1/2, where they may differ by one
    (the GPU rotates and divides in fp32, which can land a value on the
    other side of such a boundary).  Returns the number of codes that differ."""
    assert q_gpu.shape == q_ref.shape == q_exact.shape
    d = q_gpu.astype(np.int16) - q_ref.astype(np.int16)
    a = np.abs(q_exact)
    near = np.abs(a - np.floor(a) - 0.5) <= NEAR_TIE
    assert np.abs(d).max(initial=0) <= 1, f"{what}: a code differs by more than one"
    bad = (d != 0) & ~near
    assert not bad.any(), f"{what}: {int(bad.sum())} codes differ away from a rounding boundary"
    return int(np.count_nonzero(d))


# Near-tie bound of the int4 clip choice.  Each candidate's error e(c) =
# sum_k (q_k s - v_k)^2 is continuous in the rotated row v and the scale s.
# The GPU evaluates it (in fp64) on its fp32 rotation and on scales taken from
# its fp32 absmax; with those within eta * |v|_2 (eta = 2^-20, sixteen fp32
# ulps of the row norm) the two evaluations of one candidate differ by at most
# about 4 eta sqrt(e) |v|_2, so a choice can flip only between candidates whose
# exact errors differ by twice that.  The bound below is 2^-16 sqrt(e) |v|_2,
# a factor two above it.
CLIP_TIE_FACTOR = 2.0 ** -16


def assert_clip_choice(ci_gpu, errors, rot_norm, what="clip index", max_frac=0.01):
    """int4 clip search: the GPU's candidate per row is the oracle's argmin,
    or a near tie with it: errors[n, ci_gpu[n]] - min_c errors[n, c] <=
    CLIP_TIE_FACTOR * sqrt(errors[n, ci_gpu[n]]) * |rotated row n|_2.  Rows
    off the argmin must stay rare (at most max_frac of them)."""
    n = np.arange(errors.shape[0])
    e_gpu = errors[n, ci_gpu]
    e_min = errors.min(axis=1)
    slack = e_gpu - e_min
    off = ci_gpu != errors.argmin(axis=1)
    assert off.mean() <= max_frac, f"{what}: {int(off.sum())} rows off the argmin"
    bound = CLIP_TIE_FACTOR * np.sqrt(e_gpu) * rot_norm
    bad = slack > bound
    assert not bad.any(), (f"{what}: rows {np.nonzero(bad)[0][:8].tolist()} are not near ties "
                           f"(slack {slack[bad][:4]}, bound {bound[bad][:4]})")
    return int(off.sum())
