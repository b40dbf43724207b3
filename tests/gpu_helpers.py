"""Shared helpers for the GPU parity tests (marshalling and comparisons only)."""
import sys

import numpy as np

# Tolerances (the bar the HIP path is held to against the oracle):
#  - int32 accumulators from identical int8 codes: bit-exact;
#  - bf16 outputs from identical codes and scales: bit-exact (same formula,
#    same fp32 operation order, RNE);
#  - int8 codes produced by the GPU's fp32 fast Walsh-Hadamard transform vs
#    the oracle's fp64 dense product: identical except at most 1 LSB on at
#    most 0.01 % of the elements (the two rotations round differently, which
#    can move a value across a rounding boundary);
#  - fp32 scales: within 4 ulp (absmax can differ by the same rounding);
#  - bf16 end-to-end outputs: relative L2 <= 1e-3.
CODE_MISMATCH_MAX_FRAC = 1e-4
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


def assert_codes_close(q_gpu, q_ref, what="codes"):
    assert q_gpu.shape == q_ref.shape, (q_gpu.shape, q_ref.shape)
    mx, frac = code_mismatch(q_gpu, q_ref)
    assert mx <= 1, f"{what}: max code difference {mx}"
    assert frac <= CODE_MISMATCH_MAX_FRAC, f"{what}: {frac:.3e} of codes differ"
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
