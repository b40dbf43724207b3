"""Pins for the CPU oracle: closed forms, library routines, brute force.

Every check here compares the oracle with something other than itself:
scipy's Sylvester Hadamard, numpy/torch arithmetic written independently,
hand-derived worked examples (tests/golden), and invariants the definitions
fix.  A plausible slip in the oracle (a dropped 1/16, a transposed or
permuted Hadamard, half-to-even rounding, a wrong scale divisor, a swapped
nibble order, a wrong epilogue order or rounding) fails at least one test.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg
from hypothesis import given, settings, strategies as st

from w8a8_quantized_linear_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16(x):
    return wl.float_to_bf16_bits(np.asarray(x, dtype=np.float32))


def ref_rotate(x64, g):
    """Independent rotation: scipy's Sylvester matrix, numpy product per group."""
    H = scipy.linalg.hadamard(g).astype(np.float64) / np.sqrt(g)
    rows, K = x64.shape
    return (x64.reshape(rows, K // g, g) @ H).reshape(rows, K)


def ref_half_away(v):
    """Round half away from zero in fp64, exactly: v - trunc(v) is exact for
    |v| < 2^52, so the comparison with 1/2 is too (floor(|v| + 0.5) would
    misround 0.49999999999999994)."""
    v = np.asarray(v, dtype=np.float64)
    t = np.trunc(v)
    return t + np.sign(v) * (np.abs(v - t) >= 0.5)


def ref_quant_rows(rot64, qmax=127):
    """Per-row symmetric quantization of fp64 rotated rows, independent numpy
    formulation of the plain definition: fp64 absmax, the scale rounded once
    to fp32, codes decided on the fp64 quotient."""
    rot64 = np.asarray(rot64, dtype=np.float64)
    amax = np.abs(rot64).max(axis=1)
    s = (amax / qmax).astype(np.float32)                    # fp64 divide, one rounding to fp32
    safe = np.where(s == 0, np.float32(1), s).astype(np.float64)
    q = np.clip(ref_half_away(rot64 / safe[:, None]), -qmax, qmax)
    q[s == 0] = 0
    return q.astype(np.int8), s


# ------------------------------------------------------------------ Hadamard

@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_scipy_sylvester(oracle_mod, g):
    H = oracle_mod.hadamard(g)
    ref = scipy.linalg.hadamard(g).astype(np.float64) / np.sqrt(g)
    assert np.array_equal(H, ref)


def test_hadamard_orthogonal_bit_exact(oracle_mod):
    H = oracle_mod.hadamard(256)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, np.eye(256))
    H32 = H.astype(np.float32)
    assert np.array_equal(H32 @ H32.T, np.eye(256, dtype=np.float32))
    assert set(np.unique(np.abs(H))) == {1.0 / 16}


def test_rotation_matches_blockwise_library_product(oracle_mod):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 768))
    out = oracle_mod.rotate_rows(x, 256)
    ref = ref_rotate(x, 256)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_rotation_groups_are_contiguous(oracle_mod):
    # A value in group 1 must not leak into groups 0 or 2.
    x = np.zeros((1, 768))
    x[0, 256 + 3] = 1.0
    out = oracle_mod.rotate_rows(x, 256)
    assert np.all(out[0, :256] == 0) and np.all(out[0, 512:] == 0)
    assert np.all(np.abs(out[0, 256:512]) == 1.0 / 16)


def test_float_identity_xR_WR_equals_xW(oracle_mod):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((6, 512))
    w = rng.standard_normal((9, 512))
    lhs = oracle_mod.rotate_rows(x, 256) @ oracle_mod.rotate_rows(w, 256).T
    rhs = x @ w.T
    assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-13


def test_rotation_one_hot_closed_form(oracle_mod):
    for i in (0, 1, 37, 128, 255):
        x = np.zeros((1, 256))
        x[0, i] = 1.0
        out = oracle_mod.rotate_rows(x, 256)[0]
        j = np.arange(256)
        signs = np.array([(-1) ** bin(i & jj).count("1") for jj in j], dtype=np.float64)
        assert np.array_equal(out, signs / 16)


def test_rotation_constant_group_closed_form(oracle_mod):
    x = np.full((1, 256), 0.75)
    out = oracle_mod.rotate_rows(x, 256)[0]
    assert out[0] == 12.0 and np.all(out[1:] == 0)


# ------------------------------------------------------- int8 quantization

def test_worked_one_hot(oracle_mod):
    ex = golden("worked_examples.json")["one_hot"]
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, ex["index"]] = 1.0
    xq, s = oracle_mod.rotate_quant(bf16(x), ex["group"])
    assert s[0].view(np.uint32) == int(ex["scale_bits_hex"], 16)
    assert np.all(np.abs(xq) == ex["code_magnitude"])
    j = np.arange(256)
    signs = np.array([(-1) ** bin(ex["index"] & jj).count("1") for jj in j])
    assert np.array_equal(np.sign(xq[0]), signs)


def test_worked_constant_group(oracle_mod):
    ex = golden("worked_examples.json")["constant_group"]
    x = np.full((1, 256), ex["value"], dtype=np.float32)
    xq, s = oracle_mod.rotate_quant(bf16(x), ex["group"])
    assert s[0].view(np.uint32) == int(ex["scale_bits_hex"], 16)
    expect = np.zeros(256, dtype=np.int8)
    for idx, code in ex["codes_nonzero"]:
        expect[idx] = code
    assert np.array_equal(xq[0], expect)


def test_worked_half_away_ties_rotated(oracle_mod):
    ex = golden("worked_examples.json")["half_away_ties"]
    v = np.zeros(256)
    for k, val in ex["rotated"].items():
        v[int(k)] = val
    H = scipy.linalg.hadamard(256) / 16.0
    x = v @ H
    xb = bf16(x)
    assert np.array_equal(wl.bf16_bits_to_float(xb).astype(np.float64), x)  # exact in bf16
    xq, s = oracle_mod.rotate_quant(xb[None, :], 256)
    assert s[0] == ex["scale"]
    expect = np.zeros(256, dtype=np.int8)
    for idx, code in ex["codes_nonzero"]:
        expect[idx] = code
    assert np.array_equal(xq[0], expect)


def test_worked_identity_group_ties(oracle_mod):
    ex = golden("worked_examples.json")["identity_group_ties"]
    xq, s = oracle_mod.rotate_quant(bf16(np.array([ex["x"]])), ex["group"])
    assert s[0] == ex["scale"]
    assert xq[0].tolist() == ex["codes"]


def test_worked_quotient_decided_in_fp64(oracle_mod):
    ex = golden("worked_examples.json")["quotient_decided_in_fp64"]
    w = np.array([[int(h, 16) for h in ex["w_bits_hex"]]], dtype=np.uint32).view(np.float32)
    wq, ws = oracle_mod.quantize_weight_i8(w, ex["group"])
    assert ws[0].view(np.uint32) == int(ex["scale_bits_hex"], 16)
    assert wq[0].tolist() == ex["codes"]


def test_worked_rotation_kept_in_fp64(oracle_mod):
    ex = golden("worked_examples.json")["rotation_kept_in_fp64"]
    xb = bf16(np.array([ex["x"]]))
    assert np.array_equal(wl.bf16_bits_to_float(xb)[0].astype(np.float64), np.array(ex["x"]))  # exact in bf16
    xq, s = oracle_mod.rotate_quant(xb, ex["group"])
    assert s[0] == ex["scale"]
    assert xq[0].tolist() == ex["codes"]


def test_zero_row(oracle_mod):
    xq, s = oracle_mod.rotate_quant(np.zeros((2, 512), dtype=np.uint16), 256)
    assert np.all(s == 0) and np.all(xq == 0)
    wq, ws = oracle_mod.quantize_weight_i8(np.zeros((3, 256), dtype=np.float32), 256)
    assert np.all(ws == 0) and np.all(wq == 0)


def _rand_bf16(rng, M, K, outliers=0):
    x = rng.standard_normal((M, K)).astype(np.float32)
    if outliers:
        x[:, rng.choice(K, outliers, replace=False)] *= 20
    return bf16(x)


def test_codes_range_and_absmax_code(oracle_mod):
    rng = np.random.default_rng(3)
    xb = _rand_bf16(rng, 64, 1024, outliers=10)
    xq, s = oracle_mod.rotate_quant(xb, 256)
    assert xq.min() >= -127 and xq.max() <= 127
    assert np.all(np.abs(xq.astype(np.int32)).max(axis=1) == 127)
    assert s.dtype == np.float32 and s.shape == (64,)


def test_scale_is_absmax_over_127(oracle_mod):
    rng = np.random.default_rng(4)
    xb = _rand_bf16(rng, 32, 768, outliers=7)
    _, s = oracle_mod.rotate_quant(xb, 256)
    rot = ref_rotate(wl.bf16_bits_to_float(xb).astype(np.float64), 256)
    amax = np.abs(rot).max(axis=1)
    assert np.array_equal(s, (amax / 127.0).astype(np.float32))


def test_scale_invariance_power_of_two(oracle_mod):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    q1, s1 = oracle_mod.rotate_quant(bf16(x), 256)
    q2, s2 = oracle_mod.rotate_quant(bf16(x * 8.0), 256)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(8))


@settings(max_examples=40, deadline=None)
@given(M=st.integers(1, 4), G=st.integers(1, 2), seed=st.integers(0, 2**31 - 1),
       outliers=st.integers(0, 5), scale_exp=st.integers(-6, 6))
def test_rotate_quant_brute_force_tiny(oracle_mod, M, G, seed, outliers, scale_exp):
    rng = np.random.default_rng(seed)
    K = 256 * G
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(2.0 ** scale_exp)
    if outliers:
        x[:, rng.choice(K, outliers, replace=False)] *= 20
    xb = bf16(x)
    xq, s = oracle_mod.rotate_quant(xb, 256)
    rot = ref_rotate(wl.bf16_bits_to_float(xb).astype(np.float64), 256)
    q_ref, s_ref = ref_quant_rows(rot)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(xq, q_ref)


@settings(max_examples=25, deadline=None)
@given(N=st.integers(1, 8), G=st.integers(1, 2), seed=st.integers(0, 2**31 - 1))
def test_quantize_weight_i8_brute_force_tiny(oracle_mod, N, G, seed):
    rng = np.random.default_rng(seed)
    K = 256 * G
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, ws = oracle_mod.quantize_weight_i8(w, 256)
    rot = ref_rotate(w.astype(np.float64), 256)
    q_ref, s_ref = ref_quant_rows(rot)
    assert np.array_equal(ws, s_ref)
    assert np.array_equal(wq, q_ref)
    assert ws.dtype == np.float32 and ws.shape == (N,)  # one fp32 scale per output row


def test_group_one_is_plain_rowwise(oracle_mod):
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    wq, ws = oracle_mod.quantize_weight_i8(w, 1)
    q_ref, s_ref = ref_quant_rows(w.astype(np.float64))
    assert np.array_equal(wq, q_ref) and np.array_equal(ws, s_ref)


def test_invalid_arguments_rejected(oracle_mod):
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.rotate_quant(np.zeros((1, 300), dtype=np.uint16), 256)   # K % 256
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.rotate_quant(np.zeros((1, 384), dtype=np.uint16), 384)   # not a power of two


# ---------------------------------------------------------------- the GEMM

@settings(max_examples=25, deadline=None)
@given(M=st.integers(1, 6), N=st.integers(1, 9), K=st.integers(1, 300), seed=st.integers(0, 2**31 - 1))
def test_gemm_exact_vs_int64_matmul(oracle_mod, M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, (M, K), dtype=np.int8)
    b = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = oracle_mod.gemm_i8(a, b)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)


def test_gemm_extremes_and_overflow_guard(oracle_mod):
    K = 12288
    a = np.full((2, K), 127, dtype=np.int8)
    a[1] = -127
    b = np.full((3, K), -127, dtype=np.int8)
    acc = oracle_mod.gemm_i8(a, b)
    assert acc[0, 0] == -127 * 127 * K and acc[1, 2] == 127 * 127 * K
    K_big = 140000  # 127^2 * K > 2^31 - 1
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.gemm_i8(np.full((1, K_big), 127, np.int8), np.full((1, K_big), 127, np.int8))


def test_epilogue_vs_torch_bf16_cast():
    import torch
    import oracle
    rng = np.random.default_rng(7)
    acc = rng.integers(-3_000_000, 3_000_000, (17, 23)).astype(np.int32)
    xs = (rng.random(17) * 0.1).astype(np.float32)
    ws = (rng.random(23) * 0.001).astype(np.float32)
    y = oracle.epilogue(acc, xs, ws)
    prod = (acc.astype(np.float32) * xs[:, None]).astype(np.float32) * ws[None, :]
    ref = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def test_epilogue_order_and_bf16_ties():
    import oracle
    # acc * xs is exact here; the product with ws lands on bf16 ties.
    acc = np.array([[1, 3]], dtype=np.int32)
    xs = np.array([1.0], dtype=np.float32)
    tie_even = np.array([0x3F808000], dtype=np.uint32).view(np.float32)[0]  # 1.00390625: tie, round down
    tie_odd = np.array([0x3F818000], dtype=np.uint32).view(np.float32)[0]   # tie, round up
    y = oracle.epilogue(np.array([[1, 1]], dtype=np.int32), xs, np.array([tie_even, tie_odd], np.float32))
    assert y[0].tolist() == [0x3F80, 0x3F82]
    # large accumulators convert to fp32 with round-to-nearest-even
    big = np.array([[16777217]], dtype=np.int32)  # 2^24 + 1 -> 2^24
    y = oracle.epilogue(big, xs, np.array([1.0], np.float32))
    assert y[0, 0] == 0x4B80  # 2^24 in bf16
    del acc


def _bf16_round(v):
    import torch
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_epilogue_multiplies_token_scale_first():
    """Reading: ((float)acc * x_scale) * w_scale.  Search for triples where the
    other association rounds to a different bf16 value and check the oracle
    follows the stated order on every one of them."""
    import oracle
    rng = np.random.default_rng(77)
    n = 1 << 22
    a = rng.integers(-2_000_000, 2_000_000, n).astype(np.int32)
    xs = (rng.random(n) * 0.05 + 1e-3).astype(np.float32)
    ws = (rng.random(n) * 0.002 + 1e-5).astype(np.float32)
    af = a.astype(np.float32)
    first = (af * xs).astype(np.float32) * ws
    other = af * (xs * ws).astype(np.float32)
    hit = np.nonzero(_bf16_round(first) != _bf16_round(other))[0][:64]
    assert hit.size >= 8
    for i in hit:
        y = oracle.epilogue(a[i:i + 1].reshape(1, 1), xs[i:i + 1], ws[i:i + 1])
        assert y[0, 0] == _bf16_round(first[i:i + 1])[0]


# ----------------------------------------------------------- end to end

def test_w8a8_composition(oracle_mod):
    rng = np.random.default_rng(8)
    xb = _rand_bf16(rng, 12, 512, outliers=4)
    w = (rng.standard_normal((20, 512)) * 0.02).astype(np.float32)
    wq, ws = oracle_mod.quantize_weight_i8(w, 256)
    y = oracle_mod.w8a8_linear(xb, wq, ws, 256)
    xq, xs = oracle_mod.rotate_quant(xb, 256)
    acc = xq.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(y, oracle_mod.epilogue(acc.astype(np.int32), xs, ws))


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_rotation_suppresses_outlier_error(oracle_mod):
    """Behaviour the pages claim ('Why ConvRot'): with 1 % outlier channels the
    rotated W8A8 output is several times closer to the exact product than
    plain row-wise int8 (group 1)."""
    M, K, N = 64, 4096, 256
    x = wl.make_activations(M, K, 41, seed=21)
    w = wl.make_weight(N, K, seed=21)
    exact = wl.bf16_bits_to_float(x).astype(np.float64) @ w.astype(np.float64).T
    errs = {}
    for g in (256, 1):
        wq, ws = oracle_mod.quantize_weight_i8(w, g)
        y = wl.bf16_bits_to_float(oracle_mod.w8a8_linear(x, wq, ws, g)).astype(np.float64)
        errs[g] = _rel_l2(y, exact)
    assert errs[256] < 0.02, errs
    assert errs[1] > 0.035, errs
    assert errs[1] > 3 * errs[256], errs


# ------------------------------------------------------------------- int4

def ref_unpack(b):
    b = np.asarray(b, dtype=np.int16)
    lo = ((b & 0xF) ^ 8) - 8
    hi = (((b >> 4) & 0xF) ^ 8) - 8
    return lo, hi


def test_unpack_all_256_bytes(oracle_mod):
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = oracle_mod.unpack_i4(b)
    lo, hi = ref_unpack(b[0])
    assert np.array_equal(q[0, 0::2], lo) and np.array_equal(q[0, 1::2], hi)
    assert q.min() == -8 and q.max() == 7


def test_worked_nibble_order(oracle_mod):
    ex = golden("worked_examples.json")["int4_nibble_order"]
    q = oracle_mod.unpack_i4(np.array([ex["bytes"]], dtype=np.uint8))
    assert q[0].reshape(-1, 2).tolist() == ex["pairs"]


def test_worked_int4_equal_magnitude(oracle_mod):
    ex = golden("worked_examples.json")["int4_equal_magnitude_row"]
    rng = np.random.default_rng(9)
    a = ex["magnitude"]
    w = (np.where(rng.random((3, 64)) < 0.5, -a, a)).astype(np.float32)
    wq4, s, ci = oracle_mod.quantize_weight_i4(w, ex["group"])
    assert np.all(ci == ex["clip_index"])
    assert np.all(s == np.float32(a * 100 / 700))
    q = oracle_mod.unpack_i4(wq4)
    assert np.all(np.abs(q) == 7)
    assert np.array_equal(np.sign(q), np.sign(w).astype(np.int8))


def _ref_int4_row(rot_row):
    """Brute-force clip search for one fp64 rotated row, independent numpy:
    every candidate's scale from the fp64 absmax, codes on the fp64 quotient,
    fp64 error; returns (best error, index, scale, codes, all errors)."""
    rot_row = np.asarray(rot_row, dtype=np.float64)
    amax = np.abs(rot_row).max()
    best, errs = None, []
    for i in range(51):
        s = np.float32(amax * (100 - i) / 700.0)
        if s == 0:
            q = np.zeros_like(rot_row)
        else:
            q = np.clip(ref_half_away(rot_row / np.float64(s)), -7, 7)
        err = float(np.sum((q * np.float64(s) - rot_row) ** 2))
        errs.append(err)
        if best is None or err < best[0]:
            best = (err, i, s, q.astype(np.int8))
    return best + (np.array(errs),)


@settings(max_examples=15, deadline=None)
@given(N=st.integers(1, 5), seed=st.integers(0, 2**31 - 1), heavy=st.booleans())
def test_int4_clip_search_brute_force(oracle_mod, N, seed, heavy):
    rng = np.random.default_rng(seed)
    K = 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if heavy:
        w[:, rng.choice(K, 3, replace=False)] *= 30
    wq4, s, ci, errs = oracle_mod.quantize_weight_i4(w, 256, with_errors=True)
    assert wq4.shape == (N, K // 2) and wq4.dtype == np.uint8     # two codes per byte
    rot = ref_rotate(w.astype(np.float64), 256)
    q = oracle_mod.unpack_i4(wq4)
    for n in range(N):
        err, i, s_ref, q_ref, errs_ref = _ref_int4_row(rot[n])
        assert ci[n] == i and s[n] == s_ref
        assert np.array_equal(q[n], q_ref)
        assert np.abs(q[n]).max() <= 7
        assert np.allclose(errs[n], errs_ref, rtol=1e-12, atol=0)


def test_int4_forced_candidate(oracle_mod):
    """Forcing each row's candidate gives that candidate's scale and codes
    (checked against the numpy search), and forcing the argmin reproduces the
    unforced result bit for bit."""
    rng = np.random.default_rng(21)
    N, K = 6, 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq4, s, ci = oracle_mod.quantize_weight_i4(w, 256)
    wq4_f, s_f, ci_f = oracle_mod.quantize_weight_i4(w, 256, force_index=ci)
    assert np.array_equal(wq4, wq4_f) and np.array_equal(s, s_f) and np.array_equal(ci, ci_f)
    force = rng.integers(0, 51, N).astype(np.int32)
    wq4_g, s_g, ci_g = oracle_mod.quantize_weight_i4(w, 256, force_index=force)
    assert np.array_equal(ci_g, force)
    rot = ref_rotate(w.astype(np.float64), 256)
    q = oracle_mod.unpack_i4(wq4_g)
    for n in range(N):
        amax = np.abs(rot[n]).max()
        s_ref = np.float32(amax * (100 - force[n]) / 700.0)
        assert s_g[n] == s_ref
        assert np.array_equal(q[n], np.clip(ref_half_away(rot[n] / np.float64(s_ref)), -7, 7).astype(np.int8))
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.quantize_weight_i4(w, 256, force_index=np.full(N, 51, np.int32))


def test_int4_clip_ties_keep_the_larger_c(oracle_mod):
    """Equal errors keep the first candidate, i.e. the larger clip factor
    (the tie rule read for the clip search of 'MossInt4', 'Format').  Two
    closed-form ties (group 1, so the row is not rotated):
      - an all-zero row: every candidate has scale 0, codes 0 and error 0;
      - one subnormal value v = 513 * 2^-149: c = 1.00 and c = 0.99 both give
        the fp32 scale 73 * 2^-149 (513/7 = 73.3 and 513 * 0.99/7 = 72.6 round
        to 73 units), code 7 and error (7 * 73 - 513)^2 units^2, the minimum
        (c = 0.98 gives 72 units and a larger error)."""
    K = 32
    w = np.zeros((2, K), dtype=np.float32)
    w[1, 0] = np.float32(513 * 2.0 ** -149)
    assert w[1, 0] == 513 * 2.0 ** -149
    wq4, s, ci = oracle_mod.quantize_weight_i4(w, 1)
    q = oracle_mod.unpack_i4(wq4)
    assert ci[0] == 0 and s[0] == 0 and not q[0].any()
    assert ci[1] == 0
    assert s[1] == np.float32(73 * 2.0 ** -149)
    assert q[1, 0] == 7 and not q[1, 1:].any()


def test_int4_error_analogue(oracle_mod):
    """Mean relative row error on rotated Gaussian rows is in the range of the
    page's 11.4 % on real weights ('MossInt4', 'Format'); a consistency check,
    not a pin."""
    facts = golden("pages_format.json")
    w = wl.make_weight(64, 4096, seed=31)
    wq4, s, ci = oracle_mod.quantize_weight_i4(w, 256)
    rot = ref_rotate(w.astype(np.float64), 256)
    rec = oracle_mod.unpack_i4(wq4).astype(np.float64) * s[:, None].astype(np.float64)
    rel = np.linalg.norm(rec - rot, axis=1) / np.linalg.norm(rot, axis=1)
    assert 0.10 < rel.mean() < 0.125, rel.mean()
    assert abs(rel.mean() - facts["int4_mean_relative_row_error_on_real_weights"]["value"]) < 0.015
    assert np.all(ci > 0)  # Gaussian rows always clip


def test_w4a8_equals_w8a8_on_unpacked_codes(oracle_mod):
    rng = np.random.default_rng(10)
    xb = _rand_bf16(rng, 6, 512, outliers=3)
    w = (rng.standard_normal((10, 512)) * 0.02).astype(np.float32)
    wq4, s, _ = oracle_mod.quantize_weight_i4(w, 256)
    y4 = oracle_mod.w4a8_linear(xb, wq4, s, 256)
    y8 = oracle_mod.w8a8_linear(xb, oracle_mod.unpack_i4(wq4), s, 256)
    assert np.array_equal(y4, y8)


def test_format_facts(oracle_mod):
    facts = golden("pages_format.json")
    g = facts["group_size"]["value"]
    w = wl.make_weight(8, 2 * g, seed=1)
    wq, ws = oracle_mod.quantize_weight_i8(w, g)
    assert wq.dtype == np.int8 and ws.dtype == np.float32 and ws.shape == (8,)
    wq4, s4, _ = oracle_mod.quantize_weight_i4(w, g)
    assert wq4.shape[1] * facts["int4_weight"]["codes_per_byte"] == 2 * g


# ------------------------------------------------------------------ RMSNorm
# The norm that precedes the quantized linears multiplies by (1 + w) (the
# SmoothQuant folding (1 + w) / s - 1 of "MOSS-Image ... INT8", "How it was
# made").  The pins use powers of two so that every product and square root
# along the way is exact and the expected bf16 value is fixed by hand.

def test_rmsnorm_constant_power_of_two_rows(oracle_mod):
    """A constant row c = +-2^k has rms |c|: with eps 0 and w 0 it normalises
    to +-1 exactly."""
    K = 512
    vals = [2.0 ** k for k in range(-12, 13, 3)] + [-(2.0 ** k) for k in range(-9, 10, 3)]
    x = np.array([[v] * K for v in vals], dtype=np.float32)
    y = wl.bf16_bits_to_float(oracle_mod.rmsnorm(bf16(x), np.zeros(K, np.float32), eps=0.0))
    assert np.array_equal(y, np.sign(x))


@pytest.mark.parametrize("K", [256, 1024, 4096])
def test_rmsnorm_one_hot_gives_sqrt_k(oracle_mod, K):
    """A single nonzero a = 2^k has mean square a^2 / K: the normalised value
    is sqrt(K) (a power of two for these K), every other entry 0."""
    rng = np.random.default_rng(K)
    x = np.zeros((6, K), np.float32)
    pos = rng.choice(K, 6, replace=False)
    for r, p in enumerate(pos):
        x[r, p] = (-1) ** r * 2.0 ** (r - 3)
    y = wl.bf16_bits_to_float(oracle_mod.rmsnorm(bf16(x), np.zeros(K, np.float32), eps=0.0))
    expect = np.zeros_like(x)
    expect[np.arange(6), pos] = np.sign(x[np.arange(6), pos]) * np.sqrt(K)
    assert np.array_equal(y, expect)


def test_rmsnorm_weight_enters_as_one_plus_w(oracle_mod):
    """w = 1 and w = 3 scale the output by exactly 2 and 4; w = -1 zeroes it."""
    rng = np.random.default_rng(5)
    K = 256
    xb = bf16(rng.standard_normal((4, K)).astype(np.float32))
    y0 = wl.bf16_bits_to_float(oracle_mod.rmsnorm(xb, np.zeros(K, np.float32), 1e-6))
    w = np.zeros(K, np.float32)
    w[: K // 3] = 1.0
    w[K // 3: 2 * K // 3] = 3.0
    w[2 * K // 3:] = -1.0
    y = wl.bf16_bits_to_float(oracle_mod.rmsnorm(xb, w, 1e-6))
    assert np.array_equal(y, y0 * (1.0 + w))


def test_rmsnorm_eps_inside_the_root(oracle_mod):
    """Constant row c = 2^k with eps = c^2: the root is sqrt(2) c, so every
    output is bf16(1/sqrt(2)) = 0.70703125."""
    K = 256
    for k in (-4, 0, 5):
        c = 2.0 ** k
        x = np.full((1, K), c, np.float32)
        y = wl.bf16_bits_to_float(oracle_mod.rmsnorm(bf16(x), np.zeros(K, np.float32), eps=c * c))
        assert np.all(y == np.float32(0.70703125)), (k, y[0, :2])


def test_rmsnorm_zero_row_and_unit_rms(oracle_mod):
    """A zero row stays zero (eps > 0); ordinary rows come out with mean
    square 1 up to bf16 rounding."""
    rng = np.random.default_rng(6)
    K = 4096
    x = (rng.standard_normal((8, K)) * 7.0).astype(np.float32)
    x[0] = 0.0
    y = wl.bf16_bits_to_float(oracle_mod.rmsnorm(bf16(x), np.zeros(K, np.float32), 1e-6)).astype(np.float64)
    assert np.all(y[0] == 0.0)
    ms = (y[1:] ** 2).mean(axis=1)
    assert np.all(np.abs(ms - 1.0) < 5e-3), ms


def test_rmsnorm_rotate_quant_is_the_composition(oracle_mod):
    rng = np.random.default_rng(7)
    K = 1024
    xb = _rand_bf16(rng, 5, K, outliers=4)
    w = (rng.standard_normal(K) * 0.3).astype(np.float32)
    xq, s, y = oracle_mod.rmsnorm_rotate_quant(xb, w, 1e-6, 256)
    assert np.array_equal(y, oracle_mod.rmsnorm(xb, w, 1e-6))
    xq2, s2 = oracle_mod.rotate_quant(y, 256)
    assert np.array_equal(xq, xq2) and np.array_equal(s, s2)


# ------------------------------------------------ weight-only dequant path

def _bf16_of_f32(v32):
    """fp32 values -> bf16 bits via torch's CPU cast (round to nearest even)."""
    return wl.float_to_bf16_bits(np.asarray(v32, dtype=np.float32))


@pytest.mark.parametrize("g", [1, 4, 16, 64, 256])
def test_dequant_one_hot_closed_form(oracle_mod, g):
    """A single code c at column j of group b with scale s dequantizes to
    c*s*H[j][k]/sqrt(g) on that group's columns (Sylvester signs from
    scipy) and to zero elsewhere."""
    K = 2 * max(g, 16) if g < 256 else 512
    K -= K % g
    for b, j, c, s in [(0, 0, 127, 0.5), (K // g - 1, g - 1, -77, 2.0 ** -10), (K // g // 2, g // 3, 5, 3.0)]:
        q = np.zeros((1, K), np.int8)
        q[0, b * g + j] = c
        got = wl.bf16_bits_to_float(oracle_mod.dequantize_weight(q, np.array([s], np.float32), g))[0]
        want = np.zeros(K, np.float32)
        signs = scipy.linalg.hadamard(g)[j] if g > 1 else np.ones(1)
        want[b * g:(b + 1) * g] = np.float32(c * s / np.sqrt(g)) * signs
        assert np.array_equal(got, wl.bf16_bits_to_float(_bf16_of_f32(want)))


@pytest.mark.parametrize("g", [8, 16, 32, 128, 256])
def test_dequant_exact_zeros_are_positive_zero(oracle_mod, g):
    """Where the exact value of (wq * s) * H is zero it dequantizes to +0.
    Closed form: a group whose codes start (3, -1, -2) and are zero after
    that transforms to 3 - 1 - 2 = 0 in column 0 (every entry of H's first
    column is +1/sqrt(g)) and in some other columns (scipy's Sylvester matrix
    says which), to nonzero values in the rest; rounding each
    product by 1/sqrt(g) separately would leave RN(3a) - RN(a) - RN(2a), not
    0, for odd log2(g).  A zero row scale gives +0 everywhere (never -0)."""
    K = 2 * g
    q = np.zeros((2, K), np.int8)
    for b in range(K // g):
        q[0, b * g:b * g + 3] = (3, -1, -2)
    q[1] = np.random.default_rng(g).integers(-127, 128, K).astype(np.int8)
    s = np.array([0.0123, 0.0], np.float32)
    out = oracle_mod.dequantize_weight(q, s, g)
    t = q[0, :g].astype(np.int64) @ scipy.linalg.hadamard(g)      # the integer transform of one group
    assert t[0] == 0
    for b in range(K // g):
        grp = out[0, b * g:(b + 1) * g]
        assert np.all(grp[t == 0] == 0x0000)
        assert np.all((grp[t != 0] & 0x7fff) != 0)
    assert np.all(out[1] == 0x0000)


def test_dequant_group_one_is_scale_times_code(oracle_mod):
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, (5, 64), dtype=np.int8)
    s = (rng.random(5) * 0.03 + 1e-4).astype(np.float32)
    got = oracle_mod.dequantize_weight(q, s, 1)
    want = _bf16_of_f32(q.astype(np.float32) * s[:, None])   # each product is exact in fp32
    assert np.array_equal(got, want)


@pytest.mark.parametrize("g", [16, 256])
def test_dequant_inverts_quantize_within_bound(oracle_mod, g):
    """Orthogonality: the un-rotated reconstruction error of a row equals the
    rotated one, which is at most sqrt(K) s / 2 for round-to-nearest codes;
    the bf16 rounding adds at most 2^-9 of the row's norm."""
    rng = np.random.default_rng(11)
    N, K = 16, 1024
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[:, 7] *= 30.0                                            # an outlier column
    q, s = oracle_mod.quantize_weight_i8(w, g)
    back = wl.bf16_bits_to_float(oracle_mod.dequantize_weight(q, s, g)).astype(np.float64)
    err = np.linalg.norm(back - w, axis=1)
    bound = np.sqrt(K) * s / 2 + 2.0 ** -9 * np.linalg.norm(back, axis=1) + 1e-6 * np.linalg.norm(w, axis=1)
    assert np.all(err <= bound)
    assert np.all(err >= 0.05 * np.sqrt(K) * s / 2)             # the codes' rounding is really there


def test_dequant_int4_error_is_the_clip_search_error(oracle_mod):
    """Parseval: for packed int4 rows the un-rotated reconstruction error
    equals the rotated-domain error of the chosen codes, up to bf16 rounding."""
    rng = np.random.default_rng(12)
    N, K = 8, 512
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    packed, s, _ = oracle_mod.quantize_weight_i4(w, 256)
    back = wl.bf16_bits_to_float(oracle_mod.dequantize_weight(packed, s, 256)).astype(np.float64)
    lo, hi = ref_unpack(packed)
    codes = np.stack([lo, hi], axis=-1).reshape(N, K).astype(np.float64)   # low nibble = even column
    rot = ref_rotate(w.astype(np.float64), 256)
    e_rot = np.linalg.norm(codes * s[:, None].astype(np.float64) - rot, axis=1)
    e_back = np.linalg.norm(back - w, axis=1)
    slack = 2.0 ** -9 * np.linalg.norm(back, axis=1) + 1e-6
    assert np.all(np.abs(e_back - e_rot) <= slack)


def _exact_bf16_products(rng, shape, exp_lo=-3, exp_hi=3):
    """bf16 values whose products and sums are exact in fp64 (7-bit mantissas,
    exponents in a narrow band)."""
    mant = rng.integers(128, 256, shape) * rng.choice([-1, 1], shape)
    e = rng.integers(exp_lo, exp_hi + 1, shape)
    v = (mant * np.exp2(e - 7)).astype(np.float32)
    v[rng.random(shape) < 0.1] = 0.0
    return _bf16_of_f32(v)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 4, 17, 1), (5, 7, 64, 2), (2, 9, 300, 3)])
def test_gemm_bf16_brute_force_tiny(oracle_mod, M, N, K, seed):
    """Exact rational sums, rounded to fp32 and then to bf16."""
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    x = _exact_bf16_products(rng, (M, K))
    w = _exact_bf16_products(rng, (N, K))
    xf = wl.bf16_bits_to_float(x)
    wf = wl.bf16_bits_to_float(w)
    want = np.empty((M, N), np.float32)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[m], wf[n])), Fraction(0))
            want[m, n] = np.float32(float(exact))                 # exact in fp64 here, then one fp32 rounding
    assert np.array_equal(oracle_mod.gemm_bf16(x, w), _bf16_of_f32(want))


def test_gemm_bf16_identity_and_rounding_order(oracle_mod):
    """x = I returns W exactly; and a sum just above a bf16 tie, whose fp32
    rounding lands on the tie, rounds to even (fp32 first, then bf16)."""
    rng = np.random.default_rng(4)
    K = 32
    w = _bf16_of_f32(rng.standard_normal((6, K)).astype(np.float32))
    eye = _bf16_of_f32(np.eye(K, dtype=np.float32))
    assert np.array_equal(oracle_mod.gemm_bf16(eye, w), w.T.copy())
    x = _bf16_of_f32(np.array([[1.0, 2.0 ** -8, 2.0 ** -30]], np.float32))
    ones = _bf16_of_f32(np.ones((1, 3), np.float32))
    assert wl.bf16_bits_to_float(oracle_mod.gemm_bf16(x, ones))[0, 0] == 1.0


def test_dequant_linear_is_the_composition(oracle_mod):
    rng = np.random.default_rng(5)
    x = bf16(rng.standard_normal((4, 512)))
    q = rng.integers(-127, 128, (6, 512), dtype=np.int8)
    s = (rng.random(6) * 0.01).astype(np.float32)
    assert np.array_equal(oracle_mod.dequant_linear(x, q, s, 256),
                          oracle_mod.gemm_bf16(x, oracle_mod.dequantize_weight(q, s, 256)))


def test_gemm_bf16_sum_carries_fp64(oracle_mod):
    """2^25 + 200 ones - 2^25: the exact sum 200 survives an fp64 sum (an fp32
    one would lose every 1 next to 2^25)."""
    vals = np.array([2.0 ** 25] + [1.0] * 200 + [-(2.0 ** 25)], np.float32)
    x = _bf16_of_f32(vals[None, :])
    ones = _bf16_of_f32(np.ones((1, vals.size), np.float32))
    assert wl.bf16_bits_to_float(oracle_mod.gemm_bf16(x, ones))[0, 0] == 200.0
