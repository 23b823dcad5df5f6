"""Pins of the fp64 oracle against facts fixed by the definitions and by mathematics.

Each test checks the oracle against something other than itself: a hand-written fixture, a
closed form, an invariant, a library routine the case reduces to, or exact brute force on a
tiny input. No GPU.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle.numpy_ref import NumpyModel, dequant as np_dequant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- number formats

def test_f16_decode_every_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.fixture(autouse=True)
def _quiet_overflow():
    with np.errstate(over="ignore"):
        yield


def _f16_test_values(rng):
    # log-uniform magnitudes from deep subnormal to overflow, both signs, plus exact ties
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 20000))
    vals = mags * rng.choice([-1.0, 1.0], mags.size)
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    ties = (h[:-1] + h[1:]) / 2  # midpoints between neighbours (exact in fp64)
    return np.concatenate([vals, ties, -ties, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0**-25, 2.0**-24 * 1.5]])


def test_f16_encode_round_to_nearest_even_matches_numpy():
    rng = np.random.default_rng(1)
    vals = _f16_test_values(rng)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_generator_f16_encoder_matches_numpy():
    rng = np.random.default_rng(2)
    vals = _f16_test_values(rng)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([synth.f16_bits(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_decode_every_pattern_matches_torch():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    ref = bits.to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_encode_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(3)
    f32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    # exact ties: fp32 patterns whose low 16 bits are 0x8000
    tie_bits = (rng.integers(0, 2**15, 4000, dtype=np.uint32) << 16) | 0x8000
    ties = tie_bits.view(np.float32)
    vals = np.concatenate([f32, ties, np.float32([1e-40, -3e-39, 3.3895e38])])
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert np.isnan(oracle.bf16_to_f64(oracle.f64_to_bf16(float("nan"))))


def test_fp8_decode_every_pattern_matches_torch():
    """OCP FP8 E4M3 decode of all 256 patterns against torch.float8_e4m3fn."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8_to_f64(b) for b in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)  # 0x7F and 0xFF only
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.fp8_to_f64(0x7E) == 448.0 and oracle.fp8_to_f64(0x01) == 2.0 ** -9


def test_fp8_encode_round_to_nearest_even_matches_torch():
    """Below the saturation point (|v| < 464) the encode is torch's round to nearest even."""
    finite = np.array([oracle.fp8_to_f64(b) for b in range(128) if b != 0x7F])  # 0 .. 448
    mids = (finite[:-1] + finite[1:]) / 2  # exact ties
    rng = np.random.default_rng(5)
    rand = rng.uniform(-1, 1, 20000) * np.exp(rng.uniform(-9, 6.1, 20000))
    vals = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), rand])
    vals = np.concatenate([vals, -vals]).astype(np.float32)  # all exact in fp32
    vals = vals[np.abs(vals) < 464]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f64_to_fp8(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_fp8_encode_saturates_and_special_cases():
    # ties to even at both ends of the subnormal range and at the top of the range
    assert oracle.f64_to_fp8(2.0 ** -10) == 0x00 and oracle.f64_to_fp8(-(2.0 ** -10)) == 0x80
    assert oracle.f64_to_fp8(3 * 2.0 ** -10) == 0x02
    assert oracle.f64_to_fp8(463.99) == 0x7E
    # saturating reading: beyond the midpoint above 448, infinities included, the result is +-448
    for v in (464.0, 479.0, 480.0, 1e6, float("inf")):
        assert oracle.f64_to_fp8(v) == 0x7E and oracle.f64_to_fp8(-v) == 0xFE
    assert oracle.f64_to_fp8(float("nan")) == 0x7F
    assert oracle.f64_to_fp8(0.0) == 0x00 and oracle.f64_to_fp8(-0.0) == 0x80
    # every finite pattern round-trips
    for b in range(256):
        if b & 0x7F != 0x7F:
            assert oracle.f64_to_fp8(oracle.fp8_to_f64(b)) == b


# ---------------------------------------------------------------- int4 blocks

def _golden_blocks():
    with open(os.path.join(GOLDEN, "int4_blocks.json")) as f:
        g = json.load(f)
    codes = np.frombuffer(bytes.fromhex("".join(g["codes_hex"])), dtype=np.uint8).reshape(1, -1)
    scales = np.array([int(s, 16) for s in g["scales_f16_hex"]], dtype=np.uint16).reshape(1, -1)
    return g, codes, scales


def test_dequant_matches_hand_written_fixture():
    g, codes, scales = _golden_blocks()
    W = oracle.dequant(codes, scales)
    assert W.shape == (1, g["K"])
    assert W[0].tolist() == g["expected_weights"]


def test_numpy_twin_dequant_matches_fixture():
    g, codes, scales = _golden_blocks()
    assert np_dequant(codes, scales)[0].tolist() == g["expected_weights"]


def test_dequant_exhaustive_codes_and_finite_scales_exact_in_fp32():
    # every finite fp16 scale (both signs) x every code: oracle weight == numpy's fp16 value * (q-8),
    # and the product is exact in fp32 (the bit-exact dequant contract)
    sb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sval = sb.view(np.float16)
    sb = sb[np.isfinite(sval)]
    n = sb.size
    K = 32
    for q in range(16):
        codes = np.full((n, K // 2), q | (q << 4), dtype=np.uint8)
        scales = sb.reshape(n, 1)
        W = oracle.dequant(codes, scales)
        ref = sb.view(np.float16).astype(np.float64) * (q - 8)
        assert np.array_equal(W[:, 0], ref)
        assert np.array_equal(W[:, 31], ref)
        f32 = sb.view(np.float16).astype(np.float32) * np.float32(q - 8)
        assert np.array_equal(f32.astype(np.float64), ref)


def _golden_mx():
    with open(os.path.join(GOLDEN, "mxfp4_blocks.json")) as f:
        g = json.load(f)
    codes = np.frombuffer(bytes.fromhex("".join(g["codes_hex"])), dtype=np.uint8).reshape(1, -1)
    scales = np.array(g["scales_e8m0"], dtype=np.uint8).reshape(1, -1)
    return g, codes, scales


def _torch_e8m0(e: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(e, dtype=np.uint8)).view(torch.float8_e8m0fnu).to(
        torch.float64).numpy()


def test_e2m1_codes_match_hand_written_fixture():
    g, _, _ = _golden_mx()
    got = [oracle.e2m1_to_f64(c) for c in range(16)]
    assert got == g["e2m1_values"]
    assert [np.signbit(v) for v in got] == [c >= 8 for c in range(16)]  # -0.0 is code 8
    # every magnitude is exact in E4M3 (the fp8 operand type of the scaled matrix cores)
    for v in got:
        assert oracle.fp8_to_f64(oracle.f64_to_fp8(v)) == v


def test_e8m0_every_byte_matches_torch():
    e = np.arange(256, dtype=np.uint8)
    ref = _torch_e8m0(e)
    got = np.array([oracle.e8m0_to_f64(int(b)) for b in e])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_mx_dequant_matches_hand_written_fixture():
    g, codes, scales = _golden_mx()
    W = oracle.mx_dequant(codes, scales)
    assert W.shape == (1, g["K"])
    assert W[0].tolist() == g["expected_weights"]
    assert [np.signbit(v) for v in W[0, :16]] == [c >= 8 for c in range(16)]


def test_mx_dequant_exhaustive_codes_and_scales():
    # all 16 codes x all 256 scale bytes, each code in both nibble positions: the weight is the
    # fixture's E2M1 value times torch's E8M0 value (NaN for the NaN scale)
    g, _, _ = _golden_mx()
    vals = np.array(g["e2m1_values"])
    sc = _torch_e8m0(np.arange(256))
    for c in range(16):
        codes = np.full((256, 16), c | (c << 4), dtype=np.uint8)
        W = oracle.mx_dequant(codes, np.arange(256, dtype=np.uint8).reshape(256, 1))
        ref = sc * vals[c]
        for col in (0, 1, 30, 31):
            assert np.array_equal(W[:, col], ref, equal_nan=True), (c, col)
        # and the low / high nibble positions hold different elements
        codes = np.full((1, 16), c, dtype=np.uint8)  # high nibbles zero
        W = oracle.mx_dequant(codes, np.array([[127]], dtype=np.uint8))
        assert np.array_equal(W[0, 0::2], np.full(16, vals[c])) and not np.any(W[0, 1::2])


def test_mx_matmul_matches_library_matmul_on_independent_decode():
    # W decoded here from the fixture's value table, torch's E8M0 and the layout statement
    # (element 2i low nibble, 2i+1 high nibble; block k // 32), then numpy's matmul
    g, _, _ = _golden_mx()
    vals = np.array(g["e2m1_values"])
    rng = np.random.default_rng(77)
    N, K, M = 5, 96, 3
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    W = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            c = (byte >> 4) if k % 2 else (byte & 0xF)
            W[n, k] = vals[c] * 2.0 ** (int(scales[n, k // 32]) - 127)
    assert np.array_equal(oracle.mx_dequant(codes, scales), W)
    X = rng.standard_normal((M, K))
    Y = oracle.mx_matmul(codes, scales, X)
    assert Y.shape == (M, N)
    np.testing.assert_allclose(Y, X @ W.T, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.mx_matmul(codes, scales, X[1]), X[1] @ W.T, rtol=1e-13, atol=1e-15)
    # one-hot inputs read single weights exactly; a NaN scale poisons only its own row
    for k in (0, 33, 95):
        e = np.zeros(K)
        e[k] = 1.0
        assert np.array_equal(oracle.mx_matmul(codes, scales, e), W[:, k])
    scales2 = scales.copy()
    scales2[2, 1] = 255
    y = oracle.mx_matmul(codes, scales2, X[0])
    assert np.isnan(y[2]) and np.all(np.isfinite(np.delete(y, 2)))


def test_generator_mx_matrix_layout_and_scale_range():
    c, s = synth.mx_matrix(9, synth.QKV, 2, 0, 6, 128, 117, 121)
    assert c.shape == (6, 64) and s.shape == (6, 4) and c.dtype == np.uint8 and s.dtype == np.uint8
    assert s.min() >= 117 and s.max() <= 121
    c2, s2 = synth.mx_matrix(9, synth.QKV, 2, 0, 6, 128, 117, 121)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    c3, _ = synth.mx_matrix(9, synth.QKV, 3, 0, 6, 128)
    assert not np.array_equal(c, c3)
    cb, sb = synth.mx_matrix(9, synth.UP, 0, 0, 512, 512, 0, 255)
    assert len(np.unique(sb)) > 200 and len(np.unique(cb & 0xF)) == 16 and len(np.unique(cb >> 4)) == 16


def test_quant_round_trip():
    rng = np.random.default_rng(4)
    N, K = 16, 256
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = np.abs(rng.standard_normal((N, K // 32)) * 0.02).astype(np.float16).view(np.uint16)
    W = oracle.dequant(codes, scales)
    assert np.array_equal(oracle.quantize(W, scales), codes)
    # within range, dequant(quantize(w)) is within half a step of w
    s = scales.view(np.float16).astype(np.float64).repeat(32, axis=1)
    w = rng.uniform(-7.5, 6.5, (N, K)) * s
    back = oracle.dequant(oracle.quantize(w, scales), scales)
    assert np.all(np.abs(back - w) <= s / 2 + 1e-18)


def test_gemv_exact_rationals_tiny():
    rng = np.random.default_rng(5)
    N, K = 3, 64
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    # power-of-two scales and small integer x: every product and partial sum is exact in fp64
    exps = rng.integers(-6, 2, (N, K // 32))
    scales = (2.0 ** exps).astype(np.float16).view(np.uint16)
    x = rng.integers(-9, 10, K).astype(np.float64)
    y = oracle.gemv(codes, scales, x)
    for n in range(N):
        acc = Fraction(0)
        for k in range(K):
            b, i = divmod(k, 32)
            byte = int(codes[n, 16 * b + (i % 16)])
            q = (byte & 15) if i < 16 else (byte >> 4)
            acc += Fraction(2) ** int(exps[n, b]) * (q - 8) * Fraction(int(x[k]))
        assert Fraction(y[n]) == acc


def test_gemv_matches_library_matmul():
    rng = np.random.default_rng(6)
    codes, scales = synth.int4_matrix(77, synth.QKV, 0, 0, 96, 512)
    x = rng.standard_normal(512)
    ref = np_dequant(codes, scales) @ x
    got = oracle.gemv(codes, scales, x)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_gemv_f16_matches_library_matmul():
    rng = np.random.default_rng(7)
    W = synth.router(9, 0, 64, 256)
    x = rng.standard_normal(256)
    ref = W.view(np.float16).astype(np.float64) @ x
    assert np.allclose(oracle.gemv_f16(W, x), ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- RMSNorm, RoPE, SiLU

def test_rmsnorm_closed_forms():
    one = np.full(8, np.float16(1.0).view(np.uint16), dtype=np.uint16)
    # [3, 4] -> x / sqrt(12.5 + eps)
    out = oracle.rmsnorm([3.0, 4.0], one[:2], 1e-6)
    assert np.allclose(out, np.array([3.0, 4.0]) / np.sqrt(12.5 + 1e-6), rtol=1e-15)
    # constant vector c: out = gamma * c / sqrt(c^2 + eps)
    g = np.array([0.5, 1.0, 1.5, 2.0], dtype=np.float16)
    out = oracle.rmsnorm([-3.0] * 4, g.view(np.uint16), 1e-6)
    assert np.allclose(out, g.astype(np.float64) * -3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-15)
    # scale invariance when eps is negligible
    rng = np.random.default_rng(8)
    x = rng.standard_normal(64) * 100
    gb = np.full(64, np.float16(1.25).view(np.uint16), dtype=np.uint16)
    assert np.allclose(oracle.rmsnorm(x, gb, 1e-6), oracle.rmsnorm(7.0 * x, gb, 1e-6), rtol=1e-9)


def test_rope_hand_example_and_invariants():
    # D = 2: one pair, angle = pos * base^0 = pos
    out = oracle.rope([1.0, 0.0], 1, 1e6)
    assert np.allclose(out, [np.cos(1.0), np.sin(1.0)], rtol=0, atol=1e-15)
    rng = np.random.default_rng(9)
    D = 128
    v = rng.standard_normal(D)
    assert np.array_equal(oracle.rope(v, 0, 1e6), v)  # position 0 is the identity
    r = oracle.rope(v, 12345, 1e6)
    half = D // 2
    assert np.allclose(r[:half] ** 2 + r[half:] ** 2, v[:half] ** 2 + v[half:] ** 2, rtol=1e-12)
    # relative position: <R_m q, R_n k> depends only on m - n
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    a = oracle.rope(q, 40, 1e6) @ oracle.rope(k, 17, 1e6)
    b = oracle.rope(q, 40 + 999, 1e6) @ oracle.rope(k, 17 + 999, 1e6)
    assert abs(a - b) <= 1e-10 * (np.abs(q).sum() * np.abs(k).sum())
    # the first pair rotates by exactly pos radians; the last pair by pos * base^(-(D-2)/D)
    e = np.zeros(D)
    e[0] = 1.0
    r = oracle.rope(e, 3, 1e6)
    assert np.isclose(r[0], np.cos(3.0)) and np.isclose(r[half], np.sin(3.0))
    e = np.zeros(D)
    e[half - 1] = 1.0
    th = 3 * 1e6 ** (-(D - 2) / D)
    r = oracle.rope(e, 3, 1e6)
    assert np.isclose(r[half - 1], np.cos(th)) and np.isclose(r[D - 1], np.sin(th))


def test_silu_closed_form():
    assert oracle.silu(0.0) == 0.0
    z = np.linspace(-30, 30, 601)
    assert np.allclose([oracle.silu(v) for v in z], z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- softmax, argmax, top-k

def test_softmax_rows_sum_to_one_and_match_library():
    rng = np.random.default_rng(10)
    for n in (1, 2, 17, 1000):
        s = rng.standard_normal(n) * 30
        p = oracle.softmax(s)
        assert abs(p.sum() - 1.0) < 1e-13
        assert np.allclose(p, scipy.special.softmax(s), rtol=1e-12, atol=1e-300)
        assert np.allclose(oracle.softmax(s + 123.0), p, rtol=1e-12, atol=1e-300)


def test_argmax_and_topk_brute_force_with_ties():
    v = np.array([1.0, 5.0, 3.0, 5.0, -2.0, 5.0])
    assert oracle.argmax(v) == 1 == int(np.argmax(v))
    assert oracle.topk(v, 4).tolist() == [1, 3, 5, 2]
    rng = np.random.default_rng(11)
    for _ in range(50):
        x = rng.integers(-5, 5, 64).astype(np.float64)  # many exact ties
        k = int(rng.integers(1, 64))
        ref = np.argsort(-x, kind="stable")[:k]
        assert oracle.topk(x, k).tolist() == ref.tolist()
        assert oracle.argmax(x) == int(np.argmax(x))


# ---------------------------------------------------------------- attention

def _online_softmax_attention(q, K, V, chunk):
    """Split-K attention with running max / sum merge (a different algorithm)."""
    D = q.size
    m, l, acc = -np.inf, 0.0, np.zeros(D)
    for j0 in range(0, K.shape[0], chunk):
        s = K[j0:j0 + chunk] @ q / np.sqrt(D)
        mj = s.max()
        m_new = max(m, mj)
        acc = acc * np.exp(m - m_new) + np.exp(s - m_new) @ V[j0:j0 + chunk]
        l = l * np.exp(m - m_new) + np.exp(s - m_new).sum()
        m = m_new
    return acc / l


def test_attention_naive_equals_online_softmax_split():
    rng = np.random.default_rng(12)
    D = 128
    for n in (1, 15, 16, 17, 300):
        q = rng.standard_normal(D) * 3
        K = rng.standard_normal((n, D))
        V = rng.standard_normal((n, D))
        out, p = oracle.attention(q, K, V, with_probs=True)
        assert abs(p.sum() - 1.0) < 1e-13
        for chunk in (1, 7, 64):
            assert np.allclose(out, _online_softmax_attention(q, K, V, chunk), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(13)
    D, n = 64, 40
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    assert np.allclose(oracle.attention(q, K, np.ones((n, D))), 1.0, rtol=1e-14)  # V = 1 -> 1
    V = rng.standard_normal((n, D))
    assert np.array_equal(oracle.attention(q, K[:1], V[:1]), V[0])  # one key -> v0
    Kid = np.tile(K[:1], (n, 1))  # identical keys -> mean of V
    assert np.allclose(oracle.attention(q, Kid, V), V.mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_invariant_to_page_pool_permutation():
    rng = np.random.default_rng(14)
    D, P, n, pt = 32, 9, 100, 16
    q = rng.standard_normal(D)
    Kp = rng.standard_normal((P * pt, D))
    Vp = rng.standard_normal((P * pt, D))
    table = rng.permutation(P)[: (n + pt - 1) // pt].astype(np.int32)
    out = oracle.attention_paged(q, Kp, Vp, table, pt, n)
    # logical contiguous view gives the same result
    idx = np.concatenate([np.arange(p * pt, p * pt + pt) for p in table])[:n]
    assert np.array_equal(out, oracle.attention(q, Kp[idx], Vp[idx]))
    # permute the physical pool and remap the table: bitwise identical
    perm = rng.permutation(P)  # new page id of old page p is perm[p]
    Kq = np.empty_like(Kp)
    Vq = np.empty_like(Vp)
    for p in range(P):
        Kq[perm[p] * pt:(perm[p] + 1) * pt] = Kp[p * pt:(p + 1) * pt]
        Vq[perm[p] * pt:(perm[p] + 1) * pt] = Vp[p * pt:(p + 1) * pt]
    assert np.array_equal(oracle.attention_paged(q, Kq, Vq, perm[table].astype(np.int32), pt, n), out)
    # unmapped / stale slots beyond n do not matter
    Kq2, Vq2 = Kq.copy(), Vq.copy()
    last = perm[table[-1]]
    used = n - (len(table) - 1) * pt
    Kq2[last * pt + used:(last + 1) * pt] = np.nan
    Vq2[last * pt + used:(last + 1) * pt] = np.nan
    assert np.array_equal(oracle.attention_paged(q, Kq2, Vq2, perm[table].astype(np.int32), pt, n), out)


# ---------------------------------------------------------------- generator

def test_generator_counter_based_and_distributions():
    c_full, s_full = synth.int4_matrix(5, synth.GATE, 3, 0, 64, 256)
    # any row range regenerates the same rows
    lib = synth.lib()
    part_c = np.empty((10, 128), dtype=np.uint8)
    part_s = np.empty((10, 8), dtype=np.uint16)
    lib.bws_int4_matrix(5, synth.GATE, 3, 0, 64, 256, 17, 10, part_c.ctypes.data, part_s.ctypes.data)
    assert np.array_equal(part_c, c_full[17:27]) and np.array_equal(part_s, s_full[17:27])
    # codes uniform on 0..15
    c, s = synth.int4_matrix(6, synth.DOWN, 0, 0, 512, 4096)
    q = np.concatenate([c & 15, c >> 4]).ravel()
    counts = np.bincount(q, minlength=16)
    assert np.all(np.abs(counts / q.size - 1 / 16) < 0.002)
    # scales |N(0, 0.02)|: mean 0.02*sqrt(2/pi), second moment 4e-4; subnormals kept
    sv = s.view(np.float16).astype(np.float64).ravel()
    assert np.all(sv >= 0)
    assert abs(sv.mean() - 0.02 * np.sqrt(2 / np.pi)) < 3e-4
    assert abs((sv ** 2).mean() - 4e-4) < 1e-5
    assert np.any((sv > 0) & (sv < 2 ** -14))
    # gains fp16(1 + 0.1 z)
    g = synth.norm_gain(7, synth.ATTN_NORM, 0, 100000).view(np.float16).astype(np.float64)
    assert abs(g.mean() - 1.0) < 2e-3 and abs(g.std() - 0.1) < 2e-3
    # synthetic KV: ((h & 0xFF) - 128) / 64, exact in both cache dtypes
    kv = synth.kv_fill(8, 1, 2, 100, 16, 4, 32, synth.KV_BF16)
    vals = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.all(vals * 64 == np.round(vals * 64)) and vals.min() >= -2 and vals.max() < 2
    assert vals[3, 1, 2, 5] == synth.kv_value(8, 1, 2, 103, 1, 2, 5, 4, 32)
    kvh = synth.kv_fill(8, 1, 2, 100, 16, 4, 32, synth.KV_F16).view(np.float16).astype(np.float64)
    assert np.array_equal(kvh, vals)
    # fp8 cache: (c >> 3) / 8 of the same codes c = 64 v, exact in E4M3
    kv8 = synth.kv_fill(8, 1, 2, 100, 16, 4, 32, synth.KV_FP8)
    assert kv8.dtype == np.uint8
    v8 = torch.from_numpy(kv8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v8, np.floor(vals * 8) / 8)
    assert v8[3, 1, 2, 5] == synth.kv_value_dt(8, 1, 2, 103, 1, 2, 5, 4, 32, synth.KV_FP8)
    assert synth.kv_value_dt(8, 1, 2, 103, 1, 2, 5, 4, 32, synth.KV_BF16) == vals[3, 1, 2, 5]


# ---------------------------------------------------------------- whole model

TINY = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=1024,
            vocab=1024, rms_eps=1e-6, rope_base=1e6, kv_dtype="f16")
TINY_MOE = dict(n_layers=2, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=0,
                vocab=512, rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", n_experts=8, top_k=3,
                expert_ffn=64, n_shared=1, shared_ffn=96)


@pytest.mark.parametrize("cfg", [TINY, TINY_MOE], ids=["dense", "moe"])
def test_c_oracle_equals_numpy_twin(cfg):
    seed = 1234
    m = oracle.Model(cfg, seed)
    kv = oracle.KV(m, 1, 64)
    twin = NumpyModel(cfg, seed)
    rng = np.random.default_rng(15)
    toks = rng.integers(0, cfg["vocab"], 12)
    for p, t in enumerate(toks):
        a = oracle.forward(m, kv, 0, [t], p)["logits"][0]
        b = twin.step(int(t))
        assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(b)), p


def test_multi_token_step_equals_sequential_steps():
    """Four tokens in one call (causal over the new positions) equal four single-token calls."""
    m = oracle.Model(TINY, 99)
    rng = np.random.default_rng(16)
    prompt = rng.integers(0, 1024, 5)
    toks = rng.integers(0, 1024, 4)
    kv1, kv2 = oracle.KV(m, 1, 32), oracle.KV(m, 1, 32)
    oracle.forward(m, kv1, 0, prompt, 0)
    oracle.forward(m, kv2, 0, prompt, 0)
    multi = oracle.forward(m, kv1, 0, toks, 5)["logits"]
    seq = np.stack([oracle.forward(m, kv2, 0, [t], 5 + i)["logits"][0] for i, t in enumerate(toks)])
    assert np.allclose(multi, seq, rtol=0, atol=1e-10 * np.abs(seq).max())


def test_moe_full_topk_is_softmax_mixture_and_single_expert_is_dense():
    m = oracle.Model(dict(TINY_MOE, top_k=8, n_shared=0), 5)
    rng = np.random.default_rng(17)
    h = rng.standard_normal(128)
    out, sel = m.moe_ffn(0, h)
    assert sorted(sel.tolist()) == list(range(8))
    r = m.router_logits(0, h)
    assert np.allclose(r, synth.router(5, 0, 8, 128).view(np.float16).astype(np.float64) @ h, rtol=1e-13)
    P = scipy.special.softmax(r)
    ref = sum(P[e] * m.ffn(0, h, expert=e) for e in range(8))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # one expert, top-1, no shared expert: the gate is 1 and the layer is that expert's FFN
    m1 = oracle.Model(dict(TINY_MOE, n_experts=1, top_k=1, n_shared=0), 5)
    out1, sel1 = m1.moe_ffn(1, h)
    assert sel1.tolist() == [0]
    assert np.array_equal(out1, m1.ffn(1, h, expert=0))
    # top-k selection equals a stable descending sort of the router logits
    m8 = oracle.Model(TINY_MOE, 6)
    _, sel3 = m8.moe_ffn(0, h)
    r8 = m8.router_logits(0, h)
    assert sel3.tolist() == np.argsort(-r8, kind="stable")[:3].tolist()


def _gated_mixture(m, layer, h, experts):
    """The MoE layer's definition written out for a given expert set: renormalised softmax gates
    of the router logits over the set, times each expert's SwiGLU FFN, plus the ungated shared
    expert (workload contract: softmax top-k routing, renormalised gates, one shared expert)."""
    P = scipy.special.softmax(m.router_logits(layer, h))
    z = sum(P[e] for e in experts)
    out = sum((P[e] / z) * m.ffn(layer, h, expert=int(e)) for e in experts)
    for s_ in range(m.cfg["n_shared"]):
        out = out + m.ffn(layer, h, expert=s_, shared=True)
    return out


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_moe_near_tie_adoption(seed):
    """The router's several-correct-answers rule: a proposed top-k set is adopted only when it
    differs from the oracle's by experts whose logits lie within tau of the k-th / (k+1)-th
    boundary; duplicates, ids outside [0, E) and any other difference are rejected (rc -1)."""
    m = oracle.Model(TINY_MOE, seed)
    E, k = TINY_MOE["n_experts"], TINY_MOE["top_k"]
    h = np.random.default_rng(seed).standard_normal(TINY_MOE["d_model"])
    r = m.router_logits(1, h)
    order = np.argsort(-r, kind="stable")
    kth, nxt = int(order[k - 1]), int(order[k])
    gap = r[kth] - r[nxt]
    assert gap > 0
    own = [int(e) for e in order[:k]]
    ref_own = _gated_mixture(m, 1, h, own)
    tol = dict(rtol=1e-12, atol=1e-12 * np.abs(ref_own).max())
    # the oracle's own set in another order: nothing to adopt, same output
    rc, out, used, adopted = m.moe_ffn_sel(1, h, own[::-1], 0.0)
    assert (rc, adopted) == (0, 0) and sorted(used.tolist()) == sorted(own)
    assert np.allclose(out, ref_own, **tol)
    # k-th expert swapped for the (k+1)-th: adopted when the gap is within tau ...
    swapped = own[:-1] + [nxt]
    rc, out, used, adopted = m.moe_ffn_sel(1, h, swapped, gap * 1.01)
    assert (rc, adopted) == (0, 1) and used.tolist() == swapped
    ref_sw = _gated_mixture(m, 1, h, swapped)
    assert np.allclose(out, ref_sw, **tol)
    assert not np.allclose(out, ref_own, **tol)  # adoption changes the layer's output
    # ... and rejected when it is not
    rc, _, _, adopted = m.moe_ffn_sel(1, h, swapped, gap * 0.99)
    assert (rc, adopted) == (-1, 0)
    # duplicates and out-of-range ids are never valid, whatever tau
    for bad in ([own[0], own[0]] + own[1:k - 1], own[:-1] + [E], own[:-1] + [-1]):
        rc, _, _, adopted = m.moe_ffn_sel(1, h, bad, 1e9)
        assert (rc, adopted) == (-1, 0), bad
    # an expert far below the boundary may not come in ...
    low = int(order[-1])
    assert r[nxt] - r[low] > gap * 1.01
    rc, _, _, _ = m.moe_ffn_sel(1, h, own[:-1] + [low], gap * 1.01)
    assert rc == -1
    # ... nor may an expert far above it go out (the top-1 dropped for the (k+1)-th)
    assert r[int(order[0])] - r[kth] > gap * 1.01
    rc, _, _, _ = m.moe_ffn_sel(1, h, own[1:] + [nxt], gap * 1.01)
    assert rc == -1


def test_oracle_reads_synthetic_context():
    m = oracle.Model(TINY, 3)
    kv = oracle.KV(m, 2, 8)
    kv.set_synth(1, 4242, 7, 40)
    for (l, pos, w, g, d) in itertools.product([0, 1], [0, 15, 39], [0, 1], [0, 1], [0, 63]):
        assert kv.read(1, l, pos, w, g, d) == synth.kv_value(4242, l, 7, pos, w, g, d, 2, 64)
    m8 = oracle.Model(dict(TINY, kv_dtype="fp8"), 3)
    kv8 = oracle.KV(m8, 2, 8)
    kv8.set_synth(1, 4242, 7, 40)
    for (l, pos, w, g, d) in itertools.product([0, 1], [0, 39], [0, 1], [0, 1], [0, 63]):
        v = synth.kv_value(4242, l, 7, pos, w, g, d, 2, 64)
        assert kv8.read(1, l, pos, w, g, d) == np.floor(v * 8) / 8


def test_fp8_cache_stores_e4m3_roundings():
    """With an fp8 cache every appended key and value is the E4M3 rounding of the same token's
    key and value in an fp16 cache model (the cache dtype changes nothing before the rounding at
    layer 0), and the logits stay close to the fp16 cache's."""
    m16 = oracle.Model(TINY, 11)
    m8 = oracle.Model(dict(TINY, kv_dtype="fp8"), 11)
    kv16, kv8 = oracle.KV(m16, 1, 16), oracle.KV(m8, 1, 16)
    toks = [3, 77, 512, 9]
    out16 = oracle.forward(m16, kv16, 0, toks, 0)["logits"]
    out8 = oracle.forward(m8, kv8, 0, toks, 0)["logits"]
    G, D = TINY["n_kv_heads"], TINY["head_dim"]
    n_diff = 0
    for pos, w, g, d in itertools.product(range(4), [0, 1], range(G), range(D)):
        a16, a8 = kv16.read(0, 0, pos, w, g, d), kv8.read(0, 0, pos, w, g, d)
        # layer 0's keys and values do not depend on the cache, so a16 = fp16(k) and a8 = E4M3(k)
        # of the same k: E4M3(a16) equals a8 except where a16 fell exactly on the midpoint of two
        # E4M3 neighbours (a double-rounding tie), and then a8 is one of those neighbours
        assert oracle.fp8_to_f64(oracle.f64_to_fp8(a8)) == a8
        r = oracle.fp8_to_f64(oracle.f64_to_fp8(a16))
        if r != a8:
            n_diff += 1
            assert a16 == (r + a8) / 2
    assert n_diff < 20
    assert np.max(np.abs(out8 - out16)) < 0.05 * np.max(np.abs(out16))


# ---- speculative acceptance -------------------------------------------------------------------

def test_spec_accept_hand_cases():
    """Worked cases of the acceptance rule (inputs = [last token, drafts...], argmaxes per row)."""
    # every draft matches the prediction before it: 3 stand, 4 tokens committed, nothing masked
    assert oracle.spec_accept([5, 7, 9, 11], [7, 9, 11, 13]) == (3, [7, 9, 11, 13], [])
    # the first draft misses: only the prediction after the last token is committed
    assert oracle.spec_accept([5, 8, 9, 11], [7, 9, 11, 13]) == (0, [7], [1, 2, 3])
    # the second draft misses; the third would match its row but comes after a miss
    assert oracle.spec_accept([5, 7, 4, 11], [7, 9, 11, 13]) == (1, [7, 9], [2, 3])
    # t = 1: plain greedy decoding
    assert oracle.spec_accept([5], [6]) == (0, [6], [])


def _toy_next(prefix):
    """a deterministic 'model': the greedy token after a prefix (a hash of it, 16 symbols)"""
    h = 1469598103934665603
    for v in prefix:
        h = ((h ^ (int(v) + 1)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return (h >> 17) % 16


@pytest.mark.parametrize("t", [1, 2, 4, 6])
def test_spec_accept_reproduces_sequential_greedy(t):
    """The defining property: a loop of verify steps with any drafts, committing by the rule,
    yields exactly the tokens of one-token-at-a-time greedy decoding; with correct drafts it
    commits t tokens per step, with wrong drafts one."""
    rng = np.random.default_rng(t)
    prompt = [int(v) for v in rng.integers(0, 16, 5)]
    n_new = 60
    seq = list(prompt)
    for _ in range(n_new):
        seq.append(_toy_next(seq))
    greedy = seq[len(prompt):]
    for policy in ("right", "wrong", "mixed"):
        committed, cur = [], list(prompt)
        steps = 0
        while len(committed) < n_new:
            # drafts: the true continuation, a wrong one, or right for a random prefix
            truth = greedy[len(committed):len(committed) + t - 1]
            truth += [0] * (t - 1 - len(truth))
            keep = {"right": t - 1, "wrong": 0, "mixed": int(rng.integers(0, t))}[policy]
            drafts = [truth[j] if j < keep else (truth[j] + 1) % 16 for j in range(t - 1)]
            inputs = [cur[-1]] + drafts
            # the verify step: row i predicts after cur + drafts[:i]
            argm = [_toy_next(cur + drafts[:i]) for i in range(t)]
            n, toks, masked = oracle.spec_accept(inputs, argm)
            assert masked == list(range(n + 1, t))
            if policy == "right" and len(committed) + t <= n_new:
                assert n == t - 1
            if policy == "wrong":
                assert n == 0
            committed += toks
            cur += toks
            steps += 1
        assert committed[:n_new] == greedy
        if policy == "right":
            assert steps == -(-n_new // t)
        if policy == "wrong":
            assert steps == n_new
