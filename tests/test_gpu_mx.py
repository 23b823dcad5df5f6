"""MXFP4 weights on the GPU against the oracle (bw24 deep-dive page, section 1 quantisation formats
and the section 7 table: 4-bit floating-point weights; format: OCP MX, E2M1 elements with one E8M0
scale per 32).

- bw_mx_gemv (batch 1, vector units): relative L2 error within 1e-5 of the oracle's fp64 product
  (tighter than the 1e-3 per-kernel bar: every weight is exact in fp32 and only the fp32 sums
  round), at ragged shapes (K an odd number of blocks, N not a multiple of the 4 rows a wave
  takes) and the 9B layer shapes; one-hot inputs read single weights, which must equal the
  oracle's dequantised values bit for bit over every code, both nibbles and scale bytes 0..250;
  a NaN scale (byte 255) poisons exactly its row.
- bw_mx_gemm (scaled matrix cores: E4M3 x E2M1 with E8M0 block scales, X written as three MXFP8
  terms): relative L2 within 1e-3 (the per-kernel bar) at ragged shapes and at the verify shape
  (M = 128) of the 9B matrices, those sampled column by column against the oracle; one-hot rows
  of X are exact in the first term, so the product reads single weights bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import memory_bound_autoregressive_amd as bw

pytestmark = pytest.mark.gpu


def _rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _gemv(codes, scales, x):
    y = torch.empty(codes.shape[0], dtype=torch.float32, device="cuda")
    bw.bw_mx_gemv(_dev(codes), _dev(scales), _dev(x.astype(np.float32)), y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _gemm(codes, scales, X):
    N, K = codes.shape[0], codes.shape[1] * 2
    M = X.shape[0]
    ws = torch.empty(bw.bw_mx_gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    bw.bw_mx_gemm(_dev(codes), _dev(scales), _dev(X.astype(np.float32)), Y, ws)
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64)


GEMV_SHAPES = [(1, 32), (37, 96), (130, 4128), (257, 4096), (64, 12288), (9, 16384)]


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
def test_mx_gemv_matches_oracle(N, K):
    seed = 4000 + N + K
    print(f"[case] mx gemv N={N} K={K}", flush=True)
    codes, scales = synth.mx_matrix(seed, synth.QKV, 0, 0, N, K)
    x = np.random.default_rng(seed).standard_normal(K).astype(np.float32)
    got = _gemv(codes, scales, x)
    ref = oracle.mx_matmul(codes, scales, x.astype(np.float64))
    err = _rel_l2(got, ref)
    print(f"[result] mx gemv N={N} K={K}: rel L2 {err:.2e}")
    assert err <= 1e-5


def test_mx_gemv_layer_shapes_sampled():
    # the 9B layer's matrices in MXFP4 (QKV, O, gate/up, down), rows sampled against the oracle
    rng = np.random.default_rng(4100)
    for N, K in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)):
        print(f"[case] mx gemv 9B shape N={N} K={K}", flush=True)
        codes, scales = synth.mx_matrix(4100, synth.UP, 1, 0, N, K)
        x = rng.standard_normal(K).astype(np.float32)
        got = _gemv(codes, scales, x)
        rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 62)]))
        ref = oracle.mx_matmul(codes[rows], scales[rows], x.astype(np.float64))
        err = _rel_l2(got[rows], ref)
        assert err <= 1e-5, (N, K, err)
        assert np.all(np.isfinite(got))


def _one_hot_cases(K, rng):
    # the first and last two elements (both nibbles of the row's first and last byte) and a sample
    ks = {0, 1, K - 2, K - 1}
    ks.update(int(v) for v in rng.integers(0, K, 28))
    return sorted(ks)


def test_mx_gemv_one_hot_reads_weights_bit_exact():
    N, K = 512, 2048
    rng = np.random.default_rng(4200)
    codes, _ = synth.mx_matrix(4200, synth.O, 0, 0, N, K)
    # scale bytes 0..250 (6 * 2^123 is the largest product below fp32's range), all rows
    scales = rng.integers(0, 251, (N, K // 32)).astype(np.uint8)
    scales[:251, 0] = np.arange(251)
    W = oracle.mx_dequant(codes, scales)
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W), "every weight exact in fp32"
    ks = _one_hot_cases(K, rng)
    for k in ks:
        x = np.zeros(K, dtype=np.float32)
        x[k] = 1.0
        got = _gemv(codes, scales, x)
        same = got == W[:, k]  # IEEE equality: a -0.0 weight may come out as +0.0
        assert np.all(same), (k, np.flatnonzero(~same)[:5])
    # every code value was read in both nibble positions
    seen = {(int(codes[n, k // 2] >> (4 * (k % 2))) & 0xF, k % 2) for n in range(N) for k in ks}
    assert len(seen) == 32


def test_mx_gemv_nan_scale_poisons_its_row():
    N, K = 40, 256
    codes, scales = synth.mx_matrix(4300, synth.O, 0, 0, N, K)
    scales = scales.copy()
    scales[17, 3] = 255
    x = np.random.default_rng(4300).standard_normal(K).astype(np.float32)
    got = _gemv(codes, scales, x)
    assert np.isnan(got[17]) and np.all(np.isfinite(np.delete(got, 17)))


def test_mx_gemv_bad_arguments():
    codes = torch.zeros((4, 24), dtype=torch.uint8, device="cuda")  # K = 48: not a multiple of 32
    scales = torch.zeros((4, 1), dtype=torch.uint8, device="cuda")
    x = torch.zeros(48, device="cuda")
    y = torch.zeros(4, device="cuda")
    with pytest.raises(bw.BWError):
        bw.bw_mx_gemv(codes, scales, x, y)


GEMM_SHAPES = [(1, 64, 64), (5, 37, 96), (33, 130, 160), (128, 256, 4096), (131, 300, 4128)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_mx_gemm_matches_oracle(M, N, K):
    seed = 5000 + M + N + K
    print(f"[case] mx gemm M={M} N={N} K={K}", flush=True)
    codes, scales = synth.mx_matrix(seed, synth.GATE, 0, 0, N, K)
    X = np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32)
    got = _gemm(codes, scales, X)
    ref = oracle.mx_matmul(codes, scales, X.astype(np.float64))
    err = _rel_l2(got, ref)
    print(f"[result] mx gemm M={M} N={N} K={K}: rel L2 {err:.2e}")
    assert err <= 1e-3
    assert np.all(np.isfinite(got))


def test_mx_gemm_verify_shapes_sampled():
    # M = 128 rows (32 sequences x 4 verified tokens) against the 9B matrices, 24 sampled columns each
    rng = np.random.default_rng(5100)
    X = rng.standard_normal((128, 12288)).astype(np.float32)
    for N, K in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)):
        print(f"[case] mx gemm 9B shape M=128 N={N} K={K}", flush=True)
        codes, scales = synth.mx_matrix(5100, synth.DOWN, 2, 0, N, K)
        Xk = np.ascontiguousarray(X[:, :K])
        got = _gemm(codes, scales, Xk)
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 22)]))
        ref = oracle.mx_matmul(codes[cols], scales[cols], Xk.astype(np.float64))
        err = _rel_l2(got[:, cols], ref)
        print(f"[result] mx gemm M=128 N={N} K={K}: rel L2 {err:.2e} on {len(cols)} columns")
        assert err <= 1e-3, (N, K, err)
        assert np.all(np.isfinite(got))


def test_mx_gemm_one_hot_rows_read_weights_bit_exact():
    M, N, K = 96, 200, 1056  # K: 33 blocks (odd), N ragged
    rng = np.random.default_rng(5200)
    codes, scales = synth.mx_matrix(5200, synth.GATE, 3, 0, N, K, 100, 150)
    W = oracle.mx_dequant(codes, scales)
    ks = _one_hot_cases(K, rng)
    ks = np.array(ks + [int(v) for v in rng.integers(0, K, M - len(ks))])
    X = np.zeros((M, K), dtype=np.float32)
    X[np.arange(M), ks] = 1.0
    got = _gemm(codes, scales, X)
    ref = W[:, ks].T
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_mx_gemm_bad_arguments():
    codes = torch.zeros((4, 32), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    X = torch.zeros((2, 64), device="cuda")
    Y = torch.zeros((2, 4), device="cuda")
    need = bw.bw_mx_gemm_workspace_bytes(2, 4, 64)
    with pytest.raises(bw.BWError):
        bw.bw_mx_gemm(codes, scales, X, Y, torch.zeros(max(need - 256, 1), dtype=torch.uint8, device="cuda"))
    with pytest.raises(bw.BWError):
        bw.bw_mx_gemm_workspace_bytes(2, 4, 48)
