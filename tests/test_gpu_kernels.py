"""Kernel-level parity of the HIP decode-step kernels against the fp64 oracle (GPU).

Each kernel runs alone through the C-ABI's parity entry points on seeded inputs; the oracle gets
the same inputs. Dequantisation and page indexing must match bit for bit; every other kernel
output must be within 1e-3 relative L2 of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import memory_bound_autoregressive_amd as bw
from memory_bound_autoregressive_amd import configs
from memory_bound_autoregressive_amd.session import Session

from helpers import KERNEL_REL_L2, kv_values, oracle_cfg, rel_l2

pytestmark = pytest.mark.gpu

TINY = configs.TINY
# one layer of the 9B shape (every matrix at its real size), small vocabulary
LAYER9B = dict(configs.DENSE_9B, n_layers=1, vocab=4096)
LAYER9B_FP8 = dict(LAYER9B, kv_dtype="fp8")
TINY_FP8 = dict(configs.TINY, kv_dtype="fp8")
KV_CODE = {"f16": synth.KV_F16, "bf16": synth.KV_BF16, "fp8": synth.KV_FP8}
# one layer of the 27B shape
LAYER27B = dict(configs.DENSE_27B, n_layers=1, vocab=2048)
# a small MoE with the 35B-A3B layer structure (router, top-k, shared expert)
MOE_SMALL = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=0, vocab=512,
                 rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16, n_experts=16, top_k=3,
                 expert_ffn=128, n_shared=1, shared_ffn=128)


def _model(cfg, seed, max_positions=512, max_tokens=8):
    print(f"[case] load model {cfg.get('name', 'custom')} seed={seed}", flush=True)
    return bw.bw_model_load_synthetic(bw.make_config(cfg, max_positions, max_tokens), seed)


def _matrices(cfg):
    names = ["qkv", "o", "lm_head"]
    if cfg.get("n_experts", 0):
        names += ["gate", "up", "down", "shared_gate", "shared_up", "shared_down"]
    else:
        names += ["gate", "up", "down"]
    return names


def _canonical(om: oracle.Model, name: str, expert: int = 0):
    which = {"shared_gate": "shared_gate", "shared_up": "shared_up", "shared_down": "shared_down"}.get(name, name)
    return om.matrix(which, 0, expert)


@pytest.mark.parametrize("cfg,seed", [(TINY, 11), (LAYER9B, 12), (MOE_SMALL, 13)], ids=["tiny", "9b-layer", "moe"])
def test_dequant_bit_exact(cfg, seed):
    m = _model(cfg, seed)
    om = oracle.Model(oracle_cfg(cfg), seed)
    try:
        for name in _matrices(cfg):
            for expert in ([0, 5] if cfg.get("n_experts", 0) and name in ("gate", "up", "down") else [0]):
                codes, scales = _canonical(om, name, expert)
                N, K = codes.shape[0], codes.shape[1] * 2
                print(f"[case] dequant {name} expert={expert} [{N}x{K}]", flush=True)
                out = torch.empty((N, K), dtype=torch.float32, device="cuda")
                bw.bw_debug_dequant(m, name, 0, expert, out)
                torch.cuda.synchronize()
                ref = oracle.dequant(codes, scales).astype(np.float32)
                got = out.cpu().numpy()
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
    finally:
        bw.bw_model_free(m)


def _one_hot_columns(K: int, n: int, rng) -> np.ndarray:
    """n column indices of a K-wide matrix: the first and last column, then pairs in sampled
    blocks, one on a low nibble (element i of the block) and one on a high nibble (element
    16 + i), so both unpack forms of every sampled block are exercised."""
    nblk = K // 32
    cols = [0, K - 1]
    blocks = rng.choice(nblk, size=min(nblk, max(1, (n - 2) // 2)), replace=False)
    for b in blocks:
        cols += [32 * b + int(rng.integers(16)), 32 * b + 16 + int(rng.integers(16))]
    return np.array(cols[:n], dtype=np.int64)


@pytest.mark.parametrize("cfg,seed", [(TINY, 14), (LAYER9B, 15), (MOE_SMALL, 16)], ids=["tiny", "9b-layer", "moe"])
def test_hot_path_dequant_bit_exact(cfg, seed):
    """Dequantisation inside the step's own products, bit for bit. With x = e_k every product but
    one is zero and the one is s (q - 8) * 1, so y[n] = W[n][k] holds exactly in fp32 (fp16 s
    times a 4-bit integer) whatever the summation order. Run through the batch-1 GEMV (one
    column per call), the matrix-core GEMM at 37 rows (16x16 tiles) and at 128 rows (the wide
    32x32 form), and compared bitwise with the oracle's dequantised columns (zeros of either sign
    count as equal: the sign of a sum's zero is the summation's, not the dequantisation's)."""
    m = _model(cfg, seed, max_tokens=128)
    bw.bw_set_gemm_min_rows(m, 2)
    om = oracle.Model(oracle_cfg(cfg), seed)
    rng = np.random.default_rng(seed)
    try:
        for name in _matrices(cfg):
            routed = cfg.get("n_experts", 0) and name in ("gate", "up", "down")
            expert = 5 if routed else 0
            codes, scales = _canonical(om, name, expert)
            N, K = codes.shape[0], codes.shape[1] * 2
            W = oracle.dequant(codes, scales).astype(np.float32)
            # rows: 1 (GEMV), 37 (16x16 GEMM), 128 (wide GEMM); routed experts take the GEMV only
            for M in ((1,) if routed else (1, 37, 128)):
                ncol = 8 if M == 1 else M
                cols = _one_hot_columns(K, ncol, rng)
                print(f"[case] one-hot dequant {name} expert={expert} [{N}x{K}] rows={M}", flush=True)
                if M == 1:
                    got = np.empty((len(cols), N), dtype=np.float32)
                    for i, k in enumerate(cols):
                        x = torch.zeros((1, K), dtype=torch.float32, device="cuda")
                        x[0, int(k)] = 1.0
                        y = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
                        bw.bw_debug_matvec(m, name, 0, expert, x, y)
                        torch.cuda.synchronize()
                        got[i] = y.cpu().numpy()[0]
                else:
                    x = torch.zeros((len(cols), K), dtype=torch.float32, device="cuda")
                    x[torch.arange(len(cols)), torch.from_numpy(cols).cuda()] = 1.0
                    y = torch.full((len(cols), N), float("nan"), dtype=torch.float32, device="cuda")
                    bw.bw_debug_matvec(m, name, 0, expert, x, y)
                    torch.cuda.synchronize()
                    got = y.cpu().numpy()
                ref = np.ascontiguousarray(W[:, cols].T)
                # bit for bit, except the sign of a zero: a zero block scale makes s (q - 8) a signed
                # zero, and the output sums it with the other blocks' +0 terms, which gives +0
                assert not np.any(np.isnan(got)), (name, M)
                bad = np.argwhere((got != ref) | ((got != 0) & (got.view(np.uint32) != ref.view(np.uint32))))
                assert bad.size == 0, (name, M, bad[:4].tolist(), got[tuple(bad[0])], ref[tuple(bad[0])])
    finally:
        bw.bw_model_free(m)


LAYER9B_3L = dict(configs.DENSE_9B, n_layers=3, vocab=4096)


@pytest.mark.parametrize("cfg,seed", [(LAYER9B_3L, 41), (MOE_SMALL, 42)], ids=["9b-3l", "moe"])
def test_export_tensor_matches_generator(cfg, seed):
    """The library's weights, exported in the canonical layout, equal the generator's tensors byte
    for byte: the last layer's matrices and norms, the lm_head, sampled embedding rows and, for
    MoE, the router, the last routed expert and the shared expert."""
    m = _model(cfg, seed)
    try:
        L, d, V = cfg["n_layers"], cfg["d_model"], cfg["vocab"]
        H, G, D = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        l = L - 1

        def export(name, dtype):
            n = bw.bw_model_tensor_bytes(m, name)
            out = np.empty(n // np.dtype(dtype).itemsize, dtype=dtype)
            bw.bw_model_export_tensor(m, name, out)
            return out

        print(f"[case] export {cfg.get('name', 'custom')} layer {l}", flush=True)
        assert np.array_equal(export("final_norm", np.uint16), synth.norm_gain(seed, synth.FINAL_NORM, 0, d))
        assert np.array_equal(export(f"layers.{l}.attn_norm", np.uint16), synth.norm_gain(seed, synth.ATTN_NORM, l, d))
        assert np.array_equal(export(f"layers.{l}.ffn_norm", np.uint16), synth.norm_gain(seed, synth.FFN_NORM, l, d))
        emb = export("embed", np.uint16).reshape(V, d)
        for r0 in (0, V // 2, V - 3):
            assert np.array_equal(emb[r0:r0 + 3], synth.embed_rows(seed, d, r0, 3))
        mats = [("lm_head", synth.LM_HEAD, 0, 0, V, d), (f"layers.{l}.qkv", synth.QKV, l, 0, (H + 2 * G) * D, d),
                (f"layers.{l}.o", synth.O, l, 0, d, H * D)]
        if cfg.get("n_experts", 0):
            E, Fe, Fs = cfg["n_experts"], cfg["expert_ffn"], cfg["shared_ffn"]
            assert np.array_equal(export(f"layers.{l}.router", np.uint16).reshape(E, d), synth.router(seed, l, E, d))
            mats += [(f"layers.{l}.experts.{E - 1}.gate", synth.GATE, l, E, Fe, d),
                     (f"layers.{l}.experts.{E - 1}.up", synth.UP, l, E, Fe, d),
                     (f"layers.{l}.experts.{E - 1}.down", synth.DOWN, l, E, d, Fe),
                     (f"layers.{l}.shared.0.gate", synth.GATE, l, synth.SHARED_EXPERT, Fs, d),
                     (f"layers.{l}.shared.0.up", synth.UP, l, synth.SHARED_EXPERT, Fs, d),
                     (f"layers.{l}.shared.0.down", synth.DOWN, l, synth.SHARED_EXPERT, d, Fs)]
        else:
            F = cfg["ffn_dim"]
            mats += [(f"layers.{l}.gate", synth.GATE, l, 0, F, d), (f"layers.{l}.up", synth.UP, l, 0, F, d),
                     (f"layers.{l}.down", synth.DOWN, l, 0, d, F)]
        for name, kind, layer, ex, N, K in mats:
            codes, scales = synth.int4_matrix(seed, kind, layer, ex, N, K)
            assert np.array_equal(export(name + ".codes", np.uint8).reshape(N, K // 2), codes), name
            assert np.array_equal(export(name + ".scales", np.uint16).reshape(N, K // 32), scales), name
        with pytest.raises(bw.BWError):
            bw.bw_model_export_tensor(m, "final_norm", np.empty(d + 1, dtype=np.uint16))  # wrong size
        with pytest.raises(bw.BWError):
            bw.bw_model_tensor_bytes(m, f"layers.{L}.o.codes")  # no such layer
    finally:
        bw.bw_model_free(m)


@pytest.mark.parametrize("cfg,seed", [(TINY, 21), (LAYER9B, 22), (LAYER27B, 24), (MOE_SMALL, 23)],
                         ids=["tiny", "9b-layer", "27b-layer", "moe"])
def test_gemv_matches_oracle(cfg, seed):
    m = _model(cfg, seed)
    om = oracle.Model(oracle_cfg(cfg), seed)
    rng = np.random.default_rng(seed)
    try:
        for name in _matrices(cfg):
            codes, scales = _canonical(om, name, 3 if (cfg.get("n_experts", 0) and name in ("gate", "up", "down")) else 0)
            expert = 3 if (cfg.get("n_experts", 0) and name in ("gate", "up", "down")) else 0
            N, K = codes.shape[0], codes.shape[1] * 2
            print(f"[case] gemv {name} [{N}x{K}]", flush=True)
            x = rng.standard_normal(K).astype(np.float32)
            xd = torch.from_numpy(x).cuda().reshape(1, K)
            y = torch.empty((1, N), dtype=torch.float32, device="cuda")
            bw.bw_debug_matvec(m, name, 0, expert, xd, y)
            torch.cuda.synchronize()
            ref = oracle.gemv(codes, scales, x.astype(np.float64))
            err = rel_l2(y.cpu().numpy()[0], ref)
            assert err <= KERNEL_REL_L2, (name, err)
            assert err <= 1e-5, (name, err)  # fp32 accumulation is far inside the bound
    finally:
        bw.bw_model_free(m)


@pytest.mark.parametrize("cfg,seed", [(TINY, 31), (LAYER9B, 32), (LAYER27B, 34), (MOE_SMALL, 33)],
                         ids=["tiny", "9b-layer", "27b-layer", "moe"])
def test_batched_gemm_matches_oracle(cfg, seed):
    """The matrix-core GEMM of the batched step (forced for every row count) against the fp64
    product of the oracle's dequantised matrix, at row counts that leave a ragged m-tile (5, 37),
    fill one workgroup's 128 rows, and spill into a second row group (131)."""
    m = _model(cfg, seed, max_tokens=136)
    bw.bw_set_gemm_min_rows(m, 1)
    om = oracle.Model(oracle_cfg(cfg), seed)
    rng = np.random.default_rng(seed)
    try:
        for name in _matrices(cfg):
            expert = 3 if (cfg.get("n_experts", 0) and name in ("gate", "up", "down")) else 0
            codes, scales = _canonical(om, name, expert)
            N, K = codes.shape[0], codes.shape[1] * 2
            W = oracle.dequant(codes, scales)
            for M in (1, 5, 37, 128, 131):
                print(f"[case] gemm {name} [{N}x{K}] rows={M}", flush=True)
                x = rng.standard_normal((M, K)).astype(np.float32)
                y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
                bw.bw_debug_matvec(m, name, 0, expert, torch.from_numpy(x).cuda(), y)
                torch.cuda.synchronize()
                ref = x.astype(np.float64) @ W.T
                got = y.cpu().numpy()
                assert np.all(np.isfinite(got)), (name, M)
                for r in range(M):
                    err = rel_l2(got[r], ref[r])
                    assert err <= 1e-5, (name, M, r, err)  # exact products, fp32 sums
    finally:
        bw.bw_model_free(m)


def test_batched_gemm_threshold_and_gemv_agree():
    """The same rows through the GEMV (threshold off) and the GEMM agree to fp32 summation order."""
    cfg, seed = LAYER9B, 35
    m = _model(cfg, seed, max_tokens=16)
    rng = np.random.default_rng(seed)
    try:
        for name in ("qkv", "down"):
            N = {"qkv": (cfg["n_q_heads"] + 2 * cfg["n_kv_heads"]) * cfg["head_dim"], "down": cfg["d_model"]}[name]
            K = {"qkv": cfg["d_model"], "down": cfg["ffn_dim"]}[name]
            x = torch.from_numpy(rng.standard_normal((16, K)).astype(np.float32)).cuda()
            outs = []
            for rows in (0, 1):
                bw.bw_set_gemm_min_rows(m, rows)
                y = torch.empty((16, N), dtype=torch.float32, device="cuda")
                bw.bw_debug_matvec(m, name, 0, 0, x, y)
                torch.cuda.synchronize()
                outs.append(y.cpu().numpy().astype(np.float64))
            for r in range(16):
                assert rel_l2(outs[1][r], outs[0][r]) <= 1e-5, (name, r)
    finally:
        bw.bw_model_free(m)


def _attention_case(cfg, seed, lens, t, pool_seed, poison=False):
    """Synthesised contexts, random rotated queries; returns (gpu out, session)."""
    H, G, D = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    B = len(lens)
    s = Session(cfg, seed=seed, max_len=[n + t for n in lens], max_tokens=B * t, pool_seed=pool_seed)
    if poison:
        s.poison(0x7E00 if cfg["kv_dtype"] == "f16" else 0x7FC0)
    s.synthesize(seed + 1, [n + t for n in lens])
    rng = np.random.default_rng(seed + 2)
    q = (rng.standard_normal((B * t, H, D)) * 2).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    out = torch.empty_like(qd)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bw.bw_debug_attention(s.model, s.pool, 0, qd, sl, s.page_table, B, t, s.max_pages, out)
    torch.cuda.synchronize()
    return q, out.cpu().numpy(), s


@pytest.mark.parametrize("cfg,lens,t", [
    (TINY, [1, 37, 300], 1), (TINY, [5, 64, 200], 4),
    (LAYER9B, [2048], 1), (LAYER9B, [1, 17, 999], 4), (LAYER27B, [700], 1),
    (TINY_FP8, [1, 37, 300], 1), (LAYER9B_FP8, [2048], 1), (LAYER9B_FP8, [1, 17, 999], 4),
], ids=["tiny-t1", "tiny-t4", "9b-2048", "9b-t4-ragged", "27b-t1", "tiny-fp8-t1", "9b-fp8-2048", "9b-fp8-t4-ragged"])
def test_attention_matches_oracle(cfg, lens, t):
    seed = 31
    H, G, D = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    rep = H // G
    dtype = KV_CODE[cfg["kv_dtype"]]
    print(f"[case] attention {cfg.get('name')} lens={lens} t={t}", flush=True)
    q, got, s = _attention_case(cfg, seed, lens, t, pool_seed=5)
    try:
        for b, n0 in enumerate(lens):
            kv = kv_values(synth, seed + 1, 0, b, n0 + t, G, D, dtype)
            for ti in range(t):
                n = n0 + ti + 1
                ref = np.stack([oracle.attention(q[b * t + ti, h].astype(np.float64), kv[:n, 0, h // rep], kv[:n, 1, h // rep])
                                for h in range(H)])
                err = rel_l2(got[b * t + ti], ref)
                assert err <= KERNEL_REL_L2, (b, ti, err)
                assert err <= 1e-5, (b, ti, err)
    finally:
        s.close()


def test_attention_invariant_to_pool_permutation_and_poison():
    cfg = LAYER9B
    lens, t = [3, 290, 1000], 4
    _, a, s1 = _attention_case(cfg, 41, lens, t, pool_seed=1)
    s1.close()
    _, b, s2 = _attention_case(cfg, 41, lens, t, pool_seed=2)
    s2.close()
    _, c, s3 = _attention_case(cfg, 41, lens, t, pool_seed=3, poison=True)
    s3.close()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    assert np.isfinite(c).all()


@pytest.mark.parametrize("cfg", [TINY, TINY_FP8], ids=["f16", "fp8"])
def test_kv_append_lands_at_page_table_slot(cfg):
    """One step at position p writes k, v (RoPE'd, rounded) to page table[p // 16], slot p % 16 and
    nothing else; the values match the oracle's cached k, v to within one unit of the cache format."""
    seed, ctx = 51, 37
    fp8 = cfg["kv_dtype"] == "fp8"
    edt = np.uint8 if fp8 else np.uint16
    G, D = cfg["n_kv_heads"], cfg["head_dim"]
    s = Session(cfg, seed=seed, max_len=[ctx + 1], max_tokens=1, pool_seed=9)
    try:
        s.synthesize(seed + 1, [ctx])
        before = {}
        for l in range(cfg["n_layers"]):
            for p in range(s.n_pages):
                buf = np.empty(G * 2 * 16 * D, dtype=edt)
                bw.bw_kv_pool_read(s.pool, l, p, buf)
                before[(l, p)] = buf
        tok = 123
        s.step(torch.tensor([tok], dtype=torch.int32, device="cuda"), torch.tensor([ctx], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        om = oracle.Model(oracle_cfg(cfg), seed)
        okv = oracle.KV(om, 1, 8)
        okv.set_synth(0, seed + 1, 0, ctx)
        oracle.forward(om, okv, 0, [tok], ctx, want_logits=False)
        page = int(s.page_table_host[0, ctx // 16])
        slot = ctx % 16
        for l in range(cfg["n_layers"]):
            for p in range(s.n_pages):
                buf = np.empty(G * 2 * 16 * D, dtype=edt)
                bw.bw_kv_pool_read(s.pool, l, p, buf)
                v = buf.reshape(G, 2, 16, D)
                w = before[(l, p)].reshape(G, 2, 16, D)
                if p != page:
                    assert np.array_equal(v, w), (l, p)
                    continue
                mask = np.ones_like(v, dtype=bool)
                mask[:, :, slot, :] = False
                assert np.array_equal(v[mask], w[mask]), (l, p)
                ref = np.array([[[okv.read(0, l, ctx, kv, g, d) for d in range(D)] for kv in range(2)] for g in range(G)])
                if fp8:
                    got = torch.from_numpy(np.ascontiguousarray(v[:, :, slot, :])).view(torch.float8_e4m3fn)
                    got = got.to(torch.float64).numpy()
                    # one E4M3 step at |ref|: 2^(e - 3), e = max(floor(log2 |ref|), -6)
                    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -9)))
                    ulp = 2.0 ** (np.maximum(e, -6) - 3)
                else:
                    got = v[:, :, slot, :].view(np.float16).astype(np.float64)  # fp16 cache (tiny)
                    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
                assert np.all(np.abs(got - ref) <= ulp + 1e-12), (l, np.max(np.abs(got - ref)))
    finally:
        s.close()


def _round_inputs(kv_dtype):
    """fp32 values spanning the format: normals, subnormals, exact ties, values beyond the range"""
    rng = np.random.default_rng(71 + kv_dtype)
    lo, hi = {bw.BW_KV_F16: (-26, 17), bw.BW_KV_BF16: (-135, 128), bw.BW_KV_FP8: (-11, 10)}[kv_dtype]
    v = rng.uniform(-1, 1, 40000) * 2.0 ** rng.uniform(lo, hi, 40000)
    if kv_dtype == bw.BW_KV_FP8:
        rep_vals = np.array([oracle.fp8_to_f64(b) for b in range(256) if b & 0x7F != 0x7F])
        dec = oracle.fp8_to_f64
    elif kv_dtype == bw.BW_KV_F16:
        rep_vals = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
        dec = oracle.f16_to_f64
    else:
        rep_vals = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
        dec = oracle.bf16_to_f64
    rep_vals = np.unique(rep_vals[np.isfinite(rep_vals)])
    mids = (rep_vals[:-1] + rep_vals[1:]) / 2
    sel = rng.choice(len(mids), min(len(mids), 20000), replace=False)
    x = np.concatenate([v, rep_vals[rng.choice(len(rep_vals), min(len(rep_vals), 5000), replace=False)], mids[sel],
                        [0.0, -0.0, 1e30, -1e30, np.inf, -np.inf, 460.0, 464.0, 470.0, -500.0]]).astype(np.float32)
    return x[np.isfinite(x) | np.isinf(x)], dec


@pytest.mark.parametrize("kv_dtype", [bw.BW_KV_F16, bw.BW_KV_BF16, bw.BW_KV_FP8], ids=["f16", "bf16", "fp8"])
def test_kv_rounding_is_bit_exact(kv_dtype):
    """The conversion that stores every key and value rounds exactly as the oracle does (nearest,
    ties to even; FP8 saturating at +-448) on the same fp32 inputs, and reads back the oracle's value."""
    x, dec = _round_inputs(kv_dtype)
    enc = {bw.BW_KV_F16: oracle.f64_to_f16, bw.BW_KV_BF16: oracle.f64_to_bf16, bw.BW_KV_FP8: oracle.f64_to_fp8}[kv_dtype]
    xd = torch.from_numpy(x).cuda()
    bits = torch.empty(x.size, dtype=torch.int16, device="cuda")
    back = torch.empty(x.size, dtype=torch.float32, device="cuda")
    print(f"[case] kv rounding dtype {kv_dtype}, {x.size} values", flush=True)
    bw.bw_debug_kv_round(kv_dtype, xd, bits, back)
    torch.cuda.synchronize()
    gb = bits.cpu().numpy().view(np.uint16)
    gv = back.cpu().numpy().astype(np.float64)
    ref = np.array([enc(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(gb != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(gb[i]), int(ref[i])) for i in bad[:8]]
    rv = np.array([dec(int(b)) for b in ref])
    assert np.array_equal(gv, rv)


def test_device_errors_are_flagged_not_faults():
    cfg = TINY
    s = Session(cfg, seed=61, max_len=[40], max_tokens=2, pool_seed=3)
    try:
        bad = s.page_table.clone()
        bad[0, 0] = s.n_pages + 5  # out of range page id
        logits = torch.empty((1, cfg["vocab"]), dtype=torch.float32, device="cuda")
        am = torch.empty(1, dtype=torch.int32, device="cuda")
        bw.bw_decode_step(s.model, s.pool, torch.tensor([1], dtype=torch.int32, device="cuda"),
                          torch.tensor([0], dtype=torch.int32, device="cuda"), bad, 1, 1, s.max_pages, logits, am)
        assert bw.bw_check_device_error(s.model) & bw.BW_DERR_PAGE
        bw.bw_decode_step(s.model, s.pool, torch.tensor([cfg["vocab"] + 3], dtype=torch.int32, device="cuda"),
                          torch.tensor([0], dtype=torch.int32, device="cuda"), s.page_table, 1, 1, s.max_pages, logits, am)
        assert bw.bw_check_device_error(s.model) & bw.BW_DERR_TOKEN
        assert bw.bw_check_device_error(s.model) == 0
        with pytest.raises(bw.BWError) as e:
            bw.bw_decode_step(s.model, s.pool, torch.zeros(3, dtype=torch.int32, device="cuda"),
                              torch.zeros(3, dtype=torch.int32, device="cuda"), s.page_table, 3, 1, s.max_pages, None, None)
        assert e.value.code == bw.BW_ERANGE
    finally:
        s.close()


LAYER9B_2L = dict(configs.DENSE_9B, n_layers=2, vocab=512)


@pytest.mark.parametrize("cfg", [TINY, TINY_FP8, LAYER9B_2L], ids=["f16", "fp8", "bf16-9b"])
def test_pool_synthesis_on_device_matches_host_form(cfg):
    """bw_kv_pool_synthesize_async (device arrays, caller's stream) writes exactly the bits of the
    host form on a ragged batch with a permuted page table (lengths 0, 1, 16, 17, 100; sequence ids
    other than b), slots it does not own stay as they were, and its pages hold the generator's
    values; a page id out of range and a negative length are flagged, not faulted."""
    seed, syn_seed = 61, 9001
    lens = [0, 1, 16, 17, 100]
    ids = [5, 0, 3, 7, 2]
    fp8 = cfg["kv_dtype"] == "fp8"
    edt = np.uint8 if fp8 else np.uint16
    G, D, L = cfg["n_kv_heads"], cfg["head_dim"], cfg["n_layers"]
    print(f"[case] device pool synthesis {cfg.get('name', cfg['kv_dtype'])} lens={lens}", flush=True)
    host = Session(cfg, seed=seed, max_len=[max(n, 1) for n in lens], max_tokens=1, pool_seed=4)
    dev = Session(cfg, seed=seed, max_len=[max(n, 1) for n in lens], max_tokens=1, pool_seed=4, model=host.model)
    try:
        host.poison()
        dev.poison()
        host.synthesize(syn_seed, lens, ids)
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        sid = torch.tensor(ids, dtype=torch.int32, device="cuda")
        bw.bw_kv_pool_synthesize_async(dev.pool, syn_seed, sid, sl, dev.page_table, len(lens), dev.max_pages)
        torch.cuda.synchronize()
        assert bw.bw_check_device_error(dev.model) == 0
        for l in range(L):
            for p in range(host.n_pages):
                a = np.empty(G * 2 * 16 * D, dtype=edt)
                b = np.empty_like(a)
                bw.bw_kv_pool_read(host.pool, l, p, a)
                bw.bw_kv_pool_read(dev.pool, l, p, b)
                assert np.array_equal(a, b), (l, p)
        # the last sequence's pages against the generator itself
        bl, n = len(lens) - 1, lens[-1]
        for l in range(L):
            want = synth.kv_fill(syn_seed, l, ids[bl], 0, n, G, D, KV_CODE[cfg["kv_dtype"]]).reshape(n, 2, G, D)
            for lp in range((n + 15) // 16):
                buf = np.empty(G * 2 * 16 * D, dtype=edt)
                bw.bw_kv_pool_read(dev.pool, l, int(dev.page_table_host[bl, lp]), buf)
                got = buf.reshape(G, 2, 16, D)
                ns = min(16, n - 16 * lp)
                assert np.array_equal(got[:, :, :ns, :], want[16 * lp:16 * lp + ns].transpose(2, 1, 0, 3)), (l, lp)
        # range errors from the device: a page id past the pool, then a negative length
        bad = dev.page_table.clone()
        bad[4, 0] = dev.n_pages
        bw.bw_kv_pool_synthesize_async(dev.pool, syn_seed, None, sl, bad, len(lens), dev.max_pages)
        torch.cuda.synchronize()
        assert bw.bw_check_device_error(dev.model) & bw.BW_DERR_PAGE
        neg = torch.tensor([-3, 1, 1, 1, 1], dtype=torch.int32, device="cuda")
        bw.bw_kv_pool_synthesize_async(dev.pool, syn_seed, None, neg, dev.page_table, len(lens), dev.max_pages)
        torch.cuda.synchronize()
        assert bw.bw_check_device_error(dev.model) & bw.BW_DERR_POS
        assert bw.bw_check_device_error(dev.model) == 0
        print(f"[result] device pool synthesis bit-identical to the host form over {L} layers x {host.n_pages} pages")
    finally:
        dev.close()
        host.close()
