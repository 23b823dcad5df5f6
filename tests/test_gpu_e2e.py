"""End-to-end parity of the decode step against the fp64 oracle (GPU).

Both sides are teacher-forced on the oracle's greedy tokens, so every step is compared on the
same inputs: logits within 2e-2 max-abs, and the GPU's greedy token equal to the oracle's wherever
the oracle's top-2 margin exceeds 1e-2. For MoE, a router selection that differs from the
oracle's only by experts within 1e-4 of the top-k boundary is a valid near tie: the oracle checks
it and follows it (any other difference fails).
"""
import numpy as np
import pytest
import torch

import oracle
import memory_bound_autoregressive_amd as bw
from memory_bound_autoregressive_amd import configs
from memory_bound_autoregressive_amd.session import Session

from helpers import LOGITS_MAX_ABS, TOKEN_MARGIN, oracle_cfg, top2_margin

pytestmark = pytest.mark.gpu

MOE_SMALL = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=0, vocab=512,
                 rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16, n_experts=16, top_k=3,
                 expert_ffn=128, n_shared=1, shared_ffn=128, name="moe-small")
# the MoE shape of the single-launch step (d 2048, nine slots of width 512, head dim 128, four query
# heads per KV head) at two layers and a small vocabulary
MOE_2K = dict(n_layers=2, d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=0, vocab=512,
              rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16, n_experts=32, top_k=8,
              expert_ffn=512, n_shared=1, shared_ffn=512, name="moe-2k", prompt=12, steps=20)
# the 27B shape (d 5120, F 17408, five query heads per KV head) at two layers and a small vocabulary
DENSE_27B_2L = dict(configs.DENSE_27B, n_layers=2, vocab=512, name="dense-27b-2l", prompt=12, steps=20)
DENSE_27B_2L.pop("context", None)
TINY_FP8 = dict(configs.TINY, kv_dtype="fp8", name="tiny-fp8")
DENSE_9B_2L_FP8 = dict(configs.DENSE_9B, n_layers=2, vocab=512, kv_dtype="fp8", name="dense-9b-2l-fp8",
                       prompt=12, steps=20)
MOE_2K_FP8 = dict(MOE_2K, kv_dtype="fp8", name="moe-2k-fp8")
DENSE_27B_2L_FP8 = dict(DENSE_27B_2L, kv_dtype="fp8", name="dense-27b-2l-fp8")
# shapes with a single-launch instantiation
SINGLE_LAUNCH_SHAPES = ("tiny", "moe-2k", "dense-27b-2l", "tiny-fp8", "dense-9b-2l-fp8", "moe-2k-fp8",
                        "dense-27b-2l-fp8")
ROUTER_TAU = 1e-4


def _cuda_i32(v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


class Pair:
    """GPU session + oracle for one sequence, stepping both on the same tokens."""

    def __init__(self, cfg, seed, max_len, ctx0=0, synth_seed=None, gemm_min_rows=None, single=True):
        self.cfg = cfg
        self.s = Session(cfg, seed=seed, max_len=[max_len], max_tokens=4, pool_seed=seed + 100)
        self.single = bw.bw_set_single_launch(self.s.model, single)
        if gemm_min_rows is not None:
            bw.bw_set_gemm_min_rows(self.s.model, gemm_min_rows)
        self.om = oracle.Model(oracle_cfg(cfg), seed)
        self.okv = oracle.KV(self.om, 1, max_len - ctx0 + 1)
        if ctx0:
            self.s.synthesize(synth_seed, [ctx0])
            self.okv.set_synth(0, synth_seed, 0, ctx0)
        self.pos = ctx0
        self.moe = cfg.get("n_experts", 0) > 0
        self.adopted = 0

    def step(self, tokens):
        t = len(tokens)
        logits, am = self.s.step(_cuda_i32(list(tokens)), _cuda_i32([self.pos]), t=t)
        g = logits.cpu().numpy().astype(np.float64)
        gam = am.cpu().numpy()
        sel_in = None
        if self.moe:
            L, k = self.cfg["n_layers"], self.cfg["top_k"]
            ex = np.empty((L, t, k), dtype=np.int32)
            bw.bw_debug_read_experts(self.s.model, t, ex)
            sel_in = np.ascontiguousarray(ex.transpose(1, 0, 2))
        r = oracle.forward(self.om, self.okv, 0, list(tokens), self.pos, sel_in=sel_in, tau=ROUTER_TAU)
        assert r["rc"] == 0, "GPU expert selection is not a near tie of the oracle's"
        self.adopted += r["adopted"]
        self.pos += t
        return g, gam, r["logits"]

    def close(self):
        self.s.close()


def _compare(g, gam, o, where):
    err = float(np.max(np.abs(g - o)))
    assert err <= LOGITS_MAX_ABS, (where, err)
    for i in range(o.shape[0]):
        ot = int(np.argmax(o[i]))
        if top2_margin(o[i]) > TOKEN_MARGIN:
            assert int(gam[i]) == ot, (where, i, int(gam[i]), ot)
    return err


@pytest.mark.parametrize("cfg,seed,gemm,single", [(configs.TINY, 1001, None, 1), (configs.TINY, 1004, None, 2),
                                                  (configs.TINY, 1003, None, 0),
                                                  (MOE_SMALL, 1011, None, 1), (configs.TINY, 1002, 1, 0),
                                                  (MOE_SMALL, 1012, 1, 0), (MOE_2K, 1013, None, 1),
                                                  (MOE_2K, 1014, None, 2), (MOE_2K, 1015, None, 0),
                                                  (DENSE_27B_2L, 1016, None, 1), (TINY_FP8, 1041, None, 1),
                                                  (TINY_FP8, 1042, None, 0), (TINY_FP8, 1043, 1, 0),
                                                  (DENSE_9B_2L_FP8, 1044, None, 1), (MOE_2K_FP8, 1045, None, 1),
                                                  (DENSE_27B_2L_FP8, 1046, None, 1)],
                         ids=["tiny", "tiny-cooperative", "tiny-chain", "moe-small", "tiny-gemm", "moe-small-gemm",
                              "moe-2k", "moe-2k-cooperative", "moe-2k-chain", "dense-27b-2l", "tiny-fp8",
                              "tiny-fp8-chain", "tiny-fp8-gemm", "dense-9b-2l-fp8", "moe-2k-fp8", "dense-27b-2l-fp8"])
def test_prompt_then_greedy_decode(cfg, seed, gemm, single):
    """single: batch-1 steps as one launch (1: ordinary, 2: cooperative; shapes with an instantiation), 0: the
    kernel chain.
    gemm = 1 runs every dense matrix of every chain step on the matrix-core GEMM path."""
    prompt_len, steps = cfg.get("prompt", 16), cfg.get("steps", 32)
    rng = np.random.default_rng(seed)
    prompt = rng.integers(0, cfg["vocab"], prompt_len)
    p = Pair(cfg, seed, prompt_len + steps + 1, gemm_min_rows=gemm, single=single)
    if single and cfg["name"] in SINGLE_LAUNCH_SHAPES:
        assert p.single, "a model of this shape has the single-launch step"
    worst = 0.0
    try:
        for i, tok in enumerate(prompt):
            g, gam, o = p.step([int(tok)])
            worst = max(worst, _compare(g, gam, o, f"prompt {i}"))
        nxt = int(np.argmax(o[0]))
        for i in range(steps):
            g, gam, o = p.step([nxt])
            worst = max(worst, _compare(g, gam, o, f"decode {i}"))
            nxt = int(np.argmax(o[0]))  # teacher forcing on the oracle's token
        print(f"[result] {cfg['name']} max |logit diff| = {worst:.3e}, near-tie router sets adopted = {p.adopted}")
    finally:
        p.close()


DENSE_9B_2L = dict(configs.DENSE_9B, n_layers=2, vocab=4096, name="dense-9b-2l")


@pytest.mark.parametrize("cfg,single", [(configs.TINY, 1), (configs.TINY, 0), (DENSE_9B_2L, 1), (DENSE_9B_2L, 0)],
                         ids=["tiny-single", "tiny-chain", "9b-2l-single", "9b-2l-chain"])
def test_argmax_takes_the_lowest_index_on_planted_ties(cfg, single):
    """Greedy argmax with exact ties: an lm_head row copied onto another gives both vocabulary
    rows bitwise equal logits, and the step must then return the lower index (single launch,
    kernel chain and, with 8 rows, the batched GEMM path). Every row is also checked against a
    brute-force argmax of the step's own logits (first index of the maximum)."""
    seed, V = 1061, cfg["vocab"]
    s = Session(cfg, seed=seed, max_len=[16], max_tokens=8, pool_seed=seed + 1)
    try:
        got = bw.bw_set_single_launch(s.model, single)
        assert got or not single
        tok = _cuda_i32([7])

        def run():
            lg, am = s.step(tok, _cuda_i32([0]))
            return lg.cpu().numpy()[0], int(am.cpu()[0])

        lg0, a0 = run()
        assert a0 == int(np.argmax(lg0))
        # the winning row copied onto a lower row in another workgroup's range (or, if the winner is
        # row 0, onto a higher one): the tie must go to the lower index
        b = a0 // 2 if a0 >= 64 else a0 + V // 2
        bw.bw_debug_copy_lm_head_row(s.model, a0, b)
        lg1, a1 = run()
        assert lg1[a0].view(np.uint32) == lg1[b].view(np.uint32) and lg1[a0] == lg1.max()
        assert a1 == min(a0, b), (a0, b, a1)
        assert a1 == int(np.flatnonzero(lg1 == lg1.max())[0])
        # eight rows at once (verify shape, matrix-core GEMM and row-wise argmax)
        toks = [7, 7, 3, 100 % V, 7, 5, 9, 7]
        lg8, am8 = s.step(_cuda_i32(toks), _cuda_i32([0]), t=8)
        lg8, am8 = lg8.cpu().numpy(), am8.cpu().numpy()
        for i in range(8):
            assert int(am8[i]) == int(np.flatnonzero(lg8[i] == lg8[i].max())[0]), i
        assert bw.bw_check_device_error(s.model) == 0
        print(f"[result] planted tie ({'single launch' if got else 'chain'}) rows {a0} and {b}: argmax {a1}")
    finally:
        s.close()


@pytest.mark.parametrize("gemm", [None, 1], ids=["gemv", "gemm"])
def test_verify_step_equals_sequential_greedy(gemm):
    """Four tokens verified in one call (the accepted token plus three drafts equal to the greedy
    continuation) give the same per-position argmax as four single-token steps."""
    cfg, seed = configs.TINY, 1021
    rng = np.random.default_rng(seed)
    prompt = rng.integers(0, cfg["vocab"], 12)
    seq = Pair(cfg, seed, 40)
    ver = Pair(cfg, seed, 40, gemm_min_rows=gemm)
    try:
        for tok in prompt[:-1]:
            seq.step([int(tok)])
            ver.step([int(tok)])
        cur = int(prompt[-1])
        toks, am_seq, lg_seq = [], [], []
        for i in range(4):
            g, gam, o = seq.step([cur])
            toks.append(cur)
            am_seq.append(int(gam[0]))
            lg_seq.append(g[0])
            cur = int(np.argmax(o[0]))
        g4, gam4, o4 = ver.step(toks)
        _compare(g4, gam4, o4, "verify")
        for i in range(4):
            if top2_margin(o4[i]) > TOKEN_MARGIN:
                assert int(gam4[i]) == am_seq[i], i
        assert np.max(np.abs(g4 - np.stack(lg_seq))) <= LOGITS_MAX_ABS
    finally:
        seq.close()
        ver.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("single,kv", [(True, "bf16"), (False, "bf16"), (True, "fp8")],
                         ids=["single-launch", "chain", "single-launch-fp8"])
def test_dense_9b_synthesized_context(single, kv):
    cfg = dict(configs.DENSE_9B, kv_dtype=kv)
    ctx, steps, seed = 2048, 3, cfg["seed"]
    p = Pair(cfg, seed, ctx + steps + 1, ctx0=ctx, synth_seed=seed + 7, single=single)
    assert p.single or not single
    try:
        nxt = int(np.random.default_rng(seed).integers(0, cfg["vocab"]))
        worst = 0.0
        for i in range(steps):
            g, gam, o = p.step([nxt])
            worst = max(worst, _compare(g, gam, o, f"9b step {i}"))
            nxt = int(np.argmax(o[0]))
        print(f"[result] dense-9b {kv} cache ({'single launch' if single else 'chain'}) max |logit diff| = {worst:.3e}")
    finally:
        p.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("single,kv", [(True, "bf16"), (False, "bf16"), (True, "fp8")],
                         ids=["single-launch", "chain", "single-launch-fp8"])
def test_last_position_of_the_longest_context(single, kv):
    """The largest size a model allows (max_positions 65536): one step at position 65535 over a
    synthesised context of 65535 positions (4096 pages per layer), 9B layer shape, two layers."""
    cfg = dict(configs.DENSE_9B, n_layers=2, vocab=512, kv_dtype=kv, name="dense-9b-2l-longest")
    ctx, seed = 65535, 1051
    print(f"[case] longest context {ctx}, {kv} cache, {'single launch' if single else 'chain'}", flush=True)
    p = Pair(cfg, seed, ctx + 1, ctx0=ctx, synth_seed=seed + 7, single=single)
    assert p.single or not single
    try:
        g, gam, o = p.step([int(np.random.default_rng(seed).integers(0, cfg["vocab"]))])
        err = _compare(g, gam, o, "position 65535")
        print(f"[result] position 65535 ({kv}, {'single launch' if single else 'chain'}): max |logit diff| = {err:.3e}")
    finally:
        p.close()


# the verify workload's layer shape (9B dimensions), two layers and a small vocabulary so that
# the oracle checks every row of the batch
VERIFY_SMALL = dict(configs.VERIFY_9B, n_layers=2, vocab=4096, name="verify-9b-2l")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_batched_verify_ragged_contexts(kv):
    """Speculative verify over a ragged batch: 8 sequences with synthesised contexts of different
    lengths (U[40, 1200], ragged final pages), 4 tokens each, one step (32 rows on the matrix-core
    GEMM path). Every row against the oracle, which decodes each sequence on its own. An FP8 cache
    is widened to bf16 for the matrix-core attention."""
    cfg, seed = dict(VERIFY_SMALL, kv_dtype=kv), 1031
    B, t = 8, 4
    rng = np.random.default_rng(seed)
    lens = [int(v) for v in rng.integers(40, 1201, B)]
    lens[0], lens[1] = 47, 1200  # a one-token-short page and a page-aligned context
    s = Session(cfg, seed=seed, max_len=[n + t for n in lens], max_tokens=B * t, pool_seed=seed + 1)
    om = oracle.Model(oracle_cfg(cfg), seed)
    okv = oracle.KV(om, B, t + 1)
    try:
        s.poison()
        s.synthesize(seed + 7, lens)
        for b in range(B):
            okv.set_synth(b, seed + 7, b, lens[b])
        toks = rng.integers(0, cfg["vocab"], B * t).astype(np.int32)
        print(f"[case] verify batch {B} x t {t}, contexts {lens}", flush=True)
        logits, am = s.step(torch.from_numpy(toks).cuda(), _cuda_i32(lens), t=t)
        g = logits.cpu().numpy().astype(np.float64)
        gam = am.cpu().numpy()
        worst = 0.0
        for b in range(B):
            r = oracle.forward(om, okv, b, [int(v) for v in toks[b * t:(b + 1) * t]], lens[b])
            worst = max(worst, _compare(g[b * t:(b + 1) * t], gam[b * t:(b + 1) * t], r["logits"], f"seq {b}"))
        print(f"[result] verify batch max |logit diff| = {worst:.3e}")
    finally:
        okv.close()
        om.close()
        s.close()


def test_single_launch_matches_chain_over_many_steps():
    """The single-launch step and the kernel chain agree step by step on the same tokens (tiny,
    64 positions: every page, the ragged last page, both layers). Both are fp32 evaluations of the
    same step in different summation orders (and the single launch exchanges activations with 21
    mantissa bits), so their difference is bounded by the sum of their distances to the exact
    result; the bound used is a tenth of the logits tolerance against the oracle."""
    cfg, seed = configs.TINY, 1041
    rng = np.random.default_rng(seed)
    toks = rng.integers(0, cfg["vocab"], 64)
    a = Session(cfg, seed=seed, max_len=[65], max_tokens=1, pool_seed=seed + 1)
    b = Session(cfg, seed=seed, max_len=[65], max_tokens=1, pool_seed=seed + 2)
    try:
        assert bw.bw_set_single_launch(a.model, True)
        bw.bw_set_single_launch(b.model, False)
        worst = 0.0
        for i, tok in enumerate(toks):
            la, ma = a.step(_cuda_i32([int(tok)]), _cuda_i32([i]))
            lb, mb = b.step(_cuda_i32([int(tok)]), _cuda_i32([i]))
            ga, gb = la.cpu().numpy()[0], lb.cpu().numpy()[0]
            d = float(np.max(np.abs(ga - gb)))
            worst = max(worst, d)
            assert d <= LOGITS_MAX_ABS / 10, (i, d)
            if top2_margin(gb.astype(np.float64)) > TOKEN_MARGIN:
                assert int(ma.cpu()[0]) == int(mb.cpu()[0]), i
        for sess in (a, b):
            assert bw.bw_check_device_error(sess.model) == 0
        print(f"[result] single launch vs chain, 64 steps: max |logit diff| = {worst:.3e}")
    finally:
        a.close()
        b.close()


def test_single_launch_9b_layers_against_the_oracle_over_many_steps():
    """Two layers of the 9B shape (every matrix at its real size: the FFN by columns and its
    partial-sum exchange) over 64 single-launch steps from an empty cache, teacher-forced with
    seeded tokens, every step against the fp64 oracle at the contract tolerance (logits within
    2e-2, tokens equal wherever the top-2 margin exceeds 1e-2): 64 epochs of the exchange tags,
    every page and the ragged last one."""
    seed = 1043
    toks = np.random.default_rng(seed).integers(0, DENSE_9B_2L["vocab"], 64)
    print(f"[case] 9b-2l single launch, 64 steps against the oracle", flush=True)
    p = Pair(DENSE_9B_2L, seed, 65, single=True)
    try:
        assert p.single
        worst = 0.0
        for i, tok in enumerate(toks):
            g, gam, o = p.step([int(tok)])
            worst = max(worst, _compare(g, gam, o, f"9b-2l step {i}"))
        assert bw.bw_check_device_error(p.s.model) == 0
        print(f"[result] 9b-2l single launch, 64 steps: max |logit diff| against the oracle = {worst:.3e}")
    finally:
        p.close()


def test_single_launch_timeout_is_reported_and_recovers():
    """A wait that passes its deadline ends the single-launch step on every workgroup with
    BW_DERR_PERSIST (forced here with a zero deadline); later steps return at once until the
    error is read, after which the step runs normally again and matches the oracle."""
    cfg, seed = configs.TINY, 1051
    p = Pair(cfg, seed, 8)
    try:
        assert p.single
        bw.bw_debug_single_launch_deadline(p.s.model, 0)
        p.s.step(_cuda_i32([5]), _cuda_i32([0]))
        torch.cuda.synchronize()
        flags = bw.bw_check_device_error(p.s.model)
        print(f"[result] device flags after a zero-deadline step: {flags}")
        bw.bw_debug_single_launch_deadline(p.s.model, 50_000_000)
        if flags:
            assert flags & bw.BW_DERR_PERSIST, flags
        g, gam, o = p.step([5])
        _compare(g, gam, o, "after recovery")
        assert bw.bw_check_device_error(p.s.model) == 0
    finally:
        p.close()
