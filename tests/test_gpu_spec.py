"""Speculative decoding loop on the GPU: verify steps of t = 4 tokens (the last committed token
and three drafts) followed by the library's greedy acceptance (bw_spec_accept).

- Every step's bookkeeping (accepted count, committed tokens in the ring, seq_lens, the next
  input token, -inf rows) is compared exactly with the acceptance rule applied on the host
  (oracle.spec_accept) to the step's own argmaxes and drafts.
- The committed stream of each sequence equals the oracle's fp64 greedy continuation of its
  prompt, token for token, up to the first position where the oracle's top-2 margin is at most
  1e-2 (a near tie that either side may break differently; after one, the sequences diverge
  legitimately and comparison stops there).
- Draft policies, while a sequence has fewer than N tokens: sequence 0 drafts the true
  continuation (3 accepted per step), sequence 1 drafts wrong tokens (0 accepted, one token per
  step), sequence 2 drafts a random number r of correct tokens and then wrong ones (r accepted).
  A sequence that has N tokens drafts wrong tokens until the others catch up.
"""
import numpy as np
import pytest
import torch

import oracle
import memory_bound_autoregressive_amd as bw
from memory_bound_autoregressive_amd import configs
from memory_bound_autoregressive_amd.session import Session

from helpers import TOKEN_MARGIN, oracle_cfg, top2_margin

pytestmark = pytest.mark.gpu


def _oracle_greedy(cfg, seed, prompts, n_new):
    """fp64 greedy continuation of each prompt: tokens and the top-2 margin of each prediction"""
    om = oracle.Model(oracle_cfg(cfg), seed)
    okv = oracle.KV(om, len(prompts), len(prompts[0]) + n_new + 1)
    out = []
    try:
        for b, pr in enumerate(prompts):
            r = oracle.forward(om, okv, b, [int(v) for v in pr], 0)
            lg = r["logits"][-1]
            toks, margins = [], []
            for k in range(n_new):
                toks.append(int(np.argmax(lg)))
                margins.append(top2_margin(lg))
                lg = oracle.forward(om, okv, b, [toks[-1]], len(pr) + k)["logits"][0]
            out.append((toks, margins))
    finally:
        okv.close()
        om.close()
    return out


# the verify workload's layer shape (9B dimensions) at two layers and a small vocabulary
VERIFY_2L = dict(configs.VERIFY_9B, n_layers=2, vocab=4096, name="verify-9b-2l")


@pytest.mark.parametrize("cfg,B,N,gemm", [(configs.TINY, 3, 40, None), (configs.TINY, 3, 40, 1000),
                                          (VERIFY_2L, 32, 12, None)],
                         ids=["gemm", "gemv", "verify-9b-2l-batch32"])
def test_speculative_loop_commits_the_greedy_stream(cfg, B, N, gemm):
    """B sequences; the first three follow the draft policies above and are checked against the
    oracle's greedy stream. At the verify shape the other 29 sequences draft random tokens: their
    bookkeeping is checked every step, and the batch has 32 x 4 = 128 rows, so each step runs the
    wide matrix-core GEMM form and 16 query rows per KV head, as the verify workload does."""
    seed = 1051
    t, P = 4, 12
    V = cfg["vocab"]
    NC = 3  # sequences checked against the oracle
    rng = np.random.default_rng(seed)
    prompts = [rng.integers(0, V, P) for _ in range(B)]
    L_max = 2 * N + 2 * t  # the most tokens any sequence commits (sequence 0 after N: one per step)
    ref = _oracle_greedy(cfg, seed, prompts[:NC], L_max + t)
    cap = 64
    # room for every step's t tokens over the most steps the loop may take
    s = Session(cfg, seed=seed, max_len=[P + max(L_max, (N + 2) * t) + 2 * t] * B, max_tokens=B * t,
                pool_seed=seed + 1)
    try:
        if gemm is not None:
            bw.bw_set_gemm_min_rows(s.model, gemm)  # above B * t: the verify rows take the GEMV path
        dev = "cuda"
        # prompt positions 0..P-2 through plain steps of the whole batch; x_0 of the first
        # verify step is each prompt's last token, at position P - 1
        for i in range(P - 1):
            tk = torch.tensor([int(pr[i]) for pr in prompts], dtype=torch.int32, device=dev)
            s.step(tk, torch.full((B,), i, dtype=torch.int32, device=dev), t=1, want_logits=False)
        tokens = torch.zeros(B * t, dtype=torch.int32, device=dev)
        tokens[0::t] = torch.tensor([int(pr[-1]) for pr in prompts], dtype=torch.int32, device=dev)
        seq_lens = torch.full((B,), P - 1, dtype=torch.int32, device=dev)
        ring = torch.full((B * cap,), -1, dtype=torch.int32, device=dev)
        count = torch.zeros(B, dtype=torch.int32, device=dev)
        accepted = torch.zeros(B, dtype=torch.int32, device=dev)
        logits = torch.empty((B * t, V), dtype=torch.float32, device=dev)
        argmax = torch.empty(B * t, dtype=torch.int32, device=dev)
        committed = [[] for _ in range(B)]
        n_hist = [[] for _ in range(B)]
        keep_hist = [[] for _ in range(B)]
        steps = 0
        while min(len(c) for c in committed[:NC]) < N:
            # drafts from the reference continuation of what each sequence has committed
            tk_host = tokens.cpu().numpy()
            for b in range(B):
                if b >= NC:  # unchecked sequences of the batch: random drafts
                    tk_host[b * t + 1:(b + 1) * t] = rng.integers(0, V, t - 1)
                    keep_hist[b].append(0)
                    continue
                c = len(committed[b])
                truth = ref[b][0][c:c + t - 1]
                keep = {0: t - 1, 1: 0, 2: int(rng.integers(0, t))}[b] if c < N else 0
                keep_hist[b].append(keep)
                for j in range(t - 1):
                    tk_host[b * t + 1 + j] = truth[j] if j < keep else (truth[j] + 1 + int(rng.integers(0, V - 1))) % V
            tokens.copy_(torch.from_numpy(tk_host))
            sl_before = seq_lens.cpu().numpy().copy()
            s.step(tokens, seq_lens, t=t, logits=logits, argmax=argmax)
            lg_before = logits.cpu().numpy().copy()
            am = argmax.cpu().numpy().copy()
            bw.bw_spec_accept(s.model, tokens, argmax, logits, seq_lens, ring, count, cap, accepted, B, t)
            torch.cuda.synchronize()
            assert bw.bw_check_device_error(s.model) == 0
            lg_after = logits.cpu().numpy()
            tk_after, sl_after = tokens.cpu().numpy(), seq_lens.cpu().numpy()
            acc, cnt, rg = accepted.cpu().numpy(), count.cpu().numpy(), ring.cpu().numpy()
            for b in range(B):
                n, toks, masked = oracle.spec_accept(tk_host[b * t:(b + 1) * t], am[b * t:(b + 1) * t])
                assert int(acc[b]) == n, (steps, b)
                assert int(sl_after[b]) == int(sl_before[b]) + n + 1
                assert int(tk_after[b * t]) == toks[-1]
                c0 = len(committed[b])
                assert int(cnt[b]) == c0 + n + 1
                assert [int(rg[b * cap + (c0 + j) % cap]) for j in range(n + 1)] == toks
                for i in range(t):
                    row = b * t + i
                    if i in masked:
                        assert np.all(np.isneginf(lg_after[row])), (steps, b, i)
                    else:
                        assert np.array_equal(lg_after[row], lg_before[row])
                committed[b] += toks
                n_hist[b].append(n)
            steps += 1
            assert steps <= N + 2
            assert max(len(c) for c in committed[:NC]) <= L_max
        worst_stop = {}
        for b in range(NC):
            toks, margins = ref[b]
            for k in range(N):
                if committed[b][k] != toks[k]:
                    assert margins[k] <= TOKEN_MARGIN, (b, k, committed[b][k], toks[k], margins[k])
                    worst_stop[b] = k
                    break
        # with the streams in agreement, the draft policies give their acceptance counts
        for b in range(NC):
            if b not in worst_stop:
                if b == 0:
                    assert all(n == t - 1 for n in n_hist[0][:N // t - 1])
                if b == 1:
                    assert all(n == 0 for n in n_hist[1])
                if b == 2:
                    lens = np.cumsum([0] + [n + 1 for n in n_hist[2]])
                    for k, (n, kp) in enumerate(zip(n_hist[2], keep_hist[2])):
                        if lens[k] + t <= N:
                            assert n == kp, (k, n, kp)
        print(f"[result] speculative loop {cfg['name']} batch {B}: {steps} verify steps, committed "
              f"{[len(c) for c in committed[:NC]]}, accepted per step {[round(float(np.mean(h)), 2) for h in n_hist[:NC]]}, "
              f"near-tie stops {worst_stop}")
    finally:
        s.close()
