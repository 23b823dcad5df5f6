"""Chunked prefill (GPU): a prompt goes in as steps of up to `chunk` tokens (the matrix-core
GEMMs and the tiled matrix-core attention, causal within each chunk), the chunks before the last
skip the lm_head. Checked against the oracle, which decodes the whole prompt at once: the logits of
the prompt's last position, then greedy decode steps teacher-forced on the oracle's tokens, whose
attention reads every key and value the chunks wrote. Chunk sizes that do not divide the prompt or
the 16-token page leave ragged chunk and page ends."""
import numpy as np
import pytest
import torch

import oracle
from memory_bound_autoregressive_amd import configs
from memory_bound_autoregressive_amd.session import Session

from helpers import oracle_cfg
from test_gpu_e2e import VERIFY_SMALL, _compare, _cuda_i32

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg,prompt_len,chunk", [(configs.TINY, 50, 16), (configs.TINY, 45, 40),
                                                  (VERIFY_SMALL, 300, 128), (VERIFY_SMALL, 77, 77),
                                                  (VERIFY_SMALL, 700, 640)],
                         ids=["tiny-16", "tiny-40", "9b-layers-128", "9b-layers-one-chunk", "9b-layers-640"])
def test_chunked_prefill_matches_oracle(cfg, prompt_len, chunk):
    seed, steps = 1061, 6
    rng = np.random.default_rng(seed)
    prompt = [int(v) for v in rng.integers(0, cfg["vocab"], prompt_len)]
    print(f"[case] chunked prefill {cfg['name']}: {prompt_len} tokens in chunks of {chunk}", flush=True)
    s = Session(cfg, seed=seed, max_len=[prompt_len + steps + 1], max_tokens=chunk, pool_seed=seed + 1)
    om = oracle.Model(oracle_cfg(cfg), seed)
    okv = oracle.KV(om, 1, prompt_len + steps + 1)
    try:
        s.poison()
        last = s.prefill_chunked(prompt, chunk)
        torch.cuda.synchronize()
        ref = oracle.forward(om, okv, 0, prompt, 0)["logits"]
        g = last.cpu().numpy().astype(np.float64)[None, :]
        worst = _compare(g, np.array([int(np.argmax(g[0]))]), ref[-1:], "prompt end")
        nxt = int(np.argmax(ref[-1]))
        for i in range(steps):
            lg, am = s.step(_cuda_i32([nxt]), _cuda_i32([prompt_len + i]), t=1)
            o = oracle.forward(om, okv, 0, [nxt], prompt_len + i)["logits"]
            worst = max(worst, _compare(lg.cpu().numpy().astype(np.float64), am.cpu().numpy(), o, f"decode {i}"))
            nxt = int(np.argmax(o[0]))
        print(f"[result] chunked prefill {cfg['name']} {prompt_len}/{chunk}: max |logit diff| = {worst:.3e}")
    finally:
        okv.close()
        om.close()
        s.close()
