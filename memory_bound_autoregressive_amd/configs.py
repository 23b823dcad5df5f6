"""The five synthetic workloads the decode step is built and measured on.

Each entry gives the model shape and the run shape. Weights are random-init from a seed
(int4 blocks of 32 with one fp16 scale, w = scale * (q - 8)); embeddings and norm gains are
fp16; the KV cache is paged at 16 tokens.
"""
from __future__ import annotations

TINY = dict(
    name="tiny", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=1024,
    vocab=1024, rms_eps=1e-6, rope_base=1e6, kv_dtype="f16", page_tokens=16,
    # run: batch 1, 16-token random prompt, then 32 greedy decode steps; pool randomly permuted
    batch=1, prompt=16, steps=32, seed=1001,
)

DENSE_9B = dict(
    name="dense-9b", n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
    ffn_dim=12288, vocab=151936, rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16,
    # run: batch 1, 2048-token random prompt prefilled, then 512 greedy decode steps timed
    batch=1, prompt=2048, steps=512, seed=1002,
)

DENSE_27B = dict(
    name="dense-27b", n_layers=64, d_model=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
    ffn_dim=17408, vocab=151936, rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16,
    # run: batch 1, context grown from 8192 to 8448 over 256 greedy decode steps
    batch=1, context=8192, steps=256, seed=1003,
)

MOE_35B_A3B = dict(
    name="moe-35b-a3b", n_layers=40, d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
    ffn_dim=0, vocab=151936, rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16,
    n_experts=256, top_k=8, expert_ffn=512, n_shared=1, shared_ffn=512,
    # run: batch 1, 4096-token context, 512 greedy decode steps
    batch=1, context=4096, steps=512, seed=1004,
)

VERIFY_9B = dict(
    DENSE_9B, name="verify-9b",
    # run: 32 sequences, ragged contexts uniform in [1024, 32768], 4 query tokens per sequence
    # per step (1 accepted + 3 drafts drawn uniformly from the vocabulary), causal, 64 steps
    batch=32, t=4, ctx_lo=1024, ctx_hi=32768, steps=64, seed=1005,
)
VERIFY_9B.pop("prompt", None)

ALL = {c["name"]: c for c in (TINY, DENSE_9B, DENSE_27B, MOE_35B_A3B, VERIFY_9B)}


def model_keys(cfg: dict) -> dict:
    """Only the model-shape fields of a workload."""
    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
            "rms_eps", "rope_base", "kv_dtype", "page_tokens", "n_experts", "top_k", "expert_ffn",
            "n_shared", "shared_ffn")
    return {k: cfg[k] for k in keys if k in cfg}
