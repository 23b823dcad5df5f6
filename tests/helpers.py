"""Shared helpers of the parity tests (inputs, tolerances, comparisons)."""
from __future__ import annotations

import numpy as np

# tolerances of the decode step
KERNEL_REL_L2 = 1e-3      # per-kernel output, relative L2 over the whole output
LOGITS_MAX_ABS = 2e-2     # logits, max absolute difference per step
TOKEN_MARGIN = 1e-2       # greedy tokens must match wherever the oracle's top-2 margin exceeds this


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def top2_margin(logits: np.ndarray) -> float:
    part = np.partition(logits, -2)
    return float(part[-1] - part[-2])


def oracle_cfg(cfg: dict) -> dict:
    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "rms_eps",
            "rope_base", "kv_dtype", "n_experts", "top_k", "expert_ffn", "n_shared", "shared_ffn")
    return {k: cfg[k] for k in keys if k in cfg}


def kv_values(synth_mod, seed: int, layer: int, seq: int, n: int, G: int, D: int, dtype: int) -> np.ndarray:
    """Logical synthetic K/V [n][2][G][D] as fp64 values."""
    import torch
    bits = synth_mod.kv_fill(seed, layer, seq, 0, n, G, D, dtype)
    if dtype == synth_mod.KV_F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == synth_mod.KV_FP8:
        return torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
