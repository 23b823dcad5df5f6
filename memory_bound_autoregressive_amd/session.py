"""Host-side driver around the C-ABI: one model handle, one shared page pool, per-sequence page
tables, prefill and decode calls. This is plumbing for callers; every step runs in libbw.

Page mapping: the pool's physical page ids are a seeded Fisher-Yates permutation of
0..n_pages-1, handed out in logical order (sequence 0's pages first). A logical page j of
sequence b is physical page table[b][j] (bw24 deep-dive page, section 6 item 2).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (bw_decode_step, bw_kv_pool_create, bw_kv_pool_fill, bw_kv_pool_free, bw_kv_pool_synthesize,
               bw_model_free, bw_model_load_synthetic, make_config)

PAGE = 16


def pages_needed(n_tokens: int) -> int:
    return (n_tokens + PAGE - 1) // PAGE


class Session:
    def __init__(self, cfg: dict, *, seed: int, max_len: list[int], max_tokens: int, pool_seed: int = 7,
                 spare_pages: int = 4, model: int | None = None, device: str = "cuda"):
        """max_len[b]: the most positions sequence b will ever hold."""
        self.cfg = cfg
        self.batch = len(max_len)
        self.max_positions = max(max_len)
        self.own_model = model is None
        self.model = model if model is not None else bw_model_load_synthetic(
            make_config(cfg, self.max_positions, max_tokens), seed)
        need = [pages_needed(n) for n in max_len]
        self.max_pages = max(need)
        self.n_pages = sum(need) + spare_pages
        self.pool = bw_kv_pool_create(self.model, self.n_pages)
        perm = np.random.default_rng(pool_seed).permutation(self.n_pages).astype(np.int32)
        table = np.full((self.batch, self.max_pages), -1, dtype=np.int32)
        off = 0
        for b, n in enumerate(need):
            table[b, :n] = perm[off:off + n]
            off += n
        self.page_table_host = table
        self.page_table = torch.from_numpy(table).to(device)
        self.device = device

    def close(self):
        if getattr(self, "pool", None):
            bw_kv_pool_free(self.pool)
            self.pool = None
        if getattr(self, "own_model", False) and getattr(self, "model", None):
            bw_model_free(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def poison(self, bits: int | None = None) -> None:
        """Fill the whole pool with a NaN pattern (0x7FC0 is NaN in bf16 and fp16, 0x7F in FP8 E4M3)."""
        if bits is None:
            bits = 0x7F7F if self.cfg.get("kv_dtype", "bf16") == "fp8" else 0x7FC0
        bw_kv_pool_fill(self.pool, bits)
        torch.cuda.synchronize()

    def synthesize(self, seed: int, seq_lens: list[int], seq_ids: list[int] | None = None) -> None:
        ids = np.asarray(seq_ids if seq_ids is not None else range(self.batch), dtype=np.int32)
        lens = np.asarray(seq_lens, dtype=np.int32)
        bw_kv_pool_synthesize(self.pool, seed, ids, lens, np.ascontiguousarray(self.page_table_host),
                              self.batch, self.max_pages)

    def step(self, tokens: torch.Tensor, seq_lens: torch.Tensor, t: int = 1, *, logits: torch.Tensor | None = None,
             argmax: torch.Tensor | None = None, want_logits: bool = True):
        """One decode step (tokens [batch*t] int32, seq_lens [batch] int32, both on the device)."""
        M = self.batch * t
        if logits is None and want_logits:
            logits = torch.empty((M, self.cfg["vocab"]), dtype=torch.float32, device=self.device)
        if argmax is None:
            argmax = torch.empty(M, dtype=torch.int32, device=self.device)
        bw_decode_step(self.model, self.pool, tokens, seq_lens, self.page_table, self.batch, t, self.max_pages,
                       logits, argmax)
        return logits, argmax

    def prefill_chunked(self, prompt: list[int] | np.ndarray, chunk: int) -> torch.Tensor:
        """Prefill one sequence (batch 1) in chunks of up to `chunk` tokens, each one step with
        t = chunk rows (matrix-core GEMMs and attention); the chunks before the last ask for no
        logits, so they skip the lm_head (bw24 deep-dive page, section 5 stage 3: the prompt goes in
        chunks, the cache grows with each, logits come back for the last). Returns the logits of
        the prompt's last position. Needs max_tokens >= chunk."""
        assert self.batch == 1
        n = len(prompt)
        out = None
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            tk = torch.tensor([int(v) for v in prompt[c0:c1]], dtype=torch.int32, device=self.device)
            sl = torch.tensor([c0], dtype=torch.int32, device=self.device)
            if c1 == n:
                out, _ = self.step(tk, sl, t=c1 - c0)
            else:
                bw_decode_step(self.model, self.pool, tk, sl, self.page_table, 1, c1 - c0, self.max_pages, None, None)
        return out[-1]

    def prefill(self, prompt: list[int] | np.ndarray, b: int = 0) -> torch.Tensor:
        """Feed a prompt of one sequence (batch 1) token by token; returns the last logits."""
        assert self.batch == 1
        out = None
        for p, tok in enumerate(prompt):
            tk = torch.tensor([int(tok)], dtype=torch.int32, device=self.device)
            sl = torch.tensor([p], dtype=torch.int32, device=self.device)
            out, _ = self.step(tk, sl)
        return out
