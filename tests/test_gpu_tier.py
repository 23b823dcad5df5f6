"""The host tier of the KV pool on the GPU (bw24 deep-dive page, section 6 item 3: cold pages go
to locked host memory, least recently used first, and come back before a read). Pages evicted to
pinned host memory and restored to other device pages give back every byte (the synthesised
context equals the generator's keys and values, the rest equals a pool that never moved), and a
decode step over the restored pages equals, bit for bit, one over pages that never moved, and
the oracle's step over the same context within the logits tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
import memory_bound_autoregressive_amd as bw
from memory_bound_autoregressive_amd import configs
from memory_bound_autoregressive_amd.session import Session, pages_needed

from helpers import oracle_cfg
from test_gpu_e2e import _compare

KV_CODE = {"f16": synth.KV_F16, "bf16": synth.KV_BF16, "fp8": synth.KV_FP8}

pytestmark = pytest.mark.gpu

LAYER9B_2L = dict(configs.DENSE_9B, n_layers=2, vocab=512, name="dense-9b-2l")


def _read_page(s, layer, page):
    es = 1 if s.cfg.get("kv_dtype") == "fp8" else 2
    buf = np.empty(s.cfg["n_kv_heads"] * 2 * 16 * s.cfg["head_dim"] * es, dtype=np.uint8)
    bw.bw_kv_pool_read(s.pool, layer, page, buf)
    return buf


@pytest.mark.parametrize("cfg", [configs.TINY, LAYER9B_2L, dict(LAYER9B_2L, kv_dtype="fp8")],
                         ids=["tiny", "9b-2l", "9b-2l-fp8"])
def test_evict_restore_round_trip_and_decode(cfg):
    seed, lens, steps = 2001, [40, 70, 33], 2
    B = len(lens)
    max_len = [n + steps + 2 for n in lens]
    ref = Session(cfg, seed=seed, max_len=max_len, max_tokens=B, pool_seed=5, spare_pages=0)
    s = Session(cfg, seed=seed, max_len=max_len, max_tokens=B, pool_seed=5, spare_pages=0)
    tier = None
    try:
        assert np.array_equal(ref.page_table_host, s.page_table_host)
        ref.synthesize(seed + 7, lens)
        s.synthesize(seed + 7, lens)
        tier = bw.bw_kv_tier_create(s.pool, s.n_pages)
        rng = np.random.default_rng(seed)
        toks = rng.integers(0, cfg["vocab"], (steps + 1, B)).astype(np.int32)
        for k in range(steps):
            sl = np.array(lens, dtype=np.int32) + k
            # step 0 touches every sequence, step 1 only sequences 0 and 2: sequence 1 is the oldest
            keep = [0, 1, 2] if k == 0 else [0, 2]
            bw.bw_kv_tier_touch(tier, s.page_table_host[keep], sl[keep], len(keep), 1, s.max_pages)
            for x in (ref, s):
                x.step(torch.from_numpy(toks[k]).cuda(), torch.from_numpy(sl).cuda())
        n_tok = [n + steps for n in lens]
        own = [s.page_table_host[b, :pages_needed(n_tok[b])].tolist() for b in range(B)]
        print(f"[case] tier {cfg['name']}: pages per sequence {[len(o) for o in own]}", flush=True)
        # least recently used first: sequence 1's pages (one stamp, so by id), then the others
        p1, h1 = bw.bw_kv_tier_evict_lru(tier, len(own[1]))
        assert p1.tolist() == sorted(own[1])
        p2, h2 = bw.bw_kv_tier_evict_lru(tier, 10 ** 6)
        assert p2.tolist() == sorted(own[0] + own[2])
        pages, slots = np.concatenate([p1, p2]), np.concatenate([h1, h2])
        assert len(set(slots.tolist())) == len(slots)
        assert bw.bw_kv_tier_stats(tier) == (0, len(pages))
        bw.bw_kv_tier_wait(tier)
        torch.cuda.synchronize()
        s.poison()  # every device page is now NaN: only the host copies hold the context
        # restore into a permutation of the same page ids and remap the page tables
        new = rng.permutation(pages).astype(np.int32)
        remap = dict(zip(pages.tolist(), new.tolist()))
        bw.bw_kv_tier_restore(tier, slots, new)
        bw.bw_kv_tier_wait(tier)
        table = s.page_table_host.copy()
        for b in range(B):
            for j in range(pages_needed(n_tok[b])):
                table[b, j] = remap[int(table[b, j])]
        s.page_table_host = table
        s.page_table = torch.from_numpy(table).cuda()
        torch.cuda.synchronize()
        assert bw.bw_kv_tier_stats(tier) == (len(pages), 0)
        G, D = cfg["n_kv_heads"], cfg["head_dim"]
        dt = np.uint8 if cfg.get("kv_dtype") == "fp8" else np.uint16
        for l in range(cfg["n_layers"]):
            for o, n in remap.items():
                assert np.array_equal(_read_page(s, l, n), _read_page(ref, l, o)), (l, o, n)
            # the synthesised context, restored, is the generator's: [tok][kv][g][d] -> page [g][kv][slot][d]
            for b in range(B):
                want = synth.kv_fill(seed + 7, l, b, 0, lens[b], G, D, KV_CODE[cfg.get("kv_dtype", "bf16")])
                for j in range(pages_needed(lens[b])):
                    page = _read_page(s, l, int(table[b, j])).view(dt).reshape(G, 2, 16, D)
                    n = min(16, lens[b] - 16 * j)
                    assert np.array_equal(page[:, :, :n, :], want[16 * j:16 * j + n].transpose(2, 1, 0, 3)), (l, b, j)
        sl = torch.from_numpy(np.array(n_tok, dtype=np.int32)).cuda()
        lr, ar = ref.step(torch.from_numpy(toks[steps]).cuda(), sl)
        ls, as_ = s.step(torch.from_numpy(toks[steps]).cuda(), sl.clone())
        torch.cuda.synchronize()
        assert torch.equal(lr.view(torch.int32), ls.view(torch.int32))
        assert torch.equal(ar, as_)
        assert bw.bw_check_device_error(s.model) == 0
        # the same three steps in the oracle, over the same synthesised context
        om = oracle.Model(oracle_cfg(cfg), seed)
        okv = oracle.KV(om, B, steps + 2)
        try:
            g, gam = ls.cpu().numpy().astype(np.float64), as_.cpu().numpy()
            for b in range(B):
                okv.set_synth(b, seed + 7, b, lens[b])
                for k in range(steps + 1):
                    o = oracle.forward(om, okv, b, [int(toks[k][b])], lens[b] + k)["logits"]
                _compare(g[b:b + 1], gam[b:b + 1], o, f"after restore, sequence {b}")
        finally:
            okv.close()
            om.close()
    finally:
        if tier:
            bw.bw_kv_tier_free(tier)
        s.close()
        ref.close()


def test_restore_rejects_bad_slots_and_pages():
    cfg = configs.TINY
    s = Session(cfg, seed=3, max_len=[40], max_tokens=1, pool_seed=5)
    tier = bw.bw_kv_tier_create(s.pool, 2)
    try:
        with pytest.raises(bw.BWError):
            bw.bw_kv_tier_restore(tier, [0], [0])  # slot 0 holds no page yet
        bw.bw_kv_tier_touch(tier, s.page_table_host, np.array([20], dtype=np.int32), 1, 1, s.max_pages)
        pages, slots = bw.bw_kv_tier_evict_lru(tier, 5)  # only 2 host slots
        assert len(pages) == 2
        with pytest.raises(bw.BWError):
            bw.bw_kv_tier_restore(tier, slots, [s.n_pages, 0])  # page id out of range
        with pytest.raises(bw.BWError):
            bw.bw_kv_tier_restore(tier, [slots[0], slots[0]], [0, 1])  # repeated slot
        bw.bw_kv_tier_restore(tier, slots, pages)
        bw.bw_kv_tier_wait(tier)
        torch.cuda.synchronize()
    finally:
        bw.bw_kv_tier_free(tier)
        s.close()
