"""The host tier of the routed expert weights on the GPU (bw24 deep-dive page, section 6 item 3:
the VRAM tier holds the currently active experts, cold ones live in locked host memory).

A MoE model decodes a few steps while the tier records each step's routing. The least recently
routed experts are evicted to pinned host memory: their host copies equal the generator's
tensors byte for byte, and a step whose router picks some of them (the kernels then read those
experts over PCIe) gives logits bit-identical to a model that never moved an expert, and equal
to the oracle's within the logits tolerance. The experts that step routed to are restored
(hot experts come back), and the next step again matches bit for bit. Freeing the tier restores
every expert. Eviction order is checked against a brute-force LRU over the recorded routing."""
import numpy as np
import pytest
import torch

import oracle
import synth
import memory_bound_autoregressive_amd as bw
from memory_bound_autoregressive_amd.session import Session

from helpers import oracle_cfg
from test_gpu_e2e import ROUTER_TAU, _compare, _cuda_i32

pytestmark = pytest.mark.gpu

MOE_2K = dict(n_layers=2, d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=0, vocab=512,
              rms_eps=1e-6, rope_base=1e6, kv_dtype="bf16", page_tokens=16, n_experts=32, top_k=8,
              expert_ffn=512, n_shared=1, shared_ffn=512, name="moe-2k")


@pytest.mark.parametrize("single", [1, 0], ids=["single-launch", "chain"])
def test_expert_tier_evict_route_restore(single):
    cfg, seed = MOE_2K, 3001
    L, E, k, d, Fe = cfg["n_layers"], cfg["n_experts"], cfg["top_k"], cfg["d_model"], cfg["expert_ffn"]
    steps_before, n_evict = 4, 40
    rng = np.random.default_rng(seed)
    toks = [int(v) for v in rng.integers(0, cfg["vocab"], steps_before + 2)]
    ref = Session(cfg, seed=seed, max_len=[16], max_tokens=1, pool_seed=seed + 1)
    s = Session(cfg, seed=seed, max_len=[16], max_tokens=1, pool_seed=seed + 1)
    om = oracle.Model(oracle_cfg(cfg), seed)
    okv = oracle.KV(om, 1, 16)
    tier = None
    try:
        for x in (ref, s):
            assert bw.bw_set_single_launch(x.model, single), "the model has a single-launch form"
        tier = bw.bw_expert_tier_create(s.model, 64)
        stamp = np.zeros((L, E), dtype=np.int64)  # brute-force LRU state from the routing read back
        clock = 1

        def step(pos, tok):
            outs = []
            for x in (ref, s):
                lg, am = x.step(_cuda_i32([tok]), _cuda_i32([pos]))
                outs.append((lg.cpu().numpy()[0], am.cpu().numpy()))
            ex = np.empty((L, 1, k), dtype=np.int32)
            bw.bw_debug_read_experts(s.model, 1, ex)
            r = oracle.forward(om, okv, 0, [tok], pos, sel_in=np.ascontiguousarray(ex.transpose(1, 0, 2)),
                               tau=ROUTER_TAU)
            assert r["rc"] == 0
            return outs, ex[:, 0, :], r["logits"]

        for i in range(steps_before):
            [(lr, _), (ls, _)], sel, o = step(i, toks[i])
            assert np.array_equal(lr.view(np.uint32), ls.view(np.uint32))
            bw.bw_expert_tier_touch(tier, 1)
            for l in range(L):
                stamp[l, sel[l]] = clock
            clock += 1
        # evict: least recently routed first, ties to the lower (layer, expert)
        ls_, es_ = bw.bw_expert_tier_evict_lru(tier, n_evict)
        order = sorted(range(L * E), key=lambda i: (stamp[i // E, i % E], i))[:n_evict]
        assert [int(a) * E + int(b) for a, b in zip(ls_, es_)] == order
        assert bw.bw_expert_tier_stats(tier) == (L * E - n_evict, n_evict)
        torch.cuda.synchronize()
        on_host = set(order)
        print(f"[case] expert tier ({'single launch' if single else 'chain'}): {n_evict} experts on the host", flush=True)
        # host copies equal the generator's tensors
        for i in order[:6] + order[-2:]:
            l, e = i // E, i % E
            for m, kind, N, K in (("gate", synth.GATE, Fe, d), ("up", synth.UP, Fe, d), ("down", synth.DOWN, d, Fe)):
                codes, scales = synth.int4_matrix(seed, kind, l, 1 + e, N, K)
                name = f"layers.{l}.experts.{e}.{m}"
                got_c = np.empty(N * K // 2, dtype=np.uint8)
                got_s = np.empty(N * K // 32, dtype=np.uint16)
                bw.bw_model_export_tensor(s.model, name + ".codes", got_c)
                bw.bw_model_export_tensor(s.model, name + ".scales", got_s)
                assert np.array_equal(got_c.reshape(N, K // 2), codes), name
                assert np.array_equal(got_s.reshape(N, K // 32), scales), name
        # a step with experts on the host: bit for bit the untouched model's, and the oracle's
        pos = steps_before
        [(lr, ar), (ls, as_)], sel, o = step(pos, toks[pos])
        routed_host = {l * E + int(e) for l in range(L) for e in sel[l]} & on_host
        assert np.array_equal(lr.view(np.uint32), ls.view(np.uint32)) and np.array_equal(ar, as_)
        _compare(ls[None].astype(np.float64), as_, o, "experts on the host")
        assert bw.bw_check_device_error(s.model) == 0
        bw.bw_expert_tier_touch(tier, 1)
        n_back = bw.bw_expert_tier_restore_routed(tier)
        assert n_back == len(routed_host), (n_back, len(routed_host))
        assert bw.bw_expert_tier_stats(tier) == (L * E - n_evict + n_back, n_evict - n_back)
        print(f"[case] expert tier: the step routed to {len(routed_host)} experts on the host, restored", flush=True)
        # after the restore, again bit for bit
        pos += 1
        [(lr, ar), (ls, as_)], sel, o = step(pos, toks[pos])
        assert np.array_equal(lr.view(np.uint32), ls.view(np.uint32)) and np.array_equal(ar, as_)
        _compare(ls[None].astype(np.float64), as_, o, "after the restore")
        # bad arguments
        with pytest.raises(bw.BWError):
            bw.bw_expert_tier_restore(tier, 0, E)  # out of range
        resident = next(i for i in range(L * E) if i not in on_host)
        with pytest.raises(bw.BWError):
            bw.bw_expert_tier_restore(tier, resident // E, resident % E)  # already on the device
        bw.bw_expert_tier_free(tier)
        tier = None
        torch.cuda.synchronize()
        # every expert back on the device: the descriptors point at device regions again
        for i in order[:3]:
            l, e = i // E, i % E
            codes, _ = synth.int4_matrix(seed, synth.GATE, l, 1 + e, Fe, d)
            got_c = np.empty(Fe * d // 2, dtype=np.uint8)
            bw.bw_model_export_tensor(s.model, f"layers.{l}.experts.{e}.gate.codes", got_c)
            assert np.array_equal(got_c.reshape(Fe, d // 2), codes)
        print(f"[result] expert tier ({'single launch' if single else 'chain'}): evicted {n_evict}, "
              f"host-routed {len(routed_host)}, restored {n_back}; logits bit-identical to an unmoved model")
    finally:
        if tier:
            bw.bw_expert_tier_free(tier)
        okv.close()
        om.close()
        s.close()
        ref.close()
