#!/usr/bin/env python3
"""Decode-step benchmark of libbw on one MI355X.

Workload (the measured configuration): 9B-shape dense decoder with int4 block weights (32 layers,
d_model 4096, 32 query / 8 KV heads of 128, SwiGLU 12288, vocab 151936, bf16 KV in 16-token pages),
batch 1, a 2048-token random prompt prefilled through the library, then `--steps` greedy decode
steps timed. Each step's argmax is fed back as the next token on the device; nothing returns to
the host inside the timed region.

Output: one JSON line (metric, value = decode tok/s, ...) plus
  - achieved step bandwidth: algorithmic bytes per step / step time, against 8 TB/s;
  - "roofline" of the dominant kernel. The step runs as one kernel launch (k_persist: all layers,
    the lm_head and the argmax), so that kernel is the step: algorithmic bytes per launch / its
    average launch time, timed with HIP events on the step's stream around each launch in a traced
    pass right after the timed region. "traffic" is the counted HBM bytes per launch from the
    committed FETCH_SIZE / WRITE_SIZE profile while the kernel's sources are unchanged and the
    profile's contexts lie within 64 positions of the traced pass's. With
    --chain the kernel chain is timed instead and the roofline is its gate/up GEMV;
  - "phases": per-layer wait / work time of each phase of the single-launch step, from GPU
    real-time-counter stamps written by one workgroup;
  - "cpu_baseline": the fp64 CPU oracle timed on this host on a bounded sample of the same
    workload (decode steps at the same context, the context synthesised rather than prefilled).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s at batch 1 (9B-shape int4) + achieved HBM GB/s vs ~8 TB/s peak"
HBM_PEAK_GBPS = 8000.0
PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)
INT4_BYTES_PER_WEIGHT = 18.0 / 32.0  # 16 bytes of codes + one fp16 scale per 32 weights


def kv_bytes(cfg: dict) -> int:
    """bytes per cached element: 2 (bf16, fp16) or 1 (FP8 E4M3)"""
    return 1 if cfg.get("kv_dtype", "bf16") == "fp8" else 2


def algorithmic_bytes(cfg: dict, ctx_mean: float) -> dict:
    """Bytes the step must move: active int4 weights, the KV read at the mean context, the new
    K/V written, one embedding row (router matrices for MoE)."""
    d, H, G, D, L = cfg["d_model"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["n_layers"]
    w_attn = ((H + 2 * G) * D * d + d * H * D) * L
    if cfg.get("n_experts", 0):
        per = 3 * cfg["expert_ffn"] * d * cfg["top_k"] + 3 * cfg["shared_ffn"] * d * cfg["n_shared"]
        w_ffn = per * L
        router = cfg["n_experts"] * d * 2 * L
    else:
        w_ffn = 3 * cfg["ffn_dim"] * d * L
        router = 0
    w_lm = cfg["vocab"] * d
    weights = (w_attn + w_ffn + w_lm) * INT4_BYTES_PER_WEIGHT
    es = kv_bytes(cfg)
    kv_read = ctx_mean * 2 * G * D * es * L
    kv_write = 2 * G * D * es * L
    embed = d * 2
    return {"weights": weights, "kv_read": kv_read, "kv_write": kv_write, "router": router,
            "embed": embed, "total": weights + kv_read + kv_write + router + embed}


# phase start / input-ready stamp slots of one layer in the single-launch step's record (16 per layer)
DENSE_PHASES = [("qkv", 0, 1), ("attention", 2, 3), ("merge", 4, 5), ("o", 6, 7), ("gate_up", 8, 9), ("down", 10, 11)]
# the 9B shape on 256 workgroups runs its FFN by columns: gate/up and the matching W_down columns in
# one pass, then each owner of residual rows adds the workgroups' partial sums
DENSE_PHASES_COLF = DENSE_PHASES[:4] + [("gate_up_down", 8, 9), ("down_reduce", 10, 11)]
MOE_PHASES = [("qkv", 0, 1), ("attention", 2, 3), ("merge", 4, 5), ("o", 6, 7), ("router", 8, 9),
              ("topk_gate_up", 10, 11), ("down", 12, 13)]


def ffn_by_columns(cfg) -> bool:
    """The single launch runs the dense FFN by columns for the 9B shape (d 4096, ffn 12288) on a
    GPU of 256 compute units (one workgroup per CU)."""
    import torch
    return (cfg.get("n_experts", 0) == 0 and cfg["d_model"] == 4096 and cfg["ffn_dim"] == 12288
            and torch.cuda.get_device_properties(0).multi_processor_count == 256)


def stamp_phases(run_once, L: int, moe: bool, n: int = 8, colf: bool = False) -> dict:
    """Per-layer wait ("wait_us": phase start until its input is in LDS) and work ("work_us": the
    rest, until the next phase starts) of each phase of the single-launch step, averaged over the
    layers of n steps, from workgroup 0's GPU real-time-counter stamps. run_once(stamps) runs one
    step with the stamp record `stamps` (int64 device tensor of L * 16 + 8) attached."""
    import numpy as np
    import torch
    slots = MOE_PHASES if moe else (DENSE_PHASES_COLF if colf else DENSE_PHASES)
    st = torch.zeros(L * 16 + 8, dtype=torch.int64, device="cuda")
    acc = np.zeros((len(slots), 2))
    lm = np.zeros(2)
    att = np.zeros(3)
    for _ in range(n):
        run_once(st)
        torch.cuda.synchronize()
        v = st.cpu().numpy().astype(np.float64) / 100.0  # us (100 MHz counter)
        per = v[:L * 16].reshape(L, 16)
        for i, (_, a, b) in enumerate(slots):
            if i + 1 < len(slots):
                end = per[:, slots[i + 1][1]]
            else:  # the next layer's first phase, or the lm_head after the last layer
                end = np.concatenate([per[1:, slots[0][1]], [v[L * 16]]])
            acc[i, 0] += np.mean(per[:, b] - per[:, a])
            acc[i, 1] += np.mean(end - per[:, b])
        lm += [v[L * 16 + 1] - v[L * 16], v[L * 16 + 3] - v[L * 16 + 1]]
        if not moe:  # attention work: page loop, wave reductions + barrier, cross-wave merge + stores
            att += [np.mean(per[:, 12] - per[:, 3]), np.mean(per[:, 13] - per[:, 12]), np.mean(per[:, 4] - per[:, 13])]
    out = {k: {"wait_us": round(float(acc[i, 0] / n), 2), "work_us": round(float(acc[i, 1] / n), 2)}
           for i, (k, _, _) in enumerate(slots)}
    out["lm_head"] = {"wait_us": round(float(lm[0] / n), 2), "work_us": round(float(lm[1] / n), 2)}
    if not moe:
        out["attention"]["work_split_us"] = {"page_loop": round(float(att[0] / n), 2),
                                             "wave_reduce": round(float(att[1] / n), 2),
                                             "merge_store": round(float(att[2] / n), 2)}
    return out


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traced_launch_us(step_fn, n: int) -> float:
    """Mean duration of one bw_decode_step launch: HIP events recorded on the step's stream right
    before and after the decode call only (bookkeeping kernels run outside the events)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a_, b_ in evs:
        step_fn(a_, b_)
    torch.cuda.synchronize()
    return sum(a_.elapsed_time(b_) for a_, b_ in evs) * 1000.0 / n


def cpu_baseline(cfg: dict, ctx: int, seconds: float) -> dict:
    """The oracle as it stands: fp64 decode steps at context `ctx` (synthesised), timed."""
    import numpy as np
    import oracle

    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "rms_eps",
            "rope_base", "kv_dtype", "n_experts", "top_k", "expert_ffn", "n_shared", "shared_ffn")
    om = oracle.Model({k: cfg[k] for k in keys if k in cfg}, cfg["seed"])
    kv = oracle.KV(om, 1, 64)
    kv.set_synth(0, cfg["seed"] + 7, 0, ctx)
    tok = int(np.random.default_rng(cfg["seed"]).integers(0, cfg["vocab"]))
    n, t0 = 0, time.perf_counter()
    while True:
        r = oracle.forward(om, kv, 0, [tok], ctx + n)
        tok = int(np.argmax(r["logits"][0]))
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 60:
            break
    om.close()
    return {"value": n / el, "unit": "tok/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} fp64 decode steps of the same model at context {ctx}..{ctx + n} "
                      f"(context synthesised, not prefilled), {el:.1f} s"}


def cpu_baseline_verify(cfg: dict, lens: list, t: int, seconds: float) -> dict:
    """The oracle on verify steps: sequences of the batch in order (shortest first), t positions
    each at its own synthesised context, until the time budget is spent."""
    import numpy as np
    import oracle

    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "rms_eps",
            "rope_base", "kv_dtype")
    om = oracle.Model({k: cfg[k] for k in keys if k in cfg}, cfg["seed"])
    order = np.argsort(lens)
    kv = oracle.KV(om, len(lens), t + 1)
    rng = np.random.default_rng(cfg["seed"])
    n, pos, t0 = 0, 0, time.perf_counter()
    done = []
    for b in order:
        kv.set_synth(int(b), cfg["seed"] + 7, int(b), lens[b])
        oracle.forward(om, kv, int(b), [int(v) for v in rng.integers(0, cfg["vocab"], t)], lens[b])
        n += 1
        pos += t
        done.append(lens[b])
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    kv.close()
    om.close()
    return {"value": pos / el, "unit": "positions/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
            "kind": "oracle", "sample": f"{n} fp64 verify steps of single sequences ({t} positions each, contexts "
                                        f"{done}, synthesised), {el:.1f} s"}


def committed_traffic(workload: str, cfg: dict, ctx: float):
    """Counted HBM bytes per launch of the single-launch step from a committed FETCH_SIZE /
    WRITE_SIZE profile of this workload whose kernel sources are unchanged and whose contexts lie
    within 64 positions of ctx (a workload may have profiles at several contexts); else None."""
    names = {"dense-9b": ["step_dense9b_traffic.json", "step_dense9b_traffic_ctx2600.json"],
             "dense-27b": ["step_dense27b_traffic_ctx8452.json"],
             "moe-35b-a3b": ["step_moe35b_traffic_ctx4612.json"]}.get(workload)
    kv = cfg.get("kv_dtype", "bf16")
    if names is None or kv != "bf16":
        return None
    from memory_bound_autoregressive_amd.build import source_digest
    for name in names:
        path = os.path.join(ROOT, "profiles", name)
        if not os.path.exists(path):
            continue
        with open(path) as f:
            tr = json.load(f)
        lo, hi = tr.get("contexts", (0, -1))
        if lo - 64 <= ctx <= hi + 64 and tr.get("kernel_source_digest") == source_digest(tuple(tr.get("kernel_sources", ()))):
            return round(tr["hbm_bytes_per_launch"])
    return None


def run_prefill(args) -> int:
    """Chunked prefill of the dense-9b workload's 2048-token prompt (chunks of --chunk tokens, one
    step each on the matrix-core path; logits for the last chunk only), timed over --steps runs
    after --warmup runs, each into a fresh cache state (positions restart at 0)."""
    import numpy as np
    import torch

    import memory_bound_autoregressive_amd as bw
    from memory_bound_autoregressive_amd import configs
    from memory_bound_autoregressive_amd.session import Session

    cfg = configs.DENSE_9B
    P, C = args.prompt, args.chunk
    K = args.steps if args.steps_set else 5
    W = args.warmup if args.warmup_set else 1
    torch.cuda.set_device(0)
    t_load = time.perf_counter()
    s = Session(cfg, seed=cfg["seed"], max_len=[P + 1], max_tokens=C, pool_seed=cfg["seed"] + 1)
    print(f"[bench] prefill-9b: model + pool ready in {time.perf_counter() - t_load:.1f} s", file=sys.stderr, flush=True)
    prompt = np.random.default_rng(cfg["seed"]).integers(0, cfg["vocab"], P).astype(np.int32)
    dev = "cuda"
    chunks = []
    for c0 in range(0, P, C):
        c1 = min(P, c0 + C)
        chunks.append((torch.from_numpy(prompt[c0:c1]).to(dev), torch.tensor([c0], dtype=torch.int32, device=dev), c1 - c0))
    logits = torch.empty((chunks[-1][2], cfg["vocab"]), dtype=torch.float32, device=dev)
    argmax = torch.empty(chunks[-1][2], dtype=torch.int32, device=dev)

    def run():
        for i, (tk, sl, t) in enumerate(chunks):
            last = i == len(chunks) - 1
            bw.bw_decode_step(s.model, s.pool, tk, sl, s.page_table, 1, t, s.max_pages,
                              logits if last else None, argmax if last else None)

    for _ in range(W):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        run()
    e1.record()
    torch.cuda.synchronize()
    if bw.bw_check_device_error(s.model) != 0:
        print("[bench] device error flag set", file=sys.stderr)
        return 1
    ms = e0.elapsed_time(e1) / K
    s.close()
    d, L = cfg["d_model"], cfg["n_layers"]
    H, G, D, F = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn_dim"]
    w_layers = ((H + 2 * G) * D * d + d * H * D + 3 * F * d) * L
    flop = 2.0 * w_layers * P + 2.0 * cfg["vocab"] * d * chunks[-1][2]  # weights x tokens (lm_head: last chunk)
    flop += 2.0 * 2 * H * D * L * P * (P + 1) / 2.0                     # causal attention (QK and PV)
    tflops = flop / (ms * 1e-3) / 1e12
    value = P * 1000.0 / ms
    print(f"[bench] prefill-9b: {P} tokens in chunks of {C}: {ms:.2f} ms, {value:.0f} tok/s, "
          f"{tflops:.1f} TFLOP/s of useful products", file=sys.stderr, flush=True)
    out = {
        "metric": "prefill tok/s (dense-9b, chunked)", "value": round(value, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (fp16 hi/lo and bf16 parts on the matrix cores)", "data": "synthetic",
        "config": {"workload": "prefill-9b", "prompt": P, "chunk": C, "chunks": len(chunks), "seed": cfg["seed"]},
        "useful_tflops": round(tflops, 2),
    }
    print(json.dumps(out))
    return 0


def run_tier(args) -> int:
    """kv-tier-9b: one dense-9b sequence's cache (context 16384: 1024 pages of 32 layers x 64 KiB)
    evicted to the pinned host tier and restored, timed with events on the caller's stream around
    each direction (each ends with the tier's dirty-page wait)."""
    import numpy as np
    import torch

    import memory_bound_autoregressive_amd as bw
    from memory_bound_autoregressive_amd import configs
    from memory_bound_autoregressive_amd.session import Session

    cfg = dict(configs.DENSE_9B)
    if args.kv:
        cfg["kv_dtype"] = args.kv
    ctx = 16384
    K = args.steps if args.steps_set else 5
    W = args.warmup if args.warmup_set else 1
    torch.cuda.set_device(0)
    s = Session(cfg, seed=cfg["seed"], max_len=[ctx + 1], max_tokens=1, pool_seed=cfg["seed"] + 1, spare_pages=0)
    s.synthesize(cfg["seed"] + 7, [ctx])
    tier = bw.bw_kv_tier_create(s.pool, s.n_pages)
    n_pg = (ctx + 15) // 16
    page_bytes = cfg["n_layers"] * 2 * cfg["n_kv_heads"] * 16 * cfg["head_dim"] * kv_bytes(cfg)
    moved = n_pg * page_bytes
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    d2h, h2d = [], []
    for it in range(W + K):
        bw.bw_kv_tier_touch(tier, s.page_table_host, np.array([ctx - 1], dtype=np.int32), 1, 1, s.max_pages)
        torch.cuda.synchronize()
        evs[0].record()
        pages, slots = bw.bw_kv_tier_evict_lru(tier, n_pg)
        bw.bw_kv_tier_wait(tier)
        evs[1].record()
        bw.bw_kv_tier_restore(tier, slots, pages)
        bw.bw_kv_tier_wait(tier)
        evs[2].record()
        torch.cuda.synchronize()
        assert len(pages) == n_pg
        if it >= W:
            d2h.append(evs[0].elapsed_time(evs[1]))
            h2d.append(evs[1].elapsed_time(evs[2]))
    bw.bw_kv_tier_free(tier)
    s.close()
    # the link as one contiguous copy of the same size each way (pinned host memory)
    dev_buf = torch.empty(moved, dtype=torch.uint8, device="cuda")
    host_buf = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    cp = []
    for it in range(2):
        evs[0].record()
        host_buf.copy_(dev_buf, non_blocking=True)
        evs[1].record()
        dev_buf.copy_(host_buf, non_blocking=True)
        evs[2].record()
        torch.cuda.synchronize()
        cp = [evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])]
    del dev_buf, host_buf
    link = [moved / (t * 1e-3) / 1e9 for t in cp]
    t_out, t_in = sum(d2h) / K, sum(h2d) / K
    gb_out, gb_in = moved / (t_out * 1e-3) / 1e9, moved / (t_in * 1e-3) / 1e9
    rt = 2 * moved / ((t_out + t_in) * 1e-3) / 1e9
    print(f"[bench] kv-tier-9b: {n_pg} pages ({moved / 2**30:.2f} GiB) out {t_out:.1f} ms ({gb_out:.1f} GB/s), "
          f"in {t_in:.1f} ms ({gb_in:.1f} GB/s); one contiguous copy: {link[0]:.1f} / {link[1]:.1f} GB/s",
          file=sys.stderr, flush=True)
    out = {
        "metric": "KV host-tier page migration GB/s (evict + restore, dense-9b pages)", "value": round(rt, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(t_out + t_in, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bytes", "data": "synthetic",
        "config": {"workload": "kv-tier-9b", "context": ctx, "pages": n_pg, "page_bytes_all_layers": page_bytes,
                   "kv": cfg.get("kv_dtype", "bf16"), "host_memory": "pinned (hipHostMalloc)",
                   "copies": "one 2-D DMA copy per page (32 layer slices) on the tier's stream"},
        "evict_gbps": round(gb_out, 2), "restore_gbps": round(gb_in, 2),
        "contiguous_copy_gbps": {"to_host": round(link[0], 2), "to_device": round(link[1], 2)},
        "roofline": {"bound": "pcie", "achieved": round(rt, 2), "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(rt / PCIE_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "DMA copies of the host tier (no kernel)"},
    }
    print(json.dumps(out))
    return 0


def run_workload(args) -> int:
    """The other timed workloads (synthesised contexts): dense-27b and moe-35b-a3b decode at batch 1
    (as one launch per step where the shape has one, else the kernel chain), and verify-9b, a speculative loop over 32 sequences (t = 4: the last
    committed token and three drafts drawn uniformly from the vocabulary, greedy acceptance on the
    device). One JSON line, like the default run, with this workload's own metric."""
    import numpy as np
    import torch

    import memory_bound_autoregressive_amd as bw
    from memory_bound_autoregressive_amd import configs
    from memory_bound_autoregressive_amd.session import Session

    cfg = dict(configs.ALL[args.workload])
    if args.kv:
        cfg["kv_dtype"] = args.kv
    seed, V = cfg["seed"], cfg["vocab"]
    K = args.steps if args.steps_set else cfg.get("steps", 512)
    W = args.warmup if args.warmup_set else 4
    dev = "cuda"
    torch.cuda.set_device(0)
    rng = np.random.default_rng(seed)
    t_load = time.perf_counter()
    if args.workload == "verify-9b":
        B, t = cfg["batch"], cfg["t"]
        lens = [int(v) for v in rng.integers(cfg["ctx_lo"], cfg["ctx_hi"] + 1, B)]
        s = Session(cfg, seed=seed, max_len=[n + (W + K + 2 + 8) * t for n in lens], max_tokens=B * t,
                    pool_seed=seed + 1)  # 8 more steps for the traced passes
        s.synthesize(seed + 7, lens)
    else:
        B, t = 1, 1
        lens = [args.context if args.context else cfg.get("context", cfg.get("prompt"))]
        # + 32 + 8: the traced pass and the phase-stamp pass after the timed steps
        s = Session(cfg, seed=seed, max_len=[lens[0] + W + K + 2 + 32 + 8], max_tokens=1, pool_seed=seed + 1)
        s.synthesize(seed + 7, lens)
    single = bool(bw.bw_set_single_launch(s.model, 0 if args.chain else 1)) and not args.chain and B * t == 1
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: model + pool ({s.n_pages} pages) ready in {time.perf_counter() - t_load:.1f} s",
          file=sys.stderr, flush=True)
    tokens = torch.from_numpy(rng.integers(0, V, B * t).astype(np.int32)).to(dev)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    argmax = torch.empty(B * t, dtype=torch.int32, device=dev)
    logits = torch.empty((B * t, V), dtype=torch.float32, device=dev) if t > 1 else None
    cap = 1024
    ring = torch.zeros(B * cap, dtype=torch.int32, device=dev)
    count = torch.zeros(B, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def step(ev=None):
        if t > 1:  # fresh drafts after each sequence's next input token
            tokens.view(B, t)[:, 1:] = torch.randint(0, V, (B, t - 1), generator=gen, device=dev, dtype=torch.int32)
        if ev is not None:
            ev[0].record()
        bw.bw_decode_step(s.model, s.pool, tokens, seq_lens, s.page_table, B, t, s.max_pages, logits, argmax)
        if ev is not None:
            ev[1].record()
        bw.bw_spec_accept(s.model, tokens, argmax, logits, seq_lens, ring, count, cap, None, B, t)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    ctx0 = seq_lens.cpu().numpy().astype(np.float64)
    c0 = int(count.sum().item())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    if bw.bw_check_device_error(s.model) != 0:
        print("[bench] device error flag set", file=sys.stderr)
        return 1
    ms_per_step = e0.elapsed_time(e1) / K
    committed = int(count.sum().item()) - c0
    ctx1 = seq_lens.cpu().numpy().astype(np.float64)
    kv_pos_layer = 2 * cfg["n_kv_heads"] * cfg["head_dim"] * kv_bytes(cfg)  # bytes per cached position and layer
    roofline, roofline_mfma, kernel_us, phases = None, None, {}, None
    if single and not args.no_trace:
        # the step is one kernel launch: events around the decode call only
        n_tr = 32
        launch_us = traced_launch_us(lambda a_, b_: step((a_, b_)), n_tr)
        ctx_tr = float(ctx1[0]) + (n_tr - 1) / 2.0
        bytes_tr = algorithmic_bytes(cfg, ctx_tr)["total"]
        achieved = bytes_tr / (launch_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": committed_traffic(args.workload, cfg, ctx_tr),
                    "kernel": f"k_persist: the whole batch-1 {args.workload} step in one launch",
                    "bytes_per_launch": round(bytes_tr), "avg_launch_us": round(launch_us, 2),
                    "context_mean": ctx_tr}
        kernel_us["k_persist"] = round(launch_us, 2)
        L = cfg["n_layers"]

        def run_stamped(st):
            bw.bw_debug_single_launch_stamps(s.model, st, L * 16 + 8)
            step()

        phases = stamp_phases(run_stamped, L, moe=cfg.get("n_experts", 0) > 0, colf=ffn_by_columns(cfg))
        bw.bw_debug_single_launch_stamps(s.model, None)
        if bw.bw_check_device_error(s.model) != 0:
            print("[bench] device error flag set in the traced passes", file=sys.stderr)
            return 1
        print(f"[bench] {args.workload}: k_persist {launch_us:.1f} us per launch; phases {phases}", file=sys.stderr,
              flush=True)
    elif t > 1 and not args.no_trace:
        # per-layer launch time of the attention (matrix-core split + merge) and the gate/up GEMM
        L = cfg["n_layers"]
        for cls in ("attn", "gate_up"):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * L)]
            for e in evs:  # torch creates its events lazily, at the first record
                e.record()
            torch.cuda.synchronize()
            arr = (ctypes.c_void_p * (2 * L))(*[ctypes.c_void_p(e.cuda_event) for e in evs])
            bw.bw_set_trace(s.model, cls, arr, L)
            tot, cnt = 0.0, 0
            sl_tr = []
            for _ in range(4):
                sl_tr.append(seq_lens.cpu().numpy().astype(np.float64))
                step()
                torch.cuda.synchronize()
                for l in range(L):
                    tot += evs[2 * l].elapsed_time(evs[2 * l + 1])
                    cnt += 1
            bw.bw_set_trace(s.model, cls, None, 0)
            kernel_us[cls] = round(1000.0 * tot / cnt, 2)
        # attention: every sequence's cached positions plus its t new ones, once per layer
        kv_layer = float(np.mean([(x + t).sum() for x in sl_tr])) * kv_pos_layer
        achieved = kv_layer / (kernel_us["attn"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                    "kernel": "verify attention per layer: k_attn_split_mfma (16 query rows per KV head, matrix "
                              "cores) + k_attn_merge", "bytes_per_launch": round(kv_layer),
                    "avg_launch_us": kernel_us["attn"]}
        d, F = cfg["d_model"], cfg["ffn_dim"]
        gu_flop = 2.0 * B * t * 2 * F * d
        tf = gu_flop / (kernel_us["gate_up"] * 1e-6) / 1e12
        roofline_mfma = {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": round(tf / 2500.0, 4), "traffic": None,
                         "kernel": f"gate/up int4 GEMM per layer ({B * t} x {2 * F} x {d}, fp16 matrix cores, "
                                   "k_gemm_w32 + epilogue); useful products only",
                         "flop_per_launch": gu_flop, "avg_launch_us": kernel_us["gate_up"]}
    if bw.bw_check_device_error(s.model) != 0:
        print("[bench] device error flag set in the traced passes", file=sys.stderr)
        return 1
    s.close()
    # algorithmic bytes per step: the weights once, each sequence's KV read at its mean context
    # over the timed steps (t positions attend, the later ones to the earlier: counted once),
    # the new K/V, and for verify the logits written
    ab1 = algorithmic_bytes(cfg, 0.0)
    # step k reads seq_lens_k + t positions; seq_lens grows by about one per step (drafts drawn at
    # random are almost never accepted; at t = 1 exactly one)
    ctx_mean = (ctx0 + ctx1) / 2.0 + t - 0.5
    kv_per_pos = 2 * cfg["n_kv_heads"] * cfg["head_dim"] * kv_bytes(cfg) * cfg["n_layers"]
    kv_read = float(ctx_mean.sum()) * kv_per_pos
    per_step = ab1["weights"] + ab1["router"] + kv_read + B * t * (kv_per_pos + ab1["embed"]) + \
        (B * t * V * 4 if t > 1 else 0)
    gbps = per_step / (ms_per_step * 1e-3) / 1e9
    kv_note = ", fp8 KV" if cfg.get("kv_dtype") == "fp8" else ""
    if t > 1:
        metric, value, unit = f"verified positions/s (verify-9b, 32 x 4 per step{kv_note})", B * t * 1000.0 / ms_per_step, "positions/s"
    else:
        metric, value, unit = f"decode tok/s at batch 1 ({args.workload} int4{kv_note})", 1000.0 / ms_per_step, "tok/s"
    print(f"[bench] {args.workload}: {K} steps, {ms_per_step * 1e3:.1f} us/step, {value:.1f} {unit}, "
          f"{gbps:.0f} GB/s algorithmic ({gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s)", file=sys.stderr, flush=True)
    out = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "step": "single launch" if single else "kernel chain (hipGraph replay)",
                   "batch": B, "t": t, "kv": cfg.get("kv_dtype", "bf16"),
                   "context": "synthesised", "context_range": [int(ctx0.min()), int(ctx1.max())],
                   "context_sum_start": int(ctx0.sum()), "seed": seed},
        "achieved_hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": round(per_step), "committed_tokens_per_s": round(committed * 1000.0 / (ms_per_step * K), 1),
        "kernel_us": kernel_us, "phases": phases, "roofline": roofline,
    }
    if roofline_mfma is not None:
        out["roofline_mfma"] = roofline_mfma
    if not args.no_cpu_baseline:
        if t > 1:
            out["cpu_baseline"] = cpu_baseline_verify(cfg, lens, t, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(cfg, lens[0], args.cpu_seconds)
        print(f"[bench] cpu baseline: {out['cpu_baseline']}", file=sys.stderr, flush=True)
    print(json.dumps(out))
    return 0


def run_mx(args) -> int:
    """mx-gemv-9b / mx-gemm-9b: the dense-9b model's weight matrices (32 layers of QKV, O, gate/up and
    down, then lm_head) in MXFP4, every matrix its own bytes in HBM. One step is one pass over all
    of them: batch 1 on the vector-unit GEMV (bw_mx_gemv) or M = 128 rows (the verify shape, 32
    sequences x 4 tokens) on the scaled matrix cores (bw_mx_gemm). Codes are uniform random bytes
    and E8M0 scales uniform on 117..121 (the generator's MXFP4 distribution), drawn on the device
    from a seeded generator; inputs are standard normal."""
    import numpy as np
    import torch

    import memory_bound_autoregressive_amd as bw
    from memory_bound_autoregressive_amd import configs

    gemm = args.workload == "mx-gemm-9b"
    cfg = configs.DENSE_9B
    d, L, V = cfg["d_model"], cfg["n_layers"], cfg["vocab"]
    H, G, D, F = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn_dim"]
    shapes = [((H + 2 * G) * D, d), (d, H * D), (2 * F, d), (d, F)] * L + [(V, d)]
    M = 128 if gemm else 1
    K = args.steps if args.steps_set else (20 if gemm else 100)
    W = args.warmup if args.warmup_set else 3
    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg["seed"])
    t0 = time.perf_counter()
    mats = []
    for N, Kd in shapes:
        c = torch.randint(0, 256, (N, Kd // 2), dtype=torch.uint8, device="cuda", generator=gen)
        sc = torch.randint(117, 122, (N, Kd // 32), dtype=torch.uint8, device="cuda", generator=gen)
        mats.append((c, sc))
    xin = {k: torch.randn((M, k), device="cuda", generator=gen) for k in {Kd for _, Kd in shapes}}
    yout = {n: torch.empty((M, n), device="cuda") for n in {N for N, _ in shapes}}
    ws = None
    if gemm:
        ws = torch.empty(max(bw.bw_mx_gemm_workspace_bytes(M, N, Kd) for N, Kd in shapes), dtype=torch.uint8,
                         device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: {len(shapes)} MXFP4 matrices ready in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)

    def one(i):
        (c, sc), (N, Kd) = mats[i], shapes[i]
        if gemm:
            bw.bw_mx_gemm(c, sc, xin[Kd], yout[N], ws)
        else:
            bw.bw_mx_gemv(c, sc, xin[Kd][0], yout[N][0])

    def step():
        for i in range(len(mats)):
            one(i)

    # One pass (129 launches) is captured once in a graph and replayed: launched one call at a time
    # from Python, the GPU would wait on the host between the small matrices' launches.
    step()
    torch.cuda.synchronize()
    eager = yout[V].clone()
    g_pass = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pass):
        step()
    # the lm_head alone, eight launches in one graph, for its own launch time
    g_lm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_lm):
        for _ in range(8):
            one(len(mats) - 1)
    for _ in range(W):
        g_pass.replay()
    torch.cuda.synchronize()
    if not torch.equal(yout[V], eager):
        print("[bench] graph replay differs from the eager pass", file=sys.stderr)
        return 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        g_pass.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    e0.record()
    for _ in range(4):
        g_lm.replay()
    e1.record()
    torch.cuda.synchronize()
    lm_us = e0.elapsed_time(e1) * 1e3 / 32
    # per launch: the pass time over its launches (each includes the graph's gap to the next launch)
    launch_us = [ms * 1e3 / len(mats)] * (len(mats) - 1) + [lm_us]
    wbytes = [N * Kd // 2 + N * Kd // 32 for N, Kd in shapes]
    xbytes = [M * Kd * 4 + M * N * 4 for N, Kd in shapes]
    step_bytes = sum(wbytes) + sum(xbytes)
    flops = sum(2.0 * M * N * Kd for N, Kd in shapes)
    kname = "k_mx_gemm" if gemm else "k_mx_gemv"
    if gemm:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": 5000.0, "unit": "TFLOP/s",
                "frac": round(ach / 5000.0, 4), "traffic": None,
                "kernel": "k_mx_gemm (with its X expansion and split-K reduction): E4M3 x E2M1 scaled products; "
                          "achieved counts useful products, the matrix cores issue three per weight (one per X term)",
                "flops_per_launch": round(flops / len(shapes)), "avg_launch_us": round(ms * 1e3 / len(shapes), 2),
                "issued_tflops": round(3 * ach, 1)}
        metric, value, unit = "MXFP4 GEMM useful TFLOP/s (dense-9b matrices, M = 128)", flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    else:
        ach = step_bytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(ach / 8000.0, 4), "traffic": None,
                "kernel": "k_mx_gemv: one MXFP4 matrix times one fp32 vector",
                "bytes_per_launch": round(step_bytes / len(shapes)), "avg_launch_us": round(ms * 1e3 / len(shapes), 2),
                "timing": "one pass captured in a graph and replayed; a launch's time includes the gap to the next",
                "lm_head_launch": {"bytes": wbytes[-1] + xbytes[-1], "us": round(launch_us[-1], 2),
                                   "gbps": round((wbytes[-1] + xbytes[-1]) / (launch_us[-1] * 1e-6) / 1e9, 1)}}
        metric, value, unit = "MXFP4 GEMV weight pass GB/s (dense-9b matrices, batch 1)", step_bytes / (ms * 1e-3) / 1e9, "GB/s"
    print(f"[bench] {args.workload}: {ms * 1e3:.1f} us per pass, {value:.1f} {unit}; roofline {roof['frac']}",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        import synth
        # the oracle's fp64 product on a bounded sample: 64 rows of a gate/up-shaped matrix
        rows, Kd = 64, d
        codes, scales = synth.mx_matrix(cfg["seed"], synth.UP, 0, 0, rows, Kd)
        X = np.random.default_rng(0).standard_normal((M, Kd))
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.mx_matmul(codes, scales, X)
            n += 1
        dt = time.perf_counter() - t0
        if gemm:
            cv = 2.0 * M * rows * Kd * n / dt / 1e12
            cpu = {"value": cv, "unit": "TFLOP/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
                   "kind": "oracle", "sample": f"{n} fp64 products of {M} x {Kd} by a {rows} x {Kd} MXFP4 matrix, {dt:.1f} s"}
        else:
            cv = (rows * Kd // 2 + rows * Kd // 32) * n / dt / 1e9
            cpu = {"value": cv, "unit": "GB/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
                   "kind": "oracle", "sample": f"{n} fp64 GEMVs of a {rows} x {Kd} MXFP4 matrix, {dt:.1f} s"}
        print(f"[bench] cpu baseline: {cpu}", file=sys.stderr, flush=True)
    out = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "E4M3 x E2M1 products (X in three scaled E4M3 terms), f32 accumulation" if gemm else
                 "f32 (E2M1 weights decoded exactly)",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": M, "matrices": len(shapes),
                   "weights": "MXFP4: E2M1 codes, one E8M0 scale per 32 (uniform 117..121)", "seed": cfg["seed"]},
        "weight_bytes_per_step": sum(wbytes), "bytes_per_step": step_bytes,
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prompt", type=int, default=2048)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--synth-context", action="store_true",
                    help="profiling aid: synthesise the --prompt positions of KV in the pool instead of "
                         "prefilling them (same bytes per step, far fewer launches under a counter profiler)")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--no-graphs", action="store_true",
                    help="kernel chain: launch the step's kernels directly instead of replaying a captured graph")
    ap.add_argument("--chain", action="store_true",
                    help="time the kernel chain instead of the single-launch step")
    ap.add_argument("--cooperative", action="store_true",
                    help="single-launch step through the cooperative launch API")
    ap.add_argument("--workload", default="dense-9b",
                    choices=("dense-9b", "dense-27b", "moe-35b-a3b", "verify-9b", "prefill-9b", "kv-tier-9b",
                             "mx-gemv-9b", "mx-gemm-9b"),
                    help="dense-9b (default): the headline line; the others time their own workload")
    ap.add_argument("--chunk", type=int, default=1024,
                    help="prefill-9b: tokens per prefill step (1024: 24.3 k tok/s against 18.7 k at 256)")
    ap.add_argument("--kv", choices=("bf16", "fp8"), default=None,
                    help="cache dtype of a decode or verify workload (default: the workload's own, bf16); "
                         "an FP8 E4M3 cache runs dense-9b on a synthesised context")
    ap.add_argument("--context", type=int, default=None,
                    help="dense-27b / moe-35b-a3b: synthesised context before the warm-up steps (default: "
                         "the workload's); a counter profile at the timed run's traced context uses it")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    args.steps_set = "--steps" in sys.argv
    args.warmup_set = "--warmup" in sys.argv
    if args.calibrate_copy:
        import torch
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 4}))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the decode step runs on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported. Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.workload == "prefill-9b":
        return run_prefill(args)
    if args.workload == "kv-tier-9b":
        return run_tier(args)
    if args.workload in ("mx-gemv-9b", "mx-gemm-9b"):
        return run_mx(args)
    if args.workload != "dense-9b" or args.kv not in (None, "bf16"):
        return run_workload(args)

    import numpy as np
    import torch

    import memory_bound_autoregressive_amd as bw
    from memory_bound_autoregressive_amd import configs
    from memory_bound_autoregressive_amd.session import Session

    cfg = configs.DENSE_9B
    P, W, K = args.prompt, args.warmup, args.steps
    n_traced = 64 + 8  # launches of the traced pass and of the phase-stamp pass after the timed steps
    total = P + W + K + n_traced + 1
    torch.cuda.set_device(0)
    t_load = time.perf_counter()
    s = Session(cfg, seed=cfg["seed"], max_len=[total], max_tokens=1, pool_seed=cfg["seed"] + 1)
    print(f"[bench] model + pool ready in {time.perf_counter() - t_load:.1f} s", file=sys.stderr, flush=True)
    if args.no_graphs:
        bw.bw_set_graphs(s.model, False)
    single = bw.bw_set_single_launch(s.model, 0 if args.chain else (2 if args.cooperative else 1)) and not args.chain
    dev = "cuda"
    prompt = torch.from_numpy(np.random.default_rng(cfg["seed"]).integers(0, cfg["vocab"], P).astype(np.int32)).to(dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    sl = torch.zeros(1, dtype=torch.int32, device=dev)
    am = torch.zeros(1, dtype=torch.int32, device=dev)
    am_sink = torch.zeros(1, dtype=torch.int32, device=dev)  # prefill: the argmax is not fed back

    def step(feed_back: bool, ev=None):
        # the decode step, then the library's greedy bookkeeping (t = 1): seq_lens += 1 and, when
        # feeding back, the argmax becomes the next input token; all on the device
        if ev is not None:
            ev[0].record()
        bw.bw_decode_step(s.model, s.pool, tok, sl, s.page_table, 1, 1, s.max_pages, None, am)
        if ev is not None:
            ev[1].record()
        bw.bw_spec_accept(s.model, tok if feed_back else am_sink, am, None, sl, None, None, 0, None, 1, 1)

    t_pf = time.perf_counter()
    if args.synth_context:
        # the pool holds P synthesised positions; decoding starts at position P from a seeded token
        s.synthesize(cfg["seed"] + 7, [P])
        tok.copy_(prompt[P - 1:P])
        sl.fill_(P)
        torch.cuda.synchronize()
        print(f"[bench] context of {P} positions synthesised in {time.perf_counter() - t_pf:.1f} s", file=sys.stderr,
              flush=True)
    else:
        # prefill: the prompt through the same decode step, one position at a time
        for i in range(P):
            tok.copy_(prompt[i:i + 1])
            step(feed_back=(i == P - 1))
        torch.cuda.synchronize()
        print(f"[bench] prefill of {P} tokens in {time.perf_counter() - t_pf:.1f} s", file=sys.stderr, flush=True)
    for _ in range(W):
        step(feed_back=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        step(feed_back=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    if bw.bw_check_device_error(s.model) != 0:
        print("[bench] device error flag set", file=sys.stderr)
        return 1
    ms_per_step = ms / K
    tok_s = 1000.0 / ms_per_step
    ctx_mean = P + W + (K - 1) / 2.0
    ab = algorithmic_bytes(cfg, ctx_mean)
    step_gbps = ab["total"] / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] {K} steps: {ms_per_step * 1e3:.1f} us/step, {tok_s:.1f} tok/s, "
          f"{step_gbps:.0f} GB/s algorithmic ({step_gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s)", file=sys.stderr, flush=True)

    kernel_us, roofline, phases = {}, None, None
    if not args.no_trace and single:
        # traced pass: each step is one kernel launch; HIP events on the step's stream around each
        # launch give the kernel's duration (the events sit outside the kernel, between launches)
        n_tr = 64
        launch_us = traced_launch_us(lambda a_, b_: step(feed_back=True, ev=(a_, b_)), n_tr)
        ctx_tr = P + W + K + (n_tr - 1) / 2.0
        bytes_tr = algorithmic_bytes(cfg, ctx_tr)["total"]
        achieved = bytes_tr / (launch_us * 1e-6) / 1e9
        # counted bytes per launch, measured at (about) this pass's context with unchanged sources
        traffic = committed_traffic("dense-9b", cfg, ctx_tr)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                    "kernel": "k_persist: the whole batch-1 step in one launch (32 layers + lm_head + argmax)",
                    "bytes_per_launch": round(bytes_tr), "avg_launch_us": round(launch_us, 2),
                    "context_mean": ctx_tr}
        kernel_us["k_persist"] = round(launch_us, 2)
        # per-phase timeline of one workgroup (GPU real-time counter stamps)
        L = cfg["n_layers"]

        def run_stamped(st):
            bw.bw_debug_single_launch_stamps(s.model, st, L * 16 + 8)
            step(feed_back=True)

        phases = stamp_phases(run_stamped, L, moe=False, colf=ffn_by_columns(cfg))
        bw.bw_debug_single_launch_stamps(s.model, None)
        if bw.bw_check_device_error(s.model) != 0:
            print("[bench] device error flag set in the traced passes", file=sys.stderr)
            return 1
        print(f"[bench] k_persist {launch_us:.1f} us per launch, {achieved:.0f} GB/s algorithmic; phases {phases}",
              file=sys.stderr, flush=True)
    elif not args.no_trace:
        L = cfg["n_layers"]
        classes = ["qkv", "attn", "o", "gate_up", "down", "lm_head"]
        n_trace = 8
        for cls in classes:
            n_pairs = 1 if cls == "lm_head" else L
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_pairs)]
            for e in evs:  # torch creates its events lazily, at the first record
                e.record()
            torch.cuda.synchronize()
            arr = (ctypes.c_void_p * (2 * n_pairs))(*[ctypes.c_void_p(e.cuda_event) for e in evs])
            bw.bw_set_trace(s.model, cls, arr, n_pairs)
            tot, cnt = 0.0, 0
            for _ in range(n_trace):
                step(feed_back=True)
                torch.cuda.synchronize()
                for l in range(n_pairs):
                    tot += evs[2 * l].elapsed_time(evs[2 * l + 1])
                    cnt += 1
            bw.bw_set_trace(s.model, cls, None, 0)
            kernel_us[cls] = round(1000.0 * tot / cnt, 2)
        d, F = cfg["d_model"], cfg["ffn_dim"]
        gu_bytes = 2 * F * d * INT4_BYTES_PER_WEIGHT
        achieved = gu_bytes / (kernel_us["gate_up"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                    "kernel": "chain: RMSNorm + gate/up int4 GEMV + SwiGLU (24576 x 4096)",
                    "bytes_per_launch": gu_bytes, "avg_launch_us": kernel_us["gate_up"]}
        print(f"[bench] per-launch kernel time (us): {kernel_us}", file=sys.stderr, flush=True)
    s.close()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, P + W, args.cpu_seconds)
        print(f"[bench] cpu baseline: {cpu}", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "dense-9b int4 decode: batch 1, 2048-token random prompt prefilled, greedy steps",
                   "step": "single launch" if single else "kernel chain (hipGraph replay)",
                   "batch": 1, "prompt": P, "context_range": [P + W, P + W + K], "weights": "int4 blocks of 32, fp16 scales",
                   "kv": "bf16, 16-token pages, permuted pool", "seed": cfg["seed"]},
        "achieved_hbm_gbps": round(step_gbps, 1), "hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": ab, "kernel_us": kernel_us, "phases": phases, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
