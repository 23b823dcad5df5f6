"""Python binding of libbw.so, the MI355X (gfx950) int4 paged-KV decode-step library.

The functions here carry the C-ABI's names (include/bw.h) and only marshal arguments: torch
tensors become device pointers, the current torch stream becomes the hipStream_t. Every step
of the decode path runs in the library's HIP kernels. PyTorch provides device memory and
streams only. If libbw.so is missing, the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import configs  # noqa: F401  (workload shapes)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbw.so")

BW_OK, BW_EINVAL, BW_ENOMEM, BW_EHIP, BW_ERANGE, BW_ESTATE = 0, -1, -2, -3, -4, -5
BW_KV_F16, BW_KV_BF16, BW_KV_FP8 = 1, 2, 3
KV_DTYPES = {"f16": BW_KV_F16, "bf16": BW_KV_BF16, "fp8": BW_KV_FP8}
BW_DERR_PAGE, BW_DERR_TOKEN, BW_DERR_POS, BW_DERR_PERSIST = 1, 2, 4, 8
MAT = {"qkv": 0, "o": 1, "gate": 2, "up": 3, "down": 4, "lm_head": 5,
       "shared_gate": 6, "shared_up": 7, "shared_down": 8}

EXPORTS = (
    "bw_model_load_synthetic", "bw_model_free", "bw_kv_pool_create", "bw_kv_pool_free",
    "bw_kv_pool_fill", "bw_kv_pool_synthesize", "bw_kv_pool_synthesize_async", "bw_kv_pool_read", "bw_decode_step",
    "bw_last_error", "bw_check_device_error", "bw_debug_dequant", "bw_debug_matvec",
    "bw_debug_attention", "bw_debug_read_experts", "bw_debug_read_hidden", "bw_set_trace", "bw_set_graphs",
    "bw_set_gemm_min_rows", "bw_set_single_launch", "bw_debug_single_launch_deadline",
    "bw_debug_single_launch_stamps", "bw_spec_accept", "bw_debug_kv_round",
    "bw_kv_tier_create", "bw_kv_tier_free", "bw_kv_tier_touch", "bw_kv_tier_evict_lru", "bw_kv_tier_restore",
    "bw_kv_tier_wait", "bw_kv_tier_stats", "bw_kv_lru_select", "bw_model_export_tensor", "bw_model_tensor_bytes",
    "bw_debug_copy_lm_head_row", "bw_attention_noalloc", "bw_expert_tier_create", "bw_expert_tier_free",
    "bw_expert_tier_touch", "bw_expert_tier_evict_lru", "bw_expert_tier_restore", "bw_expert_tier_restore_routed",
    "bw_expert_tier_stats", "bw_mx_gemv", "bw_mx_gemm_workspace_bytes", "bw_mx_gemm",
)
KERNEL_CLASS = {"qkv": 0, "attn": 1, "o": 2, "gate_up": 3, "down": 4, "lm_head": 5, "router": 6,
                "moe_gate_up": 7, "moe_down": 8}


class BWError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed with {code}: {msg}")
        self.code = code


class bw_model_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_double),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("expert_ffn", ctypes.c_int32),
        ("n_shared", ctypes.c_int32), ("shared_ffn", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32), ("max_positions", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbw.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u64, sz, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_int64
        for name in EXPORTS:
            getattr(L, name).restype = i32
        L.bw_last_error.restype = ctypes.c_char_p
        L.bw_last_error.argtypes = []
        L.bw_model_load_synthetic.argtypes = [ctypes.POINTER(bw_model_config), u64, ctypes.POINTER(vp)]
        L.bw_model_free.argtypes = [vp]
        L.bw_kv_pool_create.argtypes = [vp, i32, ctypes.POINTER(vp)]
        L.bw_kv_pool_free.argtypes = [vp]
        L.bw_kv_pool_fill.argtypes = [vp, ctypes.c_uint16, vp]
        L.bw_kv_pool_synthesize.argtypes = [vp, u64, vp, vp, vp, i32, i32]
        L.bw_kv_pool_synthesize_async.argtypes = [vp, u64, vp, vp, vp, i32, i32, vp]
        L.bw_kv_pool_read.argtypes = [vp, i32, i32, vp, sz]
        L.bw_model_export_tensor.argtypes = [vp, ctypes.c_char_p, vp, sz]
        L.bw_model_tensor_bytes.argtypes = [vp, ctypes.c_char_p, ctypes.POINTER(sz)]
        L.bw_debug_copy_lm_head_row.argtypes = [vp, i32, i32]
        L.bw_attention_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, vp]
        L.bw_mx_gemv.argtypes = [vp, vp, vp, vp, i64, i64, vp]
        L.bw_mx_gemm_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
        L.bw_mx_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp]
        L.bw_expert_tier_create.argtypes = [vp, i32, ctypes.POINTER(vp)]
        L.bw_expert_tier_free.argtypes = [vp, vp]
        L.bw_expert_tier_touch.argtypes = [vp, i32, vp]
        L.bw_expert_tier_evict_lru.argtypes = [vp, i32, vp, vp, ctypes.POINTER(i32), vp]
        L.bw_expert_tier_restore.argtypes = [vp, i32, i32, vp]
        L.bw_expert_tier_restore_routed.argtypes = [vp, ctypes.POINTER(i32), vp]
        L.bw_expert_tier_stats.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.bw_decode_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
        L.bw_check_device_error.argtypes = [vp, vp, ctypes.POINTER(i32)]
        L.bw_debug_dequant.argtypes = [vp, i32, i32, i32, vp, vp]
        L.bw_debug_matvec.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp]
        L.bw_debug_attention.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, vp]
        L.bw_debug_kv_round.argtypes = [i32, vp, ctypes.c_int64, vp, vp, vp]
        L.bw_kv_tier_create.argtypes = [vp, i32, ctypes.POINTER(vp)]
        L.bw_kv_tier_free.argtypes = [vp]
        L.bw_kv_tier_touch.argtypes = [vp, vp, vp, i32, i32, i32]
        L.bw_kv_tier_evict_lru.argtypes = [vp, i32, vp, vp, vp, vp]
        L.bw_kv_tier_restore.argtypes = [vp, vp, vp, i32, vp]
        L.bw_kv_tier_wait.argtypes = [vp, vp]
        L.bw_kv_tier_stats.argtypes = [vp, vp, vp]
        L.bw_kv_lru_select.argtypes = [vp, vp, i32, i32, vp, vp]
        L.bw_debug_read_experts.argtypes = [vp, i32, vp, vp]
        L.bw_debug_read_hidden.argtypes = [vp, i32, vp, vp]
        L.bw_set_trace.argtypes = [vp, i32, vp, i32]
        L.bw_set_graphs.argtypes = [vp, i32]
        L.bw_set_gemm_min_rows.argtypes = [vp, i32]
        L.bw_set_single_launch.argtypes = [vp, i32, ctypes.POINTER(i32)]
        L.bw_debug_single_launch_deadline.argtypes = [vp, u64]
        L.bw_debug_single_launch_stamps.argtypes = [vp, vp, i32]
        L.bw_spec_accept.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, vp]
        _lib = L
    return _lib


def bw_last_error() -> str:
    return lib().bw_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc != BW_OK:
        raise BWError(rc, where, bw_last_error())


def _ptr(t) -> int | None:
    """Device (or host) pointer of a tensor / numpy array, or None."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(cfg: dict, max_positions: int, max_tokens: int) -> bw_model_config:
    kv = cfg.get("kv_dtype", "bf16")
    return bw_model_config(
        cfg["n_layers"], cfg["d_model"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"],
        cfg.get("ffn_dim", 0), cfg["vocab"], cfg.get("rms_eps", 1e-6), cfg.get("rope_base", 1e6),
        cfg.get("n_experts", 0), cfg.get("top_k", 0), cfg.get("expert_ffn", 0),
        cfg.get("n_shared", 0), cfg.get("shared_ffn", 0),
        KV_DTYPES[kv], cfg.get("page_tokens", 16), max_positions,
        max_tokens,
    )


# ---- the C-ABI, one Python function per entry point ---------------------------------------------

def bw_model_load_synthetic(cfg: bw_model_config, seed: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().bw_model_load_synthetic(ctypes.byref(cfg), seed, ctypes.byref(h)), "bw_model_load_synthetic")
    return h.value


def bw_model_free(model: int) -> None:
    _check(lib().bw_model_free(model), "bw_model_free")


def bw_kv_pool_create(model: int, n_pages: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().bw_kv_pool_create(model, n_pages, ctypes.byref(h)), "bw_kv_pool_create")
    return h.value


def bw_kv_pool_free(pool: int) -> None:
    _check(lib().bw_kv_pool_free(pool), "bw_kv_pool_free")


def bw_kv_pool_fill(pool: int, bits: int, stream=None) -> None:
    _check(lib().bw_kv_pool_fill(pool, bits, _stream(stream)), "bw_kv_pool_fill")


def bw_kv_pool_synthesize(pool: int, seed: int, seq_ids, seq_lens, page_table, batch: int, max_pages: int) -> None:
    """Host int32 numpy arrays."""
    _check(lib().bw_kv_pool_synthesize(pool, seed, _ptr(seq_ids), _ptr(seq_lens), _ptr(page_table), batch, max_pages),
           "bw_kv_pool_synthesize")


def bw_kv_pool_synthesize_async(pool: int, seed: int, seq_ids, seq_lens, page_table, batch: int, max_pages: int,
                                stream=None) -> None:
    """seq_ids (or None: sequence b has id b), seq_lens, page_table: int32 device tensors."""
    _check(lib().bw_kv_pool_synthesize_async(pool, seed, _ptr(seq_ids), _ptr(seq_lens), _ptr(page_table), batch,
                                             max_pages, _stream(stream)), "bw_kv_pool_synthesize_async")


def bw_model_tensor_bytes(model: int, name: str) -> int:
    n = ctypes.c_size_t()
    _check(lib().bw_model_tensor_bytes(model, name.encode(), ctypes.byref(n)), "bw_model_tensor_bytes")
    return n.value


def bw_model_export_tensor(model: int, name: str, out: np.ndarray) -> None:
    """out: host numpy array of exactly the tensor's size (uint8 codes, uint16 fp16 bits)."""
    _check(lib().bw_model_export_tensor(model, name.encode(), _ptr(out), out.nbytes), "bw_model_export_tensor")


def bw_expert_tier_create(model: int, host_slots: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().bw_expert_tier_create(model, host_slots, ctypes.byref(h)), "bw_expert_tier_create")
    return h.value


def bw_expert_tier_free(tier: int, stream=None) -> None:
    _check(lib().bw_expert_tier_free(tier, _stream(stream)), "bw_expert_tier_free")


def bw_expert_tier_touch(tier: int, n_rows: int, stream=None) -> None:
    _check(lib().bw_expert_tier_touch(tier, n_rows, _stream(stream)), "bw_expert_tier_touch")


def bw_expert_tier_evict_lru(tier: int, n: int, stream=None):
    """Returns (layers, experts) of the evicted experts, least recently routed first."""
    ls = np.empty(max(n, 1), dtype=np.int32)
    es = np.empty(max(n, 1), dtype=np.int32)
    got = ctypes.c_int32()
    _check(lib().bw_expert_tier_evict_lru(tier, n, _ptr(ls), _ptr(es), ctypes.byref(got), _stream(stream)),
           "bw_expert_tier_evict_lru")
    return ls[:got.value].copy(), es[:got.value].copy()


def bw_expert_tier_restore(tier: int, layer: int, expert: int, stream=None) -> None:
    _check(lib().bw_expert_tier_restore(tier, layer, expert, _stream(stream)), "bw_expert_tier_restore")


def bw_expert_tier_restore_routed(tier: int, stream=None) -> int:
    n = ctypes.c_int32()
    _check(lib().bw_expert_tier_restore_routed(tier, ctypes.byref(n), _stream(stream)), "bw_expert_tier_restore_routed")
    return n.value


def bw_expert_tier_stats(tier: int):
    r, h = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().bw_expert_tier_stats(tier, ctypes.byref(r), ctypes.byref(h)), "bw_expert_tier_stats")
    return r.value, h.value


def bw_debug_copy_lm_head_row(model: int, src: int, dst: int) -> None:
    _check(lib().bw_debug_copy_lm_head_row(model, src, dst), "bw_debug_copy_lm_head_row")


def bw_kv_pool_read(pool: int, layer: int, page: int, out) -> None:
    """out: host numpy array of one page-layer (uint16; uint8 for an FP8 cache)."""
    _check(lib().bw_kv_pool_read(pool, layer, page, _ptr(out), out.nbytes), "bw_kv_pool_read")


def bw_decode_step(model: int, pool: int, tokens, seq_lens, page_table, batch: int, t: int,
                   max_pages: int, logits=None, argmax=None, stream=None) -> None:
    """tokens/seq_lens/page_table/argmax: int32 device tensors; logits: float32 device tensor."""
    _check(lib().bw_decode_step(model, pool, _ptr(tokens), _ptr(seq_lens), _ptr(page_table), batch, t,
                                max_pages, _ptr(logits), _ptr(argmax), _stream(stream)), "bw_decode_step")


def bw_spec_accept(model: int, tokens, argmax, logits, seq_lens, ring, count, ring_cap: int, accepted,
                   batch: int, t: int, stream=None) -> None:
    """Greedy acceptance after a verify step (device tensors; logits, ring/count and accepted may
    be None). See include/bw.h."""
    _check(lib().bw_spec_accept(model, _ptr(tokens), _ptr(argmax), _ptr(logits), _ptr(seq_lens), _ptr(ring),
                                _ptr(count), int(ring_cap), _ptr(accepted), batch, t, _stream(stream)),
           "bw_spec_accept")


def bw_check_device_error(model: int, stream=None) -> int:
    flags = ctypes.c_int32(0)
    _check(lib().bw_check_device_error(model, _stream(stream), ctypes.byref(flags)), "bw_check_device_error")
    return flags.value


def bw_debug_dequant(model: int, which: str, layer: int, expert: int, out, stream=None) -> None:
    _check(lib().bw_debug_dequant(model, MAT[which], layer, expert, _ptr(out), _stream(stream)), "bw_debug_dequant")


def bw_debug_matvec(model: int, which: str, layer: int, expert: int, x, y, stream=None) -> None:
    _check(lib().bw_debug_matvec(model, MAT[which], layer, expert, _ptr(x), x.shape[0], _ptr(y), _stream(stream)),
           "bw_debug_matvec")


def bw_debug_attention(model: int, pool: int, layer: int, q, seq_lens, page_table, batch: int, t: int,
                       max_pages: int, out, stream=None) -> None:
    _check(lib().bw_debug_attention(model, pool, layer, _ptr(q), _ptr(seq_lens), _ptr(page_table), batch, t,
                                    max_pages, _ptr(out), _stream(stream)), "bw_debug_attention")


def bw_attention_noalloc(model: int, pool: int, layer: int, q, seq_lens, page_table, batch: int, t: int,
                         max_pages: int, out, stream=None) -> None:
    """bw_debug_attention with its split partials in the library's static device scratch (allocates
    nothing; calls on one GPU must not overlap). See include/bw.h."""
    _check(lib().bw_attention_noalloc(model, pool, layer, _ptr(q), _ptr(seq_lens), _ptr(page_table), batch, t,
                                      max_pages, _ptr(out), _stream(stream)), "bw_attention_noalloc")


def bw_mx_gemv(codes, scales, x, y, stream=None) -> None:
    """MXFP4 y = W x. codes: device uint8 [N][K/2]; scales: device uint8 E8M0 [N][K/32]; x: device
    float32 [K]; y: device float32 [N]."""
    N, K = codes.shape[0], codes.shape[1] * 2
    _check(lib().bw_mx_gemv(_ptr(codes), _ptr(scales), _ptr(x), _ptr(y), N, K, _stream(stream)), "bw_mx_gemv")


def bw_mx_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    n = ctypes.c_int64()
    _check(lib().bw_mx_gemm_workspace_bytes(M, N, K, ctypes.byref(n)), "bw_mx_gemm_workspace_bytes")
    return n.value


def bw_mx_gemm(codes, scales, X, Y, workspace, stream=None) -> None:
    """MXFP4 Y = X W^T. X: device float32 [M][K]; Y: device float32 [M][N]; workspace: device buffer of
    at least bw_mx_gemm_workspace_bytes(M, N, K) bytes."""
    N, K = codes.shape[0], codes.shape[1] * 2
    M = X.shape[0]
    _check(lib().bw_mx_gemm(_ptr(codes), _ptr(scales), _ptr(X), _ptr(Y), M, N, K, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)), "bw_mx_gemm")


def bw_debug_kv_round(kv_dtype: int, x, bits, back, stream=None) -> None:
    """x: device float32 [n]; bits: device int16/uint16 [n]; back: device float32 [n]."""
    _check(lib().bw_debug_kv_round(kv_dtype, _ptr(x), x.numel(), _ptr(bits), _ptr(back), _stream(stream)),
           "bw_debug_kv_round")


def bw_kv_tier_create(pool: int, host_pages: int) -> int:
    out = ctypes.c_void_p()
    _check(lib().bw_kv_tier_create(pool, host_pages, ctypes.byref(out)), "bw_kv_tier_create")
    return out.value


def bw_kv_tier_free(tier: int) -> None:
    _check(lib().bw_kv_tier_free(tier), "bw_kv_tier_free")


def bw_kv_tier_touch(tier: int, page_table, seq_lens, batch: int, tokens: int, max_pages: int) -> None:
    """page_table, seq_lens: host int32 numpy arrays."""
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    _check(lib().bw_kv_tier_touch(tier, _ptr(pt), _ptr(sl), batch, tokens, max_pages), "bw_kv_tier_touch")


def bw_kv_tier_evict_lru(tier: int, n: int, stream=None):
    """Returns (device pages, host slots) as int32 numpy arrays."""
    pages = np.empty(max(n, 1), dtype=np.int32)
    slots = np.empty(max(n, 1), dtype=np.int32)
    got = ctypes.c_int32()
    _check(lib().bw_kv_tier_evict_lru(tier, n, _ptr(pages), _ptr(slots), ctypes.byref(got), _stream(stream)),
           "bw_kv_tier_evict_lru")
    return pages[:got.value].copy(), slots[:got.value].copy()


def bw_kv_tier_restore(tier: int, host_slots, dev_pages, stream=None) -> None:
    hs = np.ascontiguousarray(host_slots, dtype=np.int32)
    dp = np.ascontiguousarray(dev_pages, dtype=np.int32)
    assert hs.size == dp.size
    _check(lib().bw_kv_tier_restore(tier, _ptr(hs), _ptr(dp), hs.size, _stream(stream)), "bw_kv_tier_restore")


def bw_kv_tier_wait(tier: int, stream=None) -> None:
    _check(lib().bw_kv_tier_wait(tier, _stream(stream)), "bw_kv_tier_wait")


def bw_kv_tier_stats(tier: int) -> tuple[int, int]:
    r, h = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().bw_kv_tier_stats(tier, ctypes.byref(r), ctypes.byref(h)), "bw_kv_tier_stats")
    return r.value, h.value


def bw_kv_lru_select(stamps, resident, n: int):
    """Host-only eviction order: stamps uint64 [n_pages], resident uint8 [n_pages]."""
    st = np.ascontiguousarray(stamps, dtype=np.uint64)
    rs = np.ascontiguousarray(resident, dtype=np.uint8)
    out = np.empty(max(n, 1), dtype=np.int32)
    got = ctypes.c_int32()
    _check(lib().bw_kv_lru_select(_ptr(st), _ptr(rs), st.size, n, _ptr(out), ctypes.byref(got)), "bw_kv_lru_select")
    return out[:got.value].copy()


def bw_debug_read_experts(model: int, n_rows: int, out, stream=None) -> None:
    _check(lib().bw_debug_read_experts(model, n_rows, _ptr(out), _stream(stream)), "bw_debug_read_experts")


def bw_debug_read_hidden(model: int, n_rows: int, out, stream=None) -> None:
    _check(lib().bw_debug_read_hidden(model, n_rows, _ptr(out), _stream(stream)), "bw_debug_read_hidden")


def bw_set_trace(model: int, kernel_class: str, events, n_layers: int) -> None:
    """events: a ctypes array of 2 * n_layers hipEvent_t handles (or None to clear)."""
    _check(lib().bw_set_trace(model, KERNEL_CLASS[kernel_class], events, n_layers), "bw_set_trace")


def bw_set_graphs(model: int, enable: bool) -> None:
    _check(lib().bw_set_graphs(model, int(bool(enable))), "bw_set_graphs")


def bw_set_single_launch(model: int, mode: int | bool) -> bool:
    """Batch-1 steps as one launch (mode 1 / True: ordinary launch, 2: cooperative launch) or as
    the kernel chain (0 / False); returns whether the model has the single-launch form."""
    avail = ctypes.c_int32(0)
    _check(lib().bw_set_single_launch(model, int(mode), ctypes.byref(avail)), "bw_set_single_launch")
    return bool(avail.value)


def bw_debug_single_launch_deadline(model: int, ticks: int) -> None:
    _check(lib().bw_debug_single_launch_deadline(model, int(ticks)), "bw_debug_single_launch_deadline")


def bw_debug_single_launch_stamps(model: int, stamps, n: int = 0) -> None:
    """stamps: a device int64 tensor of n >= 16 * n_layers + 8 entries, or None to stop."""
    _check(lib().bw_debug_single_launch_stamps(model, _ptr(stamps) if stamps is not None else None, int(n)),
           "bw_debug_single_launch_stamps")


def bw_set_gemm_min_rows(model: int, min_rows: int) -> None:
    _check(lib().bw_set_gemm_min_rows(model, int(min_rows)), "bw_set_gemm_min_rows")
