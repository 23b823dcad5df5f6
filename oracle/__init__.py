"""fp64 CPU oracle of the int4 paged-KV decode step (ctypes view of oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the library under memory_bound_autoregressive_amd/ never
does. The oracle shares no code with the HIP path; both link only the seeded input generator
(synth/), which holds none of the method's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

KV_F16, KV_BF16, KV_FP8 = 1, 2, 3
KV_DTYPES = {"f16": KV_F16, "bf16": KV_BF16, "fp8": KV_FP8}


def build() -> str:
    """Compile oracle.c with gcc (fp64, OpenMP, no fast-math) and link the generator object."""
    obj = synth.OBJ if os.path.exists(synth.OBJ) else synth.build()
    subprocess.check_call([
        "gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
        "-std=c11", "-Wall", "-Wno-unknown-pragmas", SRC, obj, "-o", LIB, "-lm",
    ])
    return LIB


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_double), ("rope_base", ctypes.c_double),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("expert_ffn", ctypes.c_int32),
        ("n_shared", ctypes.c_int32), ("shared_ffn", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        vp, i64, i32, u64, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_double
        L.or_f16_to_f64.restype = dbl
        L.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_f64.restype = dbl
        L.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_f64_to_f16.restype = ctypes.c_uint16
        L.or_f64_to_f16.argtypes = [dbl]
        L.or_f64_to_bf16.restype = ctypes.c_uint16
        L.or_f64_to_bf16.argtypes = [dbl]
        L.or_fp8_to_f64.restype = dbl
        L.or_fp8_to_f64.argtypes = [ctypes.c_uint8]
        L.or_f64_to_fp8.restype = ctypes.c_uint8
        L.or_f64_to_fp8.argtypes = [dbl]
        L.or_code.restype = i32
        L.or_code.argtypes = [vp, i64]
        L.or_dequant.argtypes = [vp, vp, i64, i64, vp]
        L.or_quantize.argtypes = [vp, vp, i64, i64, vp]
        L.or_gemv.argtypes = [vp, vp, i64, i64, vp, vp]
        L.or_gemv_f16.argtypes = [vp, i64, i64, vp, vp]
        L.or_e2m1_to_f64.restype = dbl
        L.or_e2m1_to_f64.argtypes = [i32]
        L.or_e8m0_to_f64.restype = dbl
        L.or_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.or_mx_dequant.argtypes = [vp, vp, i64, i64, vp]
        L.or_mx_matmul.argtypes = [vp, vp, i64, i64, vp, i64, vp]
        L.or_rmsnorm.argtypes = [vp, vp, i64, dbl, vp]
        L.or_rope.argtypes = [vp, i32, i64, dbl]
        L.or_silu.restype = dbl
        L.or_silu.argtypes = [dbl]
        L.or_softmax.argtypes = [vp, i64, vp]
        L.or_argmax.restype = i64
        L.or_argmax.argtypes = [vp, i64]
        L.or_topk.argtypes = [vp, i64, i32, vp]
        L.or_attention.argtypes = [vp, vp, vp, i64, i32, vp, vp]
        L.or_attention_paged.argtypes = [vp, vp, vp, vp, i32, i64, i32, vp]
        L.or_model_create.restype = vp
        L.or_model_create.argtypes = [ctypes.POINTER(Config), u64]
        L.or_model_free.argtypes = [vp]
        L.or_model_matrix.restype = i32
        L.or_model_matrix.argtypes = [vp, i32, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.or_model_ffn.argtypes = [vp, i32, i32, i32, vp, vp]
        L.or_model_router_logits.argtypes = [vp, i32, vp, vp]
        L.or_model_moe_ffn.restype = i32
        L.or_model_moe_ffn.argtypes = [vp, i32, vp, vp, vp]
        L.or_model_moe_ffn_sel.restype = i32
        L.or_model_moe_ffn_sel.argtypes = [vp, i32, vp, vp, vp, vp, dbl, vp]
        L.or_kv_create.restype = vp
        L.or_kv_create.argtypes = [vp, i32, i64]
        L.or_kv_free.argtypes = [vp]
        L.or_kv_set_synth.argtypes = [vp, i32, u64, ctypes.c_uint32, i64]
        L.or_kv_set.restype = i32
        L.or_kv_set.argtypes = [vp, i32, i32, i64, vp]
        L.or_kv_read.restype = dbl
        L.or_kv_read.argtypes = [vp, i32, i32, i64, i32, i32, i32]
        L.or_forward.restype = i32
        L.or_forward.argtypes = [vp, vp, i32, vp, i32, i64, vp, vp, vp, vp, dbl, vp]
        L.or_num_threads.restype = i32
        L.or_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ---- primitives -------------------------------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return float(lib().or_f16_to_f64(int(bits)))


def bf16_to_f64(bits: int) -> float:
    return float(lib().or_bf16_to_f64(int(bits)))


def f64_to_f16(v: float) -> int:
    return int(lib().or_f64_to_f16(float(v)))


def f64_to_bf16(v: float) -> int:
    return int(lib().or_f64_to_bf16(float(v)))


def fp8_to_f64(bits: int) -> float:
    """OCP FP8 E4M3 bits -> value"""
    return float(lib().or_fp8_to_f64(int(bits)))


def f64_to_fp8(v: float) -> int:
    """value -> OCP FP8 E4M3 bits (nearest, ties to even, saturating at +-448)"""
    return int(lib().or_f64_to_fp8(float(v)))


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    N, K = codes.shape[0], codes.shape[1] * 2
    W = np.empty((N, K), dtype=np.float64)
    lib().or_dequant(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)), N, K, _p(W))
    return W


def quantize(W: np.ndarray, scales: np.ndarray) -> np.ndarray:
    N, K = W.shape
    codes = np.empty((N, K // 2), dtype=np.uint8)
    lib().or_quantize(_p(_f64(W)), _p(np.ascontiguousarray(scales, dtype=np.uint16)), N, K, _p(codes))
    return codes


def gemv(codes: np.ndarray, scales: np.ndarray, x) -> np.ndarray:
    N, K = codes.shape[0], codes.shape[1] * 2
    x = _f64(x)
    y = np.empty(N, dtype=np.float64)
    lib().or_gemv(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)), N, K, _p(x), _p(y))
    return y


def gemv_f16(W: np.ndarray, x) -> np.ndarray:
    N, K = W.shape
    x = _f64(x)
    y = np.empty(N, dtype=np.float64)
    lib().or_gemv_f16(_p(np.ascontiguousarray(W, dtype=np.uint16)), N, K, _p(x), _p(y))
    return y


def e2m1_to_f64(code: int) -> float:
    """OCP MX E2M1 code (4 bits) -> value"""
    return float(lib().or_e2m1_to_f64(int(code)))


def e8m0_to_f64(bits: int) -> float:
    """OCP MX E8M0 scale byte -> 2^(bits - 127) (NaN for 255)"""
    return float(lib().or_e8m0_to_f64(int(bits)))


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 matrix (codes uint8 [N][K/2], E8M0 scales uint8 [N][K/32]) -> fp64 [N][K]"""
    N, K = codes.shape[0], codes.shape[1] * 2
    W = np.empty((N, K), dtype=np.float64)
    lib().or_mx_dequant(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales, dtype=np.uint8)), N, K,
                        _p(W))
    return W


def mx_matmul(codes: np.ndarray, scales: np.ndarray, X) -> np.ndarray:
    """Y = X W^T for X [M][K] (or a vector [K]) against an MXFP4 matrix W [N][K], in fp64"""
    N, K = codes.shape[0], codes.shape[1] * 2
    X = _f64(X)
    vec = X.ndim == 1
    X2 = X.reshape(-1, K)
    Y = np.empty((X2.shape[0], N), dtype=np.float64)
    lib().or_mx_matmul(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales, dtype=np.uint8)), N, K,
                       _p(np.ascontiguousarray(X2)), X2.shape[0], _p(Y))
    return Y[0] if vec else Y


def rmsnorm(x, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    x = _f64(x)
    out = np.empty_like(x)
    lib().or_rmsnorm(_p(x), _p(np.ascontiguousarray(gamma_bits, dtype=np.uint16)), x.size, eps, _p(out))
    return out


def rope(v, pos: int, base: float) -> np.ndarray:
    v = _f64(v).copy()
    lib().or_rope(_p(v), v.size, pos, base)
    return v


def silu(z: float) -> float:
    return float(lib().or_silu(float(z)))


def softmax(s) -> np.ndarray:
    s = _f64(s)
    p = np.empty_like(s)
    lib().or_softmax(_p(s), s.size, _p(p))
    return p


def argmax(v) -> int:
    v = _f64(v)
    return int(lib().or_argmax(_p(v), v.size))


def topk(v, k: int) -> np.ndarray:
    v = _f64(v)
    idx = np.empty(k, dtype=np.int32)
    lib().or_topk(_p(v), v.size, k, _p(idx))
    return idx


def attention(q, K, V, with_probs: bool = False):
    q, K, V = _f64(q), _f64(K), _f64(V)
    n, D = K.shape
    out = np.empty(D, dtype=np.float64)
    probs = np.empty(max(n, 1), dtype=np.float64)
    lib().or_attention(_p(q), _p(K), _p(V), n, D, _p(out), _p(probs) if with_probs else None)
    return (out, probs[:n]) if with_probs else out


def attention_paged(q, Kpool, Vpool, page_table, page_tokens: int, n: int) -> np.ndarray:
    q, Kpool, Vpool = _f64(q), _f64(Kpool), _f64(Vpool)
    D = q.size
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    out = np.empty(D, dtype=np.float64)
    lib().or_attention_paged(_p(q), _p(Kpool), _p(Vpool), _p(pt), page_tokens, n, D, _p(out))
    return out


# ---- model --------------------------------------------------------------------------------------

class Model:
    """The oracle's model: weights regenerated from the seed by the shared generator."""

    def __init__(self, cfg: dict, seed: int):
        self.cfg = dict(cfg)
        self.seed = seed
        c = Config(
            cfg["n_layers"], cfg["d_model"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"],
            cfg.get("ffn_dim", 0), cfg["vocab"], cfg.get("rms_eps", 1e-6), cfg.get("rope_base", 1e6),
            cfg.get("n_experts", 0), cfg.get("top_k", 0), cfg.get("expert_ffn", 0),
            cfg.get("n_shared", 0), cfg.get("shared_ffn", 0),
            KV_DTYPES[cfg.get("kv_dtype", "bf16")],
        )
        self._c = c
        self.h = lib().or_model_create(ctypes.byref(c), seed)

    def close(self):
        if self.h:
            lib().or_model_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def matrix(self, which: str, layer: int = 0, expert: int = 0):
        """Canonical (codes, scales) of a generated matrix (views of oracle memory, copied)."""
        code = {"qkv": 0, "o": 1, "gate": 2, "up": 3, "down": 4, "lm_head": 5,
                "shared_gate": 6, "shared_up": 7, "shared_down": 8}[which]
        pc, ps = ctypes.c_void_p(), ctypes.c_void_p()
        N, K = ctypes.c_int64(), ctypes.c_int64()
        rc = lib().or_model_matrix(self.h, code, layer, expert, ctypes.byref(pc), ctypes.byref(ps),
                                   ctypes.byref(N), ctypes.byref(K))
        if rc != 0:
            raise KeyError(which)
        n, k = N.value, K.value
        codes = np.ctypeslib.as_array((ctypes.c_uint8 * (n * k // 2)).from_address(pc.value)).reshape(n, k // 2).copy()
        scales = np.ctypeslib.as_array((ctypes.c_uint16 * (n * k // 32)).from_address(ps.value)).reshape(n, k // 32).copy()
        return codes, scales

    def ffn(self, layer: int, h, expert: int = 0, shared: bool = False) -> np.ndarray:
        h = _f64(h)
        out = np.empty(self.cfg["d_model"], dtype=np.float64)
        lib().or_model_ffn(self.h, layer, expert, int(shared), _p(h), _p(out))
        return out

    def router_logits(self, layer: int, h) -> np.ndarray:
        h = _f64(h)
        r = np.empty(self.cfg["n_experts"], dtype=np.float64)
        lib().or_model_router_logits(self.h, layer, _p(h), _p(r))
        return r

    def moe_ffn(self, layer: int, h):
        h = _f64(h)
        out = np.empty(self.cfg["d_model"], dtype=np.float64)
        sel = np.empty(self.cfg["top_k"], dtype=np.int32)
        lib().or_model_moe_ffn(self.h, layer, _p(h), _p(out), _p(sel))
        return out, sel

    def moe_ffn_sel(self, layer: int, h, sel_in, tau: float):
        """MoE FFN with a proposed expert set (the near-tie rule): (rc, out, set used, adopted)."""
        h = _f64(h)
        k = self.cfg["top_k"]
        sin = np.ascontiguousarray(sel_in, dtype=np.int32)
        assert sin.shape == (k,)
        out = np.empty(self.cfg["d_model"], dtype=np.float64)
        sel = np.empty(k, dtype=np.int32)
        adopted = ctypes.c_int32(0)
        rc = lib().or_model_moe_ffn_sel(self.h, layer, _p(h), _p(out), _p(sin), _p(sel), tau,
                                        ctypes.byref(adopted))
        return rc, out, sel, adopted.value


class KV:
    """The oracle's logical KV state for n_seqs sequences."""

    def __init__(self, model: Model, n_seqs: int, cap: int):
        self.model = model
        self.h = lib().or_kv_create(model.h, n_seqs, cap)

    def close(self):
        if self.h:
            lib().or_kv_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_synth(self, seq: int, synth_seed: int, synth_seq: int, ctx0: int):
        lib().or_kv_set_synth(self.h, seq, synth_seed, synth_seq, ctx0)

    def read(self, seq: int, layer: int, pos: int, which: int, g: int, d: int) -> float:
        return float(lib().or_kv_read(self.h, seq, layer, pos, which, g, d))

    def set(self, seq: int, layer: int, pos: int, vals) -> None:
        """Store given keys and values [2][G][D] of one position (values already in the cache dtype)."""
        v = _f64(vals)
        assert v.shape == (2, self.model.cfg["n_kv_heads"], self.model.cfg["head_dim"])
        if lib().or_kv_set(self.h, seq, layer, pos, _p(v)) != 0:
            raise IndexError((seq, layer, pos))


def forward(model: Model, kv: KV, seq: int, tokens, pos0: int, *, want_logits=True,
            want_hidden=False, sel_in=None, tau: float = 0.0):
    """Decode len(tokens) tokens at positions pos0.. (all cached before any attends).

    Returns dict(logits [T][V], hidden [T][d], sel [T][L][k] (MoE), adopted, rc).
    """
    cfg = model.cfg
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    T = toks.size
    logits = np.empty((T, cfg["vocab"]), dtype=np.float64) if want_logits else None
    hidden = np.empty((T, cfg["d_model"]), dtype=np.float64) if want_hidden else None
    moe = cfg.get("n_experts", 0) > 0
    sel = np.empty((T, cfg["n_layers"], cfg["top_k"]), dtype=np.int32) if moe else None
    sin = np.ascontiguousarray(sel_in, dtype=np.int32) if (moe and sel_in is not None) else None
    adopted = ctypes.c_int32(0)
    rc = lib().or_forward(model.h, kv.h, seq, _p(toks), T, pos0,
                          _p(logits) if logits is not None else None,
                          _p(hidden) if hidden is not None else None,
                          _p(sel) if sel is not None else None,
                          _p(sin) if sin is not None else None, tau, ctypes.byref(adopted))
    return {"logits": logits, "hidden": hidden, "sel": sel, "adopted": adopted.value, "rc": rc}


def spec_accept(inputs, argmaxes):
    """Greedy acceptance of one verify step of one sequence.

    bw24 deep-dive page, section 1: speculative decoding must give exactly the tokens of plain
    token-by-token argmax decoding; section 5 stage 4: after the first draft that does not match,
    the later positions are masked.
    inputs = [x_0, ..., x_{t-1}]: x_0 is the last committed token, x_1.. the drafts;
    argmaxes[i] = the greedy token predicted after x_0..x_i.
    Draft x_{j+1} stands if every earlier draft stood and x_{j+1} == argmaxes[j].
    Returns (n drafts standing, committed tokens argmaxes[0..n], masked rows n+1..t-1).
    """
    n = 0
    while n + 1 < len(inputs) and int(inputs[n + 1]) == int(argmaxes[n]):
        n += 1
    return n, [int(v) for v in argmaxes[:n + 1]], list(range(n + 1, len(inputs)))


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    lib().or_set_num_threads(int(n))
