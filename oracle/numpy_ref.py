"""A second, vectorised NumPy fp64 oracle of the decode step, for small configurations.

TEST INFRASTRUCTURE ONLY. It is written independently of oracle.c (array operations instead of
loops, NumPy's own fp16 decoding, a logical KV list instead of the C state) so that agreement
between the two catches a slip in either one. Same definition: int4 blocks of 32 with
w = scale * (q - 8), RMSNorm x / sqrt(mean(x^2) + eps) * gamma, rotate-half RoPE on pairs
(i, i + D/2), GQA attention with scale 1/sqrt(D), SwiGLU, softmax top-k routing with
renormalised gates plus an ungated shared expert, untied lm_head.
"""
from __future__ import annotations

import numpy as np

import synth


def f16(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [N][K/2] canonical, scales [N][K/32] fp16 bits -> W [N][K] fp64."""
    N = codes.shape[0]
    blocks = codes.reshape(N, -1, 16)  # [N][K/32][16]
    lo = (blocks & 0x0F).astype(np.int64)
    hi = (blocks >> 4).astype(np.int64)
    q = np.concatenate([lo, hi], axis=2)  # element i (low) then element i + 16 (high)
    w = (q - 8).astype(np.float64) * f16(scales)[:, :, None]
    return w.reshape(N, -1)


def round_kv(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float64)
    if dtype != "bf16":
        raise NotImplementedError(f"the NumPy twin models fp16 and bf16 caches only, not {dtype}")
    # bf16 round-to-nearest-even via the binary32 pattern (v is fp64: go through fp32 exactly
    # only when representable; use integer rounding on the fp64 mantissa instead)
    m, e = np.frexp(v)  # v = m * 2^e, |m| in [0.5, 1)
    scaled = np.ldexp(m, 8)  # 8 significant bits
    r = np.round(scaled)  # numpy rounds half to even
    return np.ldexp(r, e - 8)


class NumpyModel:
    def __init__(self, cfg: dict, seed: int):
        self.cfg = cfg
        self.seed = seed
        L, d = cfg["n_layers"], cfg["d_model"]
        H, G, D = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        self.Wqkv = [dequant(*synth.int4_matrix(seed, synth.QKV, l, 0, (H + 2 * G) * D, d)) for l in range(L)]
        self.Wo = [dequant(*synth.int4_matrix(seed, synth.O, l, 0, d, H * D)) for l in range(L)]
        self.g_attn = [f16(synth.norm_gain(seed, synth.ATTN_NORM, l, d)) for l in range(L)]
        self.g_ffn = [f16(synth.norm_gain(seed, synth.FFN_NORM, l, d)) for l in range(L)]
        self.g_final = f16(synth.norm_gain(seed, synth.FINAL_NORM, 0, d))
        self.Wlm = dequant(*synth.int4_matrix(seed, synth.LM_HEAD, 0, 0, cfg["vocab"], d))
        self.moe = cfg.get("n_experts", 0) > 0
        if not self.moe:
            F = cfg["ffn_dim"]
            self.Wg = [dequant(*synth.int4_matrix(seed, synth.GATE, l, 0, F, d)) for l in range(L)]
            self.Wu = [dequant(*synth.int4_matrix(seed, synth.UP, l, 0, F, d)) for l in range(L)]
            self.Wd = [dequant(*synth.int4_matrix(seed, synth.DOWN, l, 0, d, F)) for l in range(L)]
        else:
            E, Fe, S, Fs = cfg["n_experts"], cfg["expert_ffn"], cfg["n_shared"], cfg["shared_ffn"]
            self.Wr = [f16(synth.router(seed, l, E, d)) for l in range(L)]
            self.Eg = [[dequant(*synth.int4_matrix(seed, synth.GATE, l, 1 + e, Fe, d)) for e in range(E)] for l in range(L)]
            self.Eu = [[dequant(*synth.int4_matrix(seed, synth.UP, l, 1 + e, Fe, d)) for e in range(E)] for l in range(L)]
            self.Ed = [[dequant(*synth.int4_matrix(seed, synth.DOWN, l, 1 + e, d, Fe)) for e in range(E)] for l in range(L)]
            sx = [synth.SHARED_EXPERT + s for s in range(S)]
            self.Sg = [[dequant(*synth.int4_matrix(seed, synth.GATE, l, x, Fs, d)) for x in sx] for l in range(L)]
            self.Su = [[dequant(*synth.int4_matrix(seed, synth.UP, l, x, Fs, d)) for x in sx] for l in range(L)]
            self.Sd = [[dequant(*synth.int4_matrix(seed, synth.DOWN, l, x, d, Fs)) for x in sx] for l in range(L)]
        # logical cache: per layer, list over positions of (K [G][D], V [G][D])
        self.K = [[] for _ in range(L)]
        self.V = [[] for _ in range(L)]

    def _rms(self, x, g):
        return x / np.sqrt(np.mean(x * x) + self.cfg.get("rms_eps", 1e-6)) * g

    def _rope(self, v, pos):
        """v [..., D] rotated by pos."""
        D = v.shape[-1]
        half = D // 2
        inv = self.cfg.get("rope_base", 1e6) ** (-2.0 * np.arange(half) / D)
        ang = pos * inv
        c, s = np.cos(ang), np.sin(ang)
        a, b = v[..., :half], v[..., half:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)

    @staticmethod
    def _swiglu(Wg, Wu, Wd, h):
        g = Wg @ h
        return Wd @ (g / (1.0 + np.exp(-g)) * (Wu @ h))

    def step(self, token: int) -> np.ndarray:
        """Append one token at the next position and return its logits."""
        cfg = self.cfg
        H, G, D = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        pos = len(self.K[0])
        x = f16(synth.embed_rows(self.seed, cfg["d_model"], token, 1)[0])
        for l in range(cfg["n_layers"]):
            h = self._rms(x, self.g_attn[l])
            qkv = self.Wqkv[l] @ h
            q = self._rope(qkv[: H * D].reshape(H, D), pos)
            k = self._rope(qkv[H * D:(H + G) * D].reshape(G, D), pos)
            v = qkv[(H + G) * D:].reshape(G, D)
            self.K[l].append(round_kv(k, cfg.get("kv_dtype", "bf16")))
            self.V[l].append(round_kv(v, cfg.get("kv_dtype", "bf16")))
            Kc = np.stack(self.K[l], axis=1)  # [G][n][D]
            Vc = np.stack(self.V[l], axis=1)
            grp = H // G
            o = np.empty((H, D))
            for hq in range(H):
                s = Kc[hq // grp] @ q[hq] / np.sqrt(D)
                p = np.exp(s - s.max())
                p /= p.sum()
                o[hq] = p @ Vc[hq // grp]
            x = x + self.Wo[l] @ o.reshape(-1)
            h2 = self._rms(x, self.g_ffn[l])
            if not self.moe:
                x = x + self._swiglu(self.Wg[l], self.Wu[l], self.Wd[l], h2)
            else:
                r = self.Wr[l] @ h2
                P = np.exp(r - r.max())
                P /= P.sum()
                order = np.argsort(-r, kind="stable")  # descending, ties to the lower index
                sel = order[: cfg["top_k"]]
                z = P[sel].sum()
                y = np.zeros_like(x)
                for e in sel:
                    y += P[e] / z * self._swiglu(self.Eg[l][e], self.Eu[l][e], self.Ed[l][e], h2)
                for s_ in range(cfg["n_shared"]):
                    y += self._swiglu(self.Sg[l][s_], self.Su[l][s_], self.Sd[l][s_], h2)
                x = x + y
        return self.Wlm @ self._rms(x, self.g_final)
