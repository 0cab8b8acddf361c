"""Oracle decoder forward (fp64, explicit mask) -- test infrastructure only.

The pages evaluate LLaMA-2 / CodeLlama decoders ([LD] §5 "Evaluation
Methodology") and state nothing more about the architecture, so the model is
the textbook LLaMA decoder (reading, also in the design doc):

    x      = E[token]
    per layer:
      h    = RMSNorm(x) * g1
      q,k,v= h Wq^T, h Wk^T, h Wv^T ; RoPE on q and k (rotate-half pairing
             (i, i + hd/2), theta = 10000) at each row's position
      a    = softmax(q k^T / sqrt(hd) under the visibility mask) v ;
             query head j reads KV head floor(j * Hkv / H)
      x   += a Wo^T
      h    = RMSNorm(x) * g2
      x   += (SiLU(h Wg^T) * (h Wu^T)) Wd^T
    logits = RMSNorm(x) * gf  W_lm^T

Precision.  Everything is computed in float64.  For bf16 models the bf16
contract rounds (to nearest even) exactly these tensors to bf16: the norm
outputs h, q and k after RoPE, v, the attention output a, and the gated MLP
activation.  The weights are bf16 values.  The residual stream, the
softmax, the accumulations and the logits stay float64 here.  fp32 models
round nothing.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even),
    returned as float64.  bfloat16 keeps 8 significant bits and float32's
    exponent range; the values here are far from overflow and underflow."""
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)              # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  A bf16 value is the upper
    half of the float32 with the same bits."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(F64)


class OracleModel:
    """Decoder with weights given in loader order (see synth.weight_names)."""

    def __init__(self, shape, weights):
        self.s = shape
        self.bf16 = shape.dtype == "bf16"
        self._w = weights
        self._cache: dict[int, np.ndarray] = {}

    # weights are decoded to float64 on demand (the 7B shape does not fit as
    # float64 all at once on small hosts); `keep` keeps decoded copies.
    keep = True

    def w(self, i: int) -> np.ndarray:
        if i in self._cache:
            return self._cache[i]
        a = self._w[i]
        v = decode_bf16(a) if self.bf16 else np.asarray(a, dtype=F64)
        if self.keep:
            self._cache[i] = v
        return v

    def rnd(self, x: np.ndarray) -> np.ndarray:
        return bf16_round(x) if self.bf16 else x

    # -- textbook pieces ---------------------------------------------------
    def rmsnorm(self, x: np.ndarray, g: np.ndarray) -> np.ndarray:
        ms = np.mean(x * x, axis=-1, keepdims=True)
        return x / np.sqrt(ms + self.s.norm_eps) * g

    def rope(self, x: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """x [T, heads, hd]; rotate pair (i, i+hd/2) by pos * theta^(-2i/hd)."""
        hd = x.shape[-1]
        half = hd // 2
        inv = self.s.rope_theta ** (-2.0 * np.arange(half, dtype=F64) / hd)
        ang = pos.astype(F64)[:, None] * inv[None, :]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)

    @staticmethod
    def silu(z: np.ndarray) -> np.ndarray:
        return z / (1.0 + np.exp(-z))

    @staticmethod
    def attention(q, k, v, vis, n_heads, n_kv):
        """q [T, H, hd]; k, v [S, Hkv, hd]; vis [T, S] bool.  Plain masked
        softmax attention with scale 1/sqrt(hd)."""
        hd = q.shape[-1]
        out = np.empty_like(q)
        for h in range(n_heads):
            kh = h * n_kv // n_heads
            s = (q[:, h, :] @ k[:, kh, :].T) / np.sqrt(hd)
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[:, h, :] = p @ v[:, kh, :]
        return out

    # -- forward ---------------------------------------------------------
    def forward(self, tokens, positions, vis, past=None):
        """Run rows `tokens` at `positions`.

        past: None or a list (per layer) of (K, V) float64 arrays
              [S_past, Hkv, hd] already in the stored precision.
        vis:  bool [T, S_past + T]; column j < S_past is past row j, column
              S_past + r is row r of this call.
        Returns (logits [T, V] float64, new_kv: list of (K, V) [T, Hkv, hd]).
        """
        s = self.s
        tokens = np.asarray(tokens, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        T = tokens.shape[0]
        H, Hkv, hd = s.n_heads, s.n_kv_heads, s.head_dim
        x = self.w(0)[tokens].copy()
        new_kv = []
        for li in range(s.n_layers):
            b = 1 + 9 * li
            h = self.rnd(self.rmsnorm(x, self.w(b)))
            q = (h @ self.w(b + 1).T).reshape(T, H, hd)
            k = (h @ self.w(b + 2).T).reshape(T, Hkv, hd)
            v = (h @ self.w(b + 3).T).reshape(T, Hkv, hd)
            q = self.rnd(self.rope(q, positions))
            k = self.rnd(self.rope(k, positions))
            v = self.rnd(v)
            new_kv.append((k, v))
            if past is not None:
                kk = np.concatenate([past[li][0], k], axis=0)
                vv = np.concatenate([past[li][1], v], axis=0)
            else:
                kk, vv = k, v
            a = self.rnd(self.attention(q, kk, vv, vis, H, Hkv)).reshape(T, H * hd)
            x = x + a @ self.w(b + 4).T
            h = self.rnd(self.rmsnorm(x, self.w(b + 5)))
            act = self.rnd(self.silu(h @ self.w(b + 6).T) * (h @ self.w(b + 7).T))
            x = x + act @ self.w(b + 8).T
        nl = 1 + 9 * s.n_layers
        h = self.rnd(self.rmsnorm(x, self.w(nl)))
        logits = h @ self.w(nl + 1).T
        return logits, new_kv


def causal_vis(n_past: int, T: int) -> np.ndarray:
    """Row r (at position n_past + r) sees every past row and rows <= r."""
    vis = np.zeros((T, n_past + T), dtype=bool)
    vis[:, :n_past] = True
    vis[:, n_past:] = np.tril(np.ones((T, T), dtype=bool))
    return vis


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Row-wise argmax; ties go to the lowest token id (reading: the pages
    do not say; np.argmax returns the first maximum)."""
    return np.argmax(logits, axis=-1).astype(np.int64)
