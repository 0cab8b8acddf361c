"""Oracle decoder forward (fp64, explicit mask) -- test infrastructure only.

The pages evaluate LLaMA-2 / CodeLlama decoders ([LD] §5 "Evaluation
Methodology") and state nothing more about the architecture, so the model is
the textbook LLaMA decoder (a reading of the pages):

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

    # Weights are decoded to float64 on demand.  keep=True caches the decoded
    # copies; keep=False (large shapes) decodes each matrix again per use, in
    # blocks of output features, so float64 copies of a 7B-70B model never
    # have to exist at once.  Both compute the same products.
    keep = True
    BLOCK = 2048
    on_layer = None  # optional progress callback, called with each finished layer

    def w(self, i: int) -> np.ndarray:
        if i in self._cache:
            return self._cache[i]
        a = self._w[i]
        v = decode_bf16(a) if self.bf16 else np.asarray(a, dtype=F64)
        if self.keep:
            self._cache[i] = v
        return v

    def _decode_rows(self, i: int, lo: int, hi: int) -> np.ndarray:
        a = self._w[i][lo:hi]
        if not self.bf16:
            return np.asarray(a, dtype=F64)
        import torch
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()

    # Accumulation precision of the products: "f64" (default) or "f32".  The
    # second computes each product in float32 from the same (exactly
    # representable) operands, the fp32-accumulation reading of the oracle;
    # the two differ only by rounding, which measures how far apart two
    # exact evaluations of a bf16 model can drift.
    acc = "f64"

    def mm(self, x: np.ndarray, i: int) -> np.ndarray:
        """x @ W_i^T for weight i of shape [out, in]."""
        if self.acc == "f32":
            return self._mm32(x, i)
        if self.keep:
            return x @ self.w(i).T
        n_out = self._w[i].shape[0]
        out = np.empty((x.shape[0], n_out))
        for lo in range(0, n_out, self.BLOCK):
            hi = min(n_out, lo + self.BLOCK)
            out[:, lo:hi] = x @ self._decode_rows(i, lo, hi).T
        return out

    def _mm32(self, x: np.ndarray, i: int) -> np.ndarray:
        import torch
        xf = torch.from_numpy(np.asarray(x, dtype=np.float32))
        n_out = self._w[i].shape[0]
        out = np.empty((x.shape[0], n_out))
        for lo in range(0, n_out, self.BLOCK):
            hi = min(n_out, lo + self.BLOCK)
            wf = torch.from_numpy(self._decode_rows(i, lo, hi).astype(np.float32))
            out[:, lo:hi] = (xf @ wf.T).double().numpy()
        return out

    def emb_rows(self, tokens: np.ndarray) -> np.ndarray:
        if self.keep:
            return self.w(0)[tokens].copy()
        a = self._w[0][tokens]
        return decode_bf16(a) if self.bf16 else np.asarray(a, dtype=F64)

    def vec(self, i: int) -> np.ndarray:
        a = self._w[i]
        return decode_bf16(a) if self.bf16 else np.asarray(a, dtype=F64)

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

    # -- one layer, step by step (forward composes these; a checker can also
    #    feed each step the inputs another implementation produced) ----------
    def attn_norm(self, x, li):
        return self.rnd(self.rmsnorm(x, self.vec(1 + 9 * li)))

    def qkv(self, h, li, positions):
        """q [T, H, hd], k, v [T, Hkv, hd]; q and k after RoPE."""
        s, b, T = self.s, 1 + 9 * li, h.shape[0]
        q = self.mm(h, b + 1).reshape(T, s.n_heads, s.head_dim)
        k = self.mm(h, b + 2).reshape(T, s.n_kv_heads, s.head_dim)
        v = self.mm(h, b + 3).reshape(T, s.n_kv_heads, s.head_dim)
        positions = np.asarray(positions, dtype=np.int64)
        return self.rnd(self.rope(q, positions)), self.rnd(self.rope(k, positions)), self.rnd(v)

    def attend(self, q, kk, vv, vis):
        """Attention output [T, H*hd] of rows q over keys/values kk, vv."""
        T = q.shape[0]
        return self.rnd(self.attention(q, kk, vv, vis, self.s.n_heads, self.s.n_kv_heads)).reshape(T, -1)

    def attn_residual(self, x, a, li):
        return x + self.mm(a, 1 + 9 * li + 4)

    def mlp_norm(self, x, li):
        return self.rnd(self.rmsnorm(x, self.vec(1 + 9 * li + 5)))

    def mlp_act(self, h, li):
        b = 1 + 9 * li
        return self.rnd(self.silu(self.mm(h, b + 6)) * self.mm(h, b + 7))

    def mlp_residual(self, x, act, li):
        return x + self.mm(act, 1 + 9 * li + 8)

    def final_norm(self, x):
        return self.rnd(self.rmsnorm(x, self.vec(1 + 9 * self.s.n_layers)))

    def lm_head(self, h):
        return self.mm(h, 2 + 9 * self.s.n_layers)

    # -- forward ---------------------------------------------------------
    def forward(self, tokens, positions, vis, past=None):
        """Run rows `tokens` at `positions`.

        past: None or a list (per layer) of (K, V) float64 arrays
              [S_past, Hkv, hd] already in the stored precision.
        vis:  bool [T, S_past + T]; column j < S_past is past row j, column
              S_past + r is row r of this call.
        Returns (logits [T, V] float64, new_kv: list of (K, V) [T, Hkv, hd]).
        """
        tokens = np.asarray(tokens, dtype=np.int64)
        x = self.emb_rows(tokens)
        new_kv = []
        for li in range(self.s.n_layers):
            h = self.attn_norm(x, li)
            q, k, v = self.qkv(h, li, positions)
            new_kv.append((k, v))
            if past is not None:
                kk = np.concatenate([past[li][0], k], axis=0)
                vv = np.concatenate([past[li][1], v], axis=0)
            else:
                kk, vv = k, v
            x = self.attn_residual(x, self.attend(q, kk, vv, vis), li)
            x = self.mlp_residual(x, self.mlp_act(self.mlp_norm(x, li), li), li)
            if self.on_layer is not None:
                self.on_layer(li)
        return self.lm_head(self.final_norm(x)), new_kv


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
