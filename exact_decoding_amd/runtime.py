"""Convenience layer over the C-ABI binding: torch owns the device memory
(weights, workspace) and the stream; every computation runs in libla.so."""
from __future__ import annotations

import numpy as np

from . import binding as B


def _torch():
    import torch
    return torch


PACKED = ("wq", "wk", "wv", "wo", "wg", "wu", "wd", "lm_head")


def pack(t, stream=None):
    """bf16 [N][K] device tensor -> packed-layout device tensor (see la.h)."""
    torch = _torch()
    N, K = t.shape
    dst = torch.empty(B.la_packed_bytes(N, K), dtype=torch.uint8, device=t.device)
    B.la_pack_weight(t, N, K, dst, stream)
    return dst


def is_packed_name(name: str) -> bool:
    return name.split(".")[-1] in PACKED


def upload(arr: np.ndarray, device: str = "cuda"):
    """numpy weight (float32, or uint16 bf16 bit patterns) -> torch device tensor."""
    torch = _torch()
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device, non_blocking=False)


class Model:
    """A decoder registered with la_model_load.  `weights` are device tensors
    (or numpy arrays, uploaded here) in loader order."""

    def __init__(self, shape, weights, stream=None, device: str = "cuda"):
        torch = _torch()
        self.shape = shape
        self.device = device
        self.stream = stream if stream is not None else torch.cuda.Stream(device=device)
        self.dtype = B.LA_BF16 if shape.dtype == "bf16" else B.LA_F32
        import synth
        names = synth.weight_names(shape)
        self.tensors = []
        for name, w in zip(names, weights):
            t = w if isinstance(w, torch.Tensor) else upload(w, device)
            if self.dtype == B.LA_BF16 and is_packed_name(name) and t.dtype == torch.bfloat16:
                torch.cuda.synchronize(device)
                t = pack(t)
            self.tensors.append(t)
        desc = B.ModelDesc(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads,
                           shape.head_dim, shape.d_ff, shape.vocab, shape.rope_theta,
                           shape.norm_eps, self.dtype)
        torch.cuda.synchronize(device)
        self.handle = B.la_model_load(desc, self.tensors, self.stream)

    def session(self, prompt, N: int, W: int, G: int, max_new: int, window=None,
                prompt_ref: bool = False, ar: bool = False, graph: bool = True,
                max_ctx: int | None = None, pool_cap: int = 0, eos_id: int = -1,
                temperature: float = 0.0, seed: int = 0, top_k: int = 0,
                top_p: float = 0.0, pool_lru: bool = False,
                pool_context: bool = False, adaptive_g: bool = False,
                debug_logits: bool = False) -> "Session":
        """temperature 0: greedy; > 0: sampling verification with draws keyed
        by `seed`, optionally cut to the top_k tokens and then to a top_p share
        (0 = no cut; see la.h).  pool_lru: evict pool entries by recency
        instead of FIFO (LA_POOL_LRU); pool_context: select candidates by
        their context token first (LA_POOL_CONTEXT); adaptive_g: candidate
        rows only as far as the step's candidates need (LA_ADAPTIVE_G);
        debug_logits: keep every step's logits for Session.logits
        (LA_DEBUG_LOGITS)."""
        flags = (B.LA_PROMPT_REF if prompt_ref else 0) | (B.LA_AR if ar else 0)
        flags |= 0 if graph else B.LA_NO_GRAPH
        flags |= B.LA_POOL_LRU if pool_lru else 0
        flags |= B.LA_POOL_CONTEXT if pool_context else 0
        flags |= B.LA_ADAPTIVE_G if adaptive_g else 0
        flags |= B.LA_DEBUG_LOGITS if debug_logits else 0
        if max_ctx is None:
            max_ctx = len(prompt) + max_new + N + W + 2
        p = B.DecodeParams(N, W, G, pool_cap, max_ctx, max_new, eos_id, flags,
                           float(temperature), int(top_k), int(seed), float(top_p), 0)
        return Session(self, p, prompt, window)

    def close(self):
        if self.handle:
            B.la_model_free(self.handle)
            self.handle = None


class Session:
    def __init__(self, model: Model, params: B.DecodeParams, prompt, window):
        torch = _torch()
        self.model = model
        self.params = params
        nbytes = B.la_session_bytes(model.handle, params)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=model.device)
        torch.cuda.synchronize(model.device)
        self.handle = B.la_prefill(model.handle, params, prompt, window, self.workspace,
                                   model.stream)
        self.rows = B.la_session_rows(self.handle)
        self.done = False
        self.tokens: list[int] = []
        self.per_step: list[int] = []

    def step(self) -> list[int]:
        rc, toks = B.la_step(self.handle, max(self.params.N, 1))
        self.tokens.extend(toks)
        if toks:
            self.per_step.append(len(toks))
        self.done = rc == B.LA_DONE
        return toks

    def step_profile(self) -> tuple[list[int], dict]:
        rc, toks, prof = B.la_step_profile(self.handle, max(self.params.N, 1))
        self.tokens.extend(toks)
        if toks:
            self.per_step.append(len(toks))
        self.done = rc == B.LA_DONE
        return toks, prof

    def step_trace(self) -> tuple[list[int], dict]:
        """One step with every forward intermediate copied out (la_step_trace).
        Returns the step's tokens and a dict of host arrays: 16-bit model
        tensors as uint16 bit patterns, float32 tensors as float32."""
        torch = _torch()
        nbytes = B.la_step_trace_bytes(self.handle)
        buf = torch.empty(nbytes, dtype=torch.uint8, device=self.model.device)
        rc, toks = B.la_step_trace(self.handle, max(self.params.N, 1), buf, nbytes)
        self.tokens.extend(toks)
        if toks:
            self.per_step.append(len(toks))
        self.done = rc == B.LA_DONE
        raw = buf.cpu().numpy()
        del buf
        hdr = raw[:64].view(np.int32)
        P, M, ctx, L, d, H, Hkv, hd, F, V, dt = (int(v) for v in hdr[:11])
        edt = np.uint16 if dt == B.LA_BF16 else np.float32
        off = 64

        def take(dtype, shape):
            nonlocal off
            n = int(np.prod(shape)) * np.dtype(dtype).itemsize
            a = raw[off:off + n].view(dtype).reshape(shape)
            off += n
            return a

        t = {"P": P, "M": M, "ids": take(np.int32, (M,)), "pos": take(np.int32, (M,))}
        t["kc"] = take(edt, (L, Hkv, ctx, hd))
        t["vc"] = take(edt, (L, Hkv, ctx, hd))
        t["layers"] = []
        for _ in range(L):
            t["layers"].append({
                "x_in": take(np.float32, (M, d)), "h1": take(edt, (M, d)),
                "q": take(edt, (M, H * hd)), "attn": take(edt, (M, H * hd)),
                "x_mid": take(np.float32, (M, d)), "h2": take(edt, (M, d)),
                "act": take(edt, (M, F))})
        t["x_final"] = take(np.float32, (M, d))
        t["h_final"] = take(edt, (M, d))
        t["kb"] = take(edt, (L, M, Hkv, hd))
        t["vb"] = take(edt, (L, M, Hkv, hd))
        t["logits"] = take(np.float32, (M, V))
        assert off == nbytes, (off, nbytes)
        return toks, t

    def decode(self) -> list[int]:
        while not self.done:
            self.step()
        return self.tokens

    def stats(self) -> dict:
        return B.la_pool_stats(self.handle)

    def logits(self, rows: int | None = None) -> np.ndarray:
        return B.la_debug_logits(self.handle, rows or self.rows, self.model.shape.vocab)

    def close(self):
        if self.handle:
            B.la_session_free(self.handle)
            self.handle = None
