"""Seeded synthetic inputs for the lookahead decoding step.

This module is shared by the HIP path's tests/bench and by the oracle.  It
holds no arithmetic of the method itself: it only draws the model weights,
the prompts and the initial lookahead windows that both sides consume as
inputs.

Model shapes follow the LLaMA family the pages evaluate on (LLaMA-2 /
CodeLlama 7B, 13B, 70B; "Break the Sequential Dependency of LLM Inference
Using LOOKAHEAD DECODING", §5 "Evaluation Methodology").  Trained checkpoints
are not available, so every model is random-init: every matrix is drawn
N(0, 0.02^2) and every norm gain is 1.0.  The initial window is drawn
uniformly over the vocabulary, following the random initialisation of Jacobi
iteration (same page, §2 and §3.4 "Mathematical Reformulation").

Weights are drawn in chunks of 2^22 values; each chunk comes from its own
torch CPU generator seeded from (seed, tensor index, chunk index), so any
tensor can be regenerated on its own and the result does not depend on the
number of worker threads.  bf16 weights are the float32 draws rounded to
nearest even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "ModelShape", "SHAPES", "weight_names", "weight_shapes", "gen_weights",
    "gen_tensor", "prompt_motif", "prompt_zipf_spans", "prompt_code_lines",
    "gen_window", "bf16_bits", "bits_to_f32",
]

_CHUNK = 1 << 22  # elements per independently keyed Philox stream


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    dtype: str  # "f32" or "bf16"
    rope_theta: float = 10000.0
    norm_eps: float = 1e-5
    init_std: float = 0.02


SHAPES = {
    # fp32 tiny decoder (d 64, 4 heads, FFN 256, vocab 256, 2 layers)
    "tiny": ModelShape("tiny", 2, 64, 4, 4, 16, 256, 256, "f32"),
    # fp32 micro decoder with an 8-token vocabulary and wide weights, so its
    # next-token distributions are neither flat nor one-hot: sampling tests
    # enumerate every continuation of a few tokens
    "micro": ModelShape("micro", 1, 64, 4, 4, 16, 128, 8, "f32", init_std=0.45),
    # small bf16 decoder with the 7B head geometry (head_dim 128) used for
    # parity at sizes the oracle runs in seconds; N and vocab are chosen so the
    # GEMMs span several tiles and a ragged tail.
    "small_bf16": ModelShape("small_bf16", 2, 512, 4, 4, 128, 1408, 4000, "bf16"),
    "small_gqa_bf16": ModelShape("small_gqa_bf16", 2, 512, 4, 2, 128, 1024, 2600, "bf16"),
    "llama7b": ModelShape("llama7b", 32, 4096, 32, 32, 128, 11008, 32000, "bf16"),
    "codellama13b": ModelShape("codellama13b", 40, 5120, 40, 40, 128, 13824, 32016, "bf16"),
    "llama70b": ModelShape("llama70b", 80, 8192, 64, 8, 128, 28672, 32000, "bf16"),
}


def weight_names(s: ModelShape) -> list[str]:
    """Tensor names in the order the C-ABI model loader takes them."""
    names = ["emb"]
    for i in range(s.n_layers):
        names += [f"l{i}.attn_norm", f"l{i}.wq", f"l{i}.wk", f"l{i}.wv", f"l{i}.wo",
                  f"l{i}.mlp_norm", f"l{i}.wg", f"l{i}.wu", f"l{i}.wd"]
    names += ["final_norm", "lm_head"]
    return names


def weight_shapes(s: ModelShape) -> list[tuple[int, ...]]:
    """Shapes in loader order; matrices are [out_features, in_features]."""
    d, hd = s.d_model, s.head_dim
    shp = [(s.vocab, d)]
    for _ in range(s.n_layers):
        shp += [(d,), (s.n_heads * hd, d), (s.n_kv_heads * hd, d), (s.n_kv_heads * hd, d),
                (d, s.n_heads * hd), (d,), (s.d_ff, d), (s.d_ff, d), (d, s.d_ff)]
    shp += [(d,), (s.vocab, d)]
    return shp


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Used only to store the drawn Gaussian weights in bf16; the draws are
    finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_chunk(seed: int, tidx: int, cidx: int, n: int, std: float, bf16: bool) -> np.ndarray:
    import torch
    key = ((int(seed) * 1000003 + int(tidx)) * 1000033 + int(cidx)) & ((1 << 63) - 1)
    g = torch.Generator().manual_seed(key)
    t = torch.randn(n, generator=g, dtype=torch.float32)
    t.mul_(std)
    if bf16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def gen_tensor(s: ModelShape, seed: int, tidx: int, threads: int | None = None) -> np.ndarray:
    """Draw loader tensor `tidx` of shape `s`.

    bf16 models: uint16 bit patterns; f32 models: float32.  Norm gains are 1.
    """
    name = weight_names(s)[tidx]
    shape = weight_shapes(s)[tidx]
    n = int(np.prod(shape))
    is_norm = name.endswith("norm")
    if is_norm:
        f = np.ones(n, dtype=np.float32)
        return (bf16_bits(f) if s.dtype == "bf16" else f).reshape(shape)
    nch = (n + _CHUNK - 1) // _CHUNK
    out = np.empty(n, dtype=np.uint16 if s.dtype == "bf16" else np.float32)

    def work(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = _draw_chunk(seed, tidx, c, hi - lo, s.init_std, s.dtype == "bf16")

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    import torch
    prev = torch.get_num_threads()
    torch.set_num_threads(1)  # parallelism comes from the chunk pool
    try:
        if nch == 1 or threads <= 1:
            for c in range(nch):
                work(c)
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(work, range(nch)))
    finally:
        torch.set_num_threads(prev)
    return out.reshape(shape)


def gen_weights(s: ModelShape, seed: int = 0, threads: int | None = None) -> list[np.ndarray]:
    """All tensors of shape `s` in loader order (see gen_tensor)."""
    return [gen_tensor(s, seed, i, threads) for i in range(len(weight_names(s)))]


# ---------------------------------------------------------------------------
# prompts and windows
# ---------------------------------------------------------------------------

def prompt_motif(vocab: int, motif_len: int = 4, repeats: int = 4, seed: int = 1) -> np.ndarray:
    """One seeded motif, uniform over [0, vocab), repeated `repeats` times."""
    g = np.random.Generator(np.random.Philox(key=(0xA1 << 64) | int(seed)))
    motif = g.integers(0, vocab, size=motif_len, dtype=np.int64)
    return np.tile(motif, repeats).astype(np.int32)


def _zipf_ids(g: np.random.Generator, n: int, vocab: int, a: float) -> np.ndarray:
    out = np.empty(0, dtype=np.int64)
    while out.size < n:
        r = g.zipf(a, size=2 * n)
        out = np.concatenate([out, r[r <= vocab]])
    return (out[:n] - 1).astype(np.int64)  # rank r -> id r-1


def prompt_zipf_spans(vocab: int, length: int = 128, n_spans: int = 3, span: int = 16,
                      a: float = 1.1, seed: int = 1) -> np.ndarray:
    """Zipf(a) token ranks mapped to ids, with `n_spans` seeded 16-token spans
    copied to later, non-overlapping offsets.

    The prompt is cut into blocks of `span` tokens; `n_spans` distinct source
    blocks are drawn from the first half and copied into distinct destination
    blocks drawn from the second half.
    """
    g = np.random.Generator(np.random.Philox(key=(0xB2 << 64) | int(seed)))
    toks = _zipf_ids(g, length, vocab, a)
    nblk = length // span
    half = nblk // 2
    n_spans = min(n_spans, half, nblk - half)
    src = g.choice(half, size=n_spans, replace=False)
    dst = half + g.choice(nblk - half, size=n_spans, replace=False)
    for s_, d_ in zip(src, dst):
        toks[d_ * span:(d_ + 1) * span] = toks[s_ * span:(s_ + 1) * span]
    return toks.astype(np.int32)


def prompt_code_lines(vocab: int, length: int = 512, n_lines: int = 20, line_len: int = 24,
                      sub_vocab: int = 2000, p_repeat: float = 0.4, seed: int = 1) -> np.ndarray:
    """Code-like prompt: lines of uniform tokens from a seeded sub-vocabulary;
    each next line repeats a uniformly chosen earlier line with probability
    `p_repeat`, else it is the next new line.  Truncated to `length`."""
    g = np.random.Generator(np.random.Philox(key=(0xC3 << 64) | int(seed)))
    sub = g.choice(vocab, size=sub_vocab, replace=False)
    lines = [sub[g.integers(0, sub_vocab, size=line_len)] for _ in range(n_lines)]
    out: list[np.ndarray] = []
    used = 0
    total = 0
    while total < length:
        if out and (g.random() < p_repeat or used >= n_lines):
            ln = out[int(g.integers(0, len(out)))]
        else:
            ln = lines[used]
            used += 1
        out.append(ln)
        total += len(ln)
    return np.concatenate(out)[:length].astype(np.int32)


def gen_window(N: int, W: int, vocab: int, seed: int = 2) -> np.ndarray:
    """Initial lookahead window, (N-1) levels x W columns, level-major,
    uniform over [0, vocab)."""
    g = np.random.Generator(np.random.Philox(key=(0xD4 << 64) | int(seed)))
    return g.integers(0, vocab, size=max(N - 1, 0) * W, dtype=np.int64).astype(np.int32)
