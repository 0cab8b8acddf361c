"""Pins of the oracle's decoder forward against things other than itself:
a library LLaMA (HF transformers, float64), torch's bfloat16 conversion and
attention, and textbook special cases."""
import numpy as np
import pytest
import torch

import synth
from oracle.model import OracleModel, bf16_round, decode_bf16, causal_vis, argmax_lowest
from oracle.attention import lookahead_attention
from oracle.lookahead import block_mask


def _tiny(dtype="f32", **kw):
    base = dict(name="t", n_layers=2, d_model=64, n_heads=4, n_kv_heads=4, head_dim=16,
                d_ff=256, vocab=256, dtype=dtype)
    base.update(kw)
    return synth.ModelShape(**base)


# -- bf16 rounding -----------------------------------------------------------

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        [0.0, 1.0, -1.0, 1.00390625, 1.005859375, 3.0e-5]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.0
    assert bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert bf16_round(np.array([255.5]))[0] == 256.0


def test_decode_bf16_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_bf16(bits)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])


# -- forward against HF LLaMA --------------------------------------------------

def _hf_model(s, weights):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=s.vocab, hidden_size=s.d_model, intermediate_size=s.d_ff,
                      num_hidden_layers=s.n_layers, num_attention_heads=s.n_heads,
                      num_key_value_heads=s.n_kv_heads, head_dim=s.head_dim,
                      rms_norm_eps=s.norm_eps, rope_theta=s.rope_theta,
                      tie_word_embeddings=False, max_position_embeddings=4096,
                      attention_bias=False, mlp_bias=False)
    m = LlamaForCausalLM(cfg).double().eval()
    names = synth.weight_names(s)
    sd = {}
    hf_layer = {"attn_norm": "input_layernorm", "wq": "self_attn.q_proj", "wk": "self_attn.k_proj",
                "wv": "self_attn.v_proj", "wo": "self_attn.o_proj", "mlp_norm": "post_attention_layernorm",
                "wg": "mlp.gate_proj", "wu": "mlp.up_proj", "wd": "mlp.down_proj"}
    for n, w in zip(names, weights):
        t = torch.from_numpy(np.asarray(w, dtype=np.float64))
        if n == "emb":
            sd["model.embed_tokens.weight"] = t
        elif n == "final_norm":
            sd["model.norm.weight"] = t
        elif n == "lm_head":
            sd["lm_head.weight"] = t
        else:
            li, part = n[1:].split(".", 1)
            sd[f"model.layers.{li}.{hf_layer[part]}.weight"] = t
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    return m


@pytest.mark.parametrize("shape", [_tiny(), _tiny(n_kv_heads=2, n_layers=3, d_ff=96, vocab=97)])
def test_forward_matches_hf_llama(shape):
    w = synth.gen_weights(shape, seed=3)
    om = OracleModel(shape, w)
    toks = np.random.default_rng(1).integers(0, shape.vocab, 23)
    got, _ = om.forward(toks, np.arange(23), causal_vis(0, 23))
    hf = _hf_model(shape, w)
    with torch.no_grad():
        ref = hf(torch.from_numpy(toks)[None]).logits[0].numpy()
    # HF computes the RoPE angles and cos/sin in float32 even in a float64
    # model, which bounds agreement at ~1e-7; a wrong pairing, sign, scale
    # or missing term shows up at 1e-3 or more.
    np.testing.assert_allclose(got, ref, atol=1e-6, rtol=0)
    assert np.array_equal(argmax_lowest(got), argmax_lowest(ref))


def test_forward_with_cache_equals_full_forward():
    s = _tiny()
    om = OracleModel(s, synth.gen_weights(s, seed=4))
    toks = np.random.default_rng(2).integers(0, s.vocab, 12)
    full, _ = om.forward(toks, np.arange(12), causal_vis(0, 12))
    _, kv = om.forward(toks[:7], np.arange(7), causal_vis(0, 7))
    tail, _ = om.forward(toks[7:], np.arange(7, 12), causal_vis(7, 5), past=kv)
    np.testing.assert_allclose(tail, full[7:], atol=1e-12, rtol=0)


# -- textbook special cases -----------------------------------------------------

def test_zero_weights_give_uniform_logits():
    s = _tiny()
    w = [np.zeros_like(a) if not n.endswith("norm") else a
         for n, a in zip(synth.weight_names(s), synth.gen_weights(s, 0))]
    logits, _ = OracleModel(s, w).forward([3, 4, 5], [0, 1, 2], causal_vis(0, 3))
    assert np.all(logits == 0.0)
    assert np.all(argmax_lowest(logits) == 0)


def test_rope_identity_at_zero_and_relative():
    s = _tiny()
    om = OracleModel(s, synth.gen_weights(s, 0))
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 3, 16))
    np.testing.assert_allclose(om.rope(x, np.array([0])), x, atol=0)
    q, k = rng.standard_normal((2, 1, 1, 16))
    def dot(m, n):
        return float(np.sum(om.rope(q, np.array([m])) * om.rope(k, np.array([n]))))
    # the score depends only on the offset m - n
    assert abs(dot(7, 3) - dot(107, 103)) < 1e-10
    assert abs(dot(7, 3) - dot(8, 3)) > 1e-6
    # norm preserving
    np.testing.assert_allclose(np.linalg.norm(om.rope(x, np.array([13]))), np.linalg.norm(x))


def test_rope_pairing_rotate_half():
    """hd = 4: pair (0, 2) rotates by pos * theta^0, pair (1, 3) by
    pos * theta^(-1/2)."""
    s = _tiny(head_dim=4, d_model=16)
    om = OracleModel(s, [])
    x = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    y = om.rope(x, np.array([1]))[0, 0]
    np.testing.assert_allclose(y, [np.cos(1.0), 0.0, np.sin(1.0), 0.0], atol=1e-15)
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    y = om.rope(x, np.array([2]))[0, 0]
    a = 2 * 10000.0 ** -0.5
    np.testing.assert_allclose(y, [0.0, np.cos(a), 0.0, np.sin(a)], atol=1e-15)


def test_single_key_attention_returns_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 1, 8))
    v = rng.standard_normal((1, 1, 8))
    out = OracleModel.attention(q, k, v, np.ones((1, 1), bool), 2, 1)
    np.testing.assert_allclose(out[0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(out[0, 1], v[0, 0], atol=1e-15)


def test_rmsnorm_constant_vector():
    s = _tiny()
    om = OracleModel(s, [])
    g = np.linspace(0.5, 2.0, 64)
    y = om.rmsnorm(np.full((1, 64), -3.0), g)
    np.testing.assert_allclose(y[0], -g * 3.0 / np.sqrt(9.0 + 1e-5), rtol=1e-15)


def test_masked_attention_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    N, W, G, P, H, Hkv, hd = 4, 3, 2, 9, 4, 2, 16
    M = 1 + (W + G) * (N - 1)
    q = rng.standard_normal((M, H, hd))
    kp, vp = rng.standard_normal((2, P, Hkv, hd))
    kb, vb = rng.standard_normal((2, M, Hkv, hd))
    got = lookahead_attention(q, kp, vp, kb, vb, N, W, G)
    vis = np.concatenate([np.ones((M, P), bool), block_mask(N, W, G)], axis=1)
    K = torch.from_numpy(np.concatenate([kp, kb])).repeat_interleave(H // Hkv, dim=1)
    V = torch.from_numpy(np.concatenate([vp, vb])).repeat_interleave(H // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1), K.transpose(0, 1), V.transpose(0, 1),
        attn_mask=torch.from_numpy(vis)).transpose(0, 1).numpy()
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


def test_bf16_mode_rounds_stored_tensors():
    """In bf16 mode the KV rows the forward returns are bf16 values, and the
    logits stay close to the unrounded (fp32-mode) forward of the same
    weights."""
    s = _tiny(dtype="bf16")
    w = synth.gen_weights(s, 8)
    om = OracleModel(s, w)
    toks = np.arange(10) * 7 % s.vocab
    lg, kv = om.forward(toks, np.arange(10), causal_vis(0, 10))
    for k, v in kv:
        assert np.array_equal(bf16_round(k), k) and np.array_equal(bf16_round(v), v)
    s32 = _tiny(dtype="f32")
    om32 = OracleModel(s32, [decode_bf16(a).astype(np.float32) for a in w])
    lg32, kv32 = om32.forward(toks, np.arange(10), causal_vis(0, 10))
    assert not np.array_equal(kv32[0][0], kv[0][0])
    assert np.max(np.abs(lg - lg32)) < 2e-2


@pytest.mark.parametrize("name", ["tiny", "small_bf16"])
def test_f32_accumulation_mode_and_blocked_products(name):
    """The float32-accumulation mode and the blocked (keep=False) products
    compute the same function as the default (blocking changes only the
    float64 summation order): the fp32 model agrees to
    float32 accuracy, and for a bf16 model every stored tensor still obeys
    the bf16 contract (the logits move only by rounding-boundary flips)."""
    s = synth.SHAPES[name]
    w = synth.gen_weights(s, 0)
    toks = synth.prompt_motif(s.vocab, 4, 4, seed=3)
    T = len(toks)
    ref, _ = OracleModel(s, w).forward(toks, np.arange(T), causal_vis(0, T))
    m = OracleModel(s, w)
    m.keep = False
    m.BLOCK = 96          # several blocks and a ragged last one
    blk, _ = m.forward(toks, np.arange(T), causal_vis(0, T))
    np.testing.assert_allclose(blk, ref, rtol=0, atol=1e-12)   # BLAS order only
    m.acc = "f32"
    f32, _ = m.forward(toks, np.arange(T), causal_vis(0, T))
    scale = np.abs(ref).max()
    tol = 1e-5 if s.dtype == "f32" else 2e-2
    assert 0 < np.abs(f32 - ref).max() <= tol * max(scale, 1.0)
