"""GPU parity of the step's kernels through the C-ABI hooks.

GEMM: against its definition in float64 (a library matmul of the same bf16
values), and bit-identical per row whatever the row count and placement.
Attention: against the oracle's masked attention (materialised mask), and
bit-identical between a verification row and the same chain run as one
autoregressive query over the cache.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from exact_decoding_amd import binding as B
from oracle.attention import lookahead_attention
from oracle.lookahead import n_rows, row_kind

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(a, seed_scale=1.0):
    return torch.from_numpy(np.asarray(a, np.float32) * seed_scale).to(torch.bfloat16).to(DEV)


def _pack(w):
    N, K = w.shape
    dst = torch.empty(B.la_packed_bytes(N, K), dtype=torch.uint8, device=DEV)
    B.la_pack_weight(w, N, K, dst, None)
    torch.cuda.synchronize()
    return dst


def _gemm(x, w, dtype=B.LA_BF16, wp=None):
    M, K = x.shape
    N = w.shape[0]
    if dtype == B.LA_BF16 and wp is None:
        wp = _pack(w)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    nb = B.la_kernel_gemm_ws_bytes(M, K, N)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=DEV)
    B.la_kernel_gemm(x, M, K, wp if dtype == B.LA_BF16 else w, N, y, dtype, ws, None)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("N,K", [(37, 128), (300, 192)])
def test_pack_layout(N, K):
    """The packed layout places W[16s + lane%16][64c + 32j + 8(lane/16) + e],
    s = 8b + t, at element ((b*(K/64)*8 + c*ns(b) + t)*2 + j)*512 + lane*8 + e
    with ns(b) = min(8, ceil(N/16) - 8b) stripes in column block b; rows past
    N are 0.  N = 300: two full column blocks and a last one of 3 stripes."""
    w = torch.arange(N * K, dtype=torch.float32).reshape(N, K).to(torch.bfloat16).to(DEV)
    got = _pack(w).view(torch.bfloat16).float().cpu().numpy()
    wf = w.float().cpu().numpy()
    nch = K // 64
    S = (N + 15) // 16
    ref = np.zeros(S * 16 * K, dtype=np.float32)
    for s_ in range(S):
        b, t = divmod(s_, 8)
        ns = min(8, S - 8 * b)
        for c in range(nch):
            for j in range(2):
                for lane in range(64):
                    row = 16 * s_ + lane % 16
                    k = 64 * c + 32 * j + 8 * (lane // 16)
                    base = ((b * nch * 8 + c * ns + t) * 2 + j) * 512 + lane * 8
                    if row < N:
                        ref[base:base + 8] = wf[row, k:k + 8]
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("M,K,N", [(1, 256, 384), (17, 512, 640), (121, 4096, 4096),
                                   (121, 1024, 1000), (300, 512, 256), (121, 11008, 4096),
                                   (121, 1344, 1000), (90, 1024, 1000), (100, 1344, 1000),
                                   (121, 1024, 998), (90, 1344, 998), (121, 4096, 32000)])
def test_gemm_bf16_matches_definition(M, K, N):
    print(f"gemm M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M * 7 + K + N)
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    y = _gemm(x, w).cpu().numpy().astype(np.float64)
    ref = x.float().cpu().numpy().astype(np.float64) @ w.float().cpu().numpy().astype(np.float64).T
    err = np.abs(y - ref).max()
    scale = np.abs(ref).max()
    # fp32 accumulation of K products: error ~ sqrt(K) * 2^-24 * |terms|
    assert err <= 1e-5 * scale + 1e-6, (err, scale)


def test_gemm_f32_matches_definition():
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((9, 64)).astype(np.float32)).to(DEV)
    w = torch.from_numpy(rng.standard_normal((200, 64)).astype(np.float32)).to(DEV)
    y = _gemm(x, w, B.LA_F32).cpu().numpy()
    ref = x.cpu().numpy().astype(np.float64) @ w.cpu().numpy().astype(np.float64).T
    assert np.abs(y - ref).max() < 1e-4


@pytest.mark.parametrize("nbytes", [16, 1024 * 1024, 1024 * 1024 + 48, 5 * 1024 * 1024 + 16 * 333])
def test_probe_read_checksums(nbytes):
    """la_probe_read reads every byte once: workgroup b's word is the XOR of the
    32-bit words of its four waves' slices (whole 1 KB wave-loads, the tail
    short or empty)."""
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).copy()).to(DEV)
    out = torch.zeros(B.LA_PROBE_BLOCKS, dtype=torch.int32, device=DEV)
    B.la_probe_read(buf, nbytes, out, None)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    n16 = nbytes // 16
    waves = B.LA_PROBE_BLOCKS * 4
    per = ((n16 + waves - 1) // waves + 63) // 64 * 64
    words = host.reshape(-1, 4)
    for b in range(B.LA_PROBE_BLOCKS):
        lo, hi = min(4 * b * per, n16), min((4 * b + 4) * per, n16)
        want = np.bitwise_xor.reduce(words[lo:hi].ravel()) if hi > lo else np.uint32(0)
        assert got[b] == want, (b, lo, hi)


@pytest.mark.parametrize("K,N", [(4096, 4096), (11008, 4096), (4096, 12288)])
def test_gemm_rows_bit_identical_across_batch(K, N):
    """A row's output bits do not depend on how many rows share the call or
    where the row sits (what makes lookahead rows reproduce the
    autoregressive step).  At 121 rows the first two shapes run the
    loader / consumer kernel (the second with runs that cross a column
    block), the third the four-wave kernel; one row runs the producer-wave
    kernel and 17 rows the four-wave kernel with two row tiles."""
    print(f"gemm bit identity K={K} N={N}", flush=True)
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal((121, K)))
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    wp = _pack(w)
    full = _gemm(x, w, wp=wp)
    for r in [0, 1, 15, 16, 63, 120]:
        one = _gemm(x[r:r + 1].contiguous(), w, wp=wp)
        assert torch.equal(one[0], full[r]), r
    part = _gemm(x[5:22].contiguous(), w, wp=wp)
    assert torch.equal(part, full[5:22])


def _rand_attn(P, H, Hkv, hd, N, W, G, dtype, seed, ld_ctx=None):
    rng = np.random.default_rng(seed)
    M = n_rows(N, W, G)
    ld_ctx = ld_ctx or max(P, 1)
    q = rng.standard_normal((M, H, hd)).astype(np.float32)
    kc = rng.standard_normal((Hkv, ld_ctx, hd)).astype(np.float32)
    vc = rng.standard_normal((Hkv, ld_ctx, hd)).astype(np.float32)
    kb = rng.standard_normal((M, Hkv, hd)).astype(np.float32)
    vb = rng.standard_normal((M, Hkv, hd)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == B.LA_BF16 else torch.float32
    dev = [torch.from_numpy(a).to(tdt).to(DEV) for a in (q, kc, vc, kb, vb)]
    host = [t.float().cpu().numpy().astype(np.float64) for t in dev]
    return M, ld_ctx, dev, host, tdt


def _run_attn(dev, P, ld_ctx, H, Hkv, hd, N, W, G, dtype, tdt, M):
    q, kc, vc, kb, vb = dev
    out = torch.empty((M, H * hd), dtype=tdt, device=DEV)
    nb = B.la_kernel_attention_ws_bytes(ld_ctx, H, hd, N, W, G, dtype)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=DEV)
    B.la_kernel_attention(q, kc, vc, P, ld_ctx, kb, vb, out, H, Hkv, hd, N, W, G, dtype, ws, None)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("P,H,Hkv,hd,N,W,G,dtype", [
    (37, 4, 2, 128, 3, 4, 4, B.LA_BF16),
    (300, 8, 2, 128, 4, 5, 3, B.LA_BF16),
    (1500, 8, 8, 128, 3, 2, 2, B.LA_BF16),
    (0, 4, 4, 128, 4, 3, 2, B.LA_BF16),
    (200, 4, 4, 16, 3, 4, 4, B.LA_F32),
    (512, 32, 32, 128, 5, 15, 15, B.LA_BF16),
    (513, 32, 32, 128, 7, 7, 7, B.LA_BF16),
    (2048, 32, 32, 128, 5, 15, 15, B.LA_BF16),
    (1500, 8, 2, 128, 3, 4, 4, B.LA_BF16),
    (1100, 16, 2, 128, 5, 7, 7, B.LA_BF16),
])
def test_attention_matches_oracle(P, H, Hkv, hd, N, W, G, dtype):
    print(f"attention P={P} H={H} Hkv={Hkv} hd={hd} N={N} W={W} G={G}", flush=True)
    M, ld, dev, host, tdt = _rand_attn(P, H, Hkv, hd, N, W, G, dtype, seed=P + N)
    out = _run_attn(dev, P, ld, H, Hkv, hd, N, W, G, dtype, tdt, M)
    q, kc, vc, kb, vb = host
    ref = lookahead_attention(q, kc[:, :P].transpose(1, 0, 2), vc[:, :P].transpose(1, 0, 2), kb, vb,
                              N, W, G).reshape(M, H * hd)
    got = out.float().cpu().numpy()
    tol = 1e-2 if dtype == B.LA_BF16 else 1e-5
    assert np.abs(got - ref).max() < tol


@pytest.mark.parametrize("P,W,G,H,Hkv", [
    (5, 3, 3, 4, 4), (63, 3, 3, 4, 4), (64, 3, 3, 4, 4), (130, 3, 3, 4, 4), (300, 3, 3, 4, 4),
    (525, 3, 3, 4, 4), (1100, 3, 3, 4, 4), (130, 15, 15, 4, 4), (300, 15, 15, 4, 4),
    (525, 15, 15, 4, 4), (1100, 15, 15, 4, 4), (300, 20, 20, 4, 4), (1100, 20, 20, 4, 4),
    # grouped-query heads
    (300, 3, 3, 8, 2), (1100, 3, 3, 8, 2), (1100, 7, 7, 16, 2), (1100, 15, 15, 8, 2)])
def test_attention_verification_row_equals_ar_query(P, W, G, H, Hkv):
    """Verification row (g, i) == one query at P+i over a cache holding the
    prefix and the row's chain (what an autoregressive step computes).
    Below 1024 committed positions each wave of the MFMA prefix part holds
    one 16-row group of a 64-row block, as the single query does; from 1024
    on a workgroup takes 128 rows and every wave runs two groups together on
    each tile (W = G = 15: 121 rows; W = G = 20: 161 rows, a 128-row block
    and a 33-row one), so the rows go through the two-group path and the
    query through the one-group path; also with grouped-query heads."""
    hd, N = 128, 5
    M, ld, dev, host, tdt = _rand_attn(P, H, Hkv, hd, N, W, G, B.LA_BF16, seed=P, ld_ctx=P + 16)
    out = _run_attn(dev, P, ld, H, Hkv, hd, N, W, G, B.LA_BF16, tdt, M)
    q, kc, vc, kb, vb = dev
    for r in range(M):
        kd = row_kind(r, N, W, G)
        if kd[0] != "ver":
            continue
        _, g, i = kd
        chain = [0] + [1 + W * (N - 1) + g * (N - 1) + j - 1 for j in range(1, i + 1)]
        kc2, vc2 = kc.clone(), vc.clone()
        for j, br in enumerate(chain[:-1]):
            kc2[:, P + j] = kb[br]
            vc2[:, P + j] = vb[br]
        last = chain[-1]
        q1 = q[r:r + 1].contiguous()
        out1 = torch.empty((1, H * hd), dtype=tdt, device=DEV)
        # the autoregressive query uses the same tail depth (N - 1) as the
        # lookahead session it is compared with
        nb = B.la_kernel_attention_ws_bytes(ld, H, hd, N, 0, 0, B.LA_BF16)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=DEV)
        B.la_kernel_attention(q1, kc2, vc2, P + i, ld, kb[last:last + 1].contiguous(),
                              vb[last:last + 1].contiguous(), out1, H, Hkv, hd, N, 0, 0,
                              B.LA_BF16, ws, None)
        torch.cuda.synchronize()
        assert torch.equal(out1[0], out[r]), (r, g, i)


