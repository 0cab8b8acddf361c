"""The allocation-free GEMM entry point (la_kernel_gemm_noalloc) against the
workspace entry point (la_kernel_gemm) through the C-ABI: the same product,
split and summation order, so the outputs are bit-identical.  Two calls in a
row, the second with a smaller input (the static scratch keeps the first
call's partial sums), then a call the scratch cannot hold, which is refused
and leaves later calls unaffected."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from exact_decoding_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(M, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(DEV)
    wp = torch.empty(B.la_packed_bytes(N, K), dtype=torch.uint8, device=DEV)
    B.la_pack_weight(w, N, K, wp, None)
    return x, w, wp


def _with_workspace(x, wp, M, K, N):
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    nb = B.la_kernel_gemm_ws_bytes(M, K, N)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=DEV)
    B.la_kernel_gemm(x, M, K, wp, N, y, B.LA_BF16, ws, None)
    torch.cuda.synchronize()
    return y


def _no_alloc(x, wp, M, K, N):
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    B.la_kernel_gemm_noalloc(x, M, K, wp, N, y, B.LA_BF16, None)
    torch.cuda.synchronize()
    return y


def test_gemm_noalloc_equals_workspace_entry_point():
    # 7B O projection at the lookahead step's 121 rows (8 pieces per column
    # block, 15.9 MB of partial sums), then a smaller product
    shapes = [(121, 4096, 4096), (17, 1024, 768)]
    for i, (M, K, N) in enumerate(shapes):
        print(f"no-alloc GEMM M={M} K={K} N={N}", flush=True)
        assert 0 < B.la_kernel_gemm_ws_bytes(M, K, N) <= B.LA_NOALLOC_SCRATCH_BYTES
        x, w, wp = _case(M, K, N, seed=11 + i)
        ref = _with_workspace(x, wp, M, K, N)
        got = _no_alloc(x, wp, M, K, N)
        assert torch.equal(got, ref), (M, K, N)
        exact = (x.double() @ w.double().T).cpu().numpy()
        assert np.abs(got.double().cpu().numpy() - exact).max() < 1e-3
    # beyond the scratch: refused, nothing launched
    M, K, N = 2048, 4096, 4096
    assert B.la_kernel_gemm_ws_bytes(M, K, N) > B.LA_NOALLOC_SCRATCH_BYTES
    x, w, wp = _case(64, K, N, seed=5)
    y = torch.zeros((M, N), dtype=torch.float32, device=DEV)
    with pytest.raises(B.LaError) as ei:
        B.la_kernel_gemm_noalloc(x, M, K, wp, N, y, B.LA_BF16, None)
    assert ei.value.code == B.LA_ENOMEM
    # and a later call still matches
    ref = _with_workspace(x, wp, 64, K, N)
    assert torch.equal(_no_alloc(x, wp, 64, K, N), ref)
