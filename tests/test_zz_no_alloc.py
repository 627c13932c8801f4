"""The test GEMM entry point that allocates nothing (cac_test_gemm_noalloc) against the
allocating one (cac_test_gemm), through the C ABI: identical outputs on two calls in a row,
the second smaller than the first, with the output buffers filled with NaN beforehand; and a
call whose split-K partials exceed the library's device scratch is refused before any device
work."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_conformer_amd  # noqa: F401  (fails loudly when libcac.so is missing)
    yield


def _operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    dev = "cuda:0"
    A = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(dev).to(torch.bfloat16)
    W = torch.from_numpy((rng.standard_normal((N, K), dtype=np.float32) / np.sqrt(K)).astype(np.float32)).to(dev)
    W = W.to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(N, dtype=np.float32)).to(dev)
    return A, W, b


def test_noalloc_gemm_matches_allocating_gemm_on_two_calls():
    from cache_aware_conformer_amd.binding import CAC_BF16, test_gemm
    # first call: 4 k-ranges over 600 x 1024 (2.4 Mi floats of partials); second: smaller, 2 ranges
    for (M, N, K, path, seed) in [(600, 1024, 2048, 8, 1), (24, 512, 512, 7, 2), (130, 768, 512, 4, 3)]:
        print(f"noalloc gemm M={M} N={N} K={K} path={path}", flush=True)
        A, W, b = _operands(M, N, K, seed)
        c_new = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
        c_ref = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
        test_gemm(CAC_BF16, path, A, W, b, out=c_new, noalloc=True)
        test_gemm(CAC_BF16, path, A, W, b, out=c_ref)
        torch.cuda.synchronize()
        got, ref = c_new.cpu().numpy(), c_ref.cpu().numpy()
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref)
        exact = A.double().cpu().numpy() @ W.double().cpu().numpy().T + b.double().cpu().numpy()
        assert np.abs(got - exact).max() / np.abs(exact).max() < 1e-5


def test_noalloc_gemm_refuses_partials_beyond_its_scratch():
    from cache_aware_conformer_amd.binding import CAC_BF16, CAC_ENOMEM, CacError, test_gemm
    A, W, b = _operands(2048, 1024, 1024, 4)   # 4 ranges x 2048 x 1024 = 8 Mi floats > 4 Mi
    c = torch.full((2048, 1024), 7.0, dtype=torch.float32, device="cuda:0")
    with pytest.raises(CacError) as ei:
        test_gemm(CAC_BF16, 8, A, W, b, out=c, noalloc=True)
    assert ei.value.code == CAC_ENOMEM and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((c == 7.0).all())   # nothing was launched
