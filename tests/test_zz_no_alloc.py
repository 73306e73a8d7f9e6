"""The allocation-free fp32 GEMM (dit_gemm_f32_noalloc) against dit_gemm,
through the C ABI: bit-identical C on two calls in a row, the second smaller
than the first (the shared scratch keeps the first call's contents), on the
direct and the split-K paths; a shape beyond the built-in scratch is refused
before any launch and leaves C untouched."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    from video_audio_gen_amd import dit as d
    d.load()
    return d


def _case(rng, M, N, K):
    A = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).cuda()
    B = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).cuda()
    bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).cuda()
    return A, B, bias


@pytest.mark.parametrize("shapes", [((172, 2560, 2560), (37, 640, 1000)),   # split-K, then smaller
                                    ((300, 1024, 2048), (86, 97, 64))])      # direct/split, then tiny ragged
def test_noalloc_gemm_equals_dit_gemm_twice(dit, shapes):
    rng = np.random.default_rng(7)
    limit = dit.dit_gemm_f32_noalloc_limit()
    for (M, N, K) in shapes:
        print(f"noalloc gemm M={M} N={N} K={K}", flush=True)
        import ctypes
        need = ctypes.c_size_t()
        assert dit.load().dit_gemm_workspace_bytes(dit.DIT_F32, M, N, K, ctypes.byref(need)) == 0
        assert need.value <= limit
        A, B, bias = _case(rng, M, N, K)
        want = torch.empty(M, N, dtype=torch.float32, device="cuda")
        dit.dit_gemm(A, B, bias, want)
        got = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        dit.dit_gemm_f32_noalloc(A, B, bias, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"M={M} N={N} K={K}"


def test_noalloc_gemm_refuses_beyond_its_scratch(dit):
    # B's slices alone: 5 * 8192 * 4096 bytes = 160 MiB > 64 MiB
    M, N, K = 16, 8192, 4096
    A = torch.zeros(M, K, device="cuda")
    B = torch.zeros(N, K, device="cuda")
    C = torch.full((M, N), 7.0, device="cuda")
    with pytest.raises(dit.DitError) as e:
        dit.dit_gemm_f32_noalloc(A, B, None, C)
    assert e.value.status == "DIT_E_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
