"""Per-kernel parity through the C ABI op-level calls, against the oracle's steps.

Sizes span several tiles with ragged tails; the last cases of each kernel use
the shapes of the full workloads and check sampled outputs.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_bf16_rounded, assert_f32_close, assert_rms_rel, from_dev, rms,
                      to_bf16_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    from video_audio_gen_amd import dit as d
    d.load()
    return d


def _bf16_vals(rng, shape, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).float().numpy()


# ----------------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (300, 320, 128), (513, 768, 192), (26624 // 8, 18432 // 8, 6144),
                                   (65, 97, 64)])
def test_gemm_bf16(dit, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = _bf16_vals(rng, (M, K))
    B = _bf16_vals(rng, (N, K), 0.02)
    bias = rng.standard_normal(N).astype(np.float32)
    ref = O.linear(A, B, bias)
    Ad, Bd = to_bf16_dev(A), to_bf16_dev(B)
    C32 = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dit.dit_gemm(Ad, Bd, torch.from_numpy(bias).cuda(), C32)
    g = from_dev(C32)
    # products of bf16 values are exact in fp32; only the fp32 accumulation order differs
    assert np.abs(g - ref).max() <= 3e-5 * rms(ref) + 1e-6
    C16 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dit.dit_gemm(Ad, Bd, torch.from_numpy(bias).cuda(), C16)
    assert_bf16_rounded(from_dev(C16), ref, "gemm bf16 -> bf16", slack=1e-5)


# (172, 20480, 2560): the music model's MLP-in projection; (60, 6144, 16384):
# a long K with several splits.  Tiles are 176 rows, the last 16 of them a
# block that runs two slices per MFMA: M = 160, 175, 176, 177, 352, 353, 528
# put the matrix end before, inside, at and past that block and tile edges.
@pytest.mark.parametrize("M,N,K", [(1, 4, 4), (100, 70, 36), (172, 2560, 2560), (172, 2560, 10240), (160, 1024, 128),
                                   (400, 300, 96), (70, 130, 20000), (172, 20480, 2560), (60, 6144, 16384),
                                   (37, 33, 64), (173, 97, 2560), (175, 64, 96), (176, 130, 64), (177, 66, 128),
                                   (352, 64, 64), (353, 70, 160), (528, 128, 96)])
def test_gemm_f32_int8_slices(dit, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    A[:, :5] *= 40.0  # outlier channels widen each row's range
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    ref = O.linear(A, B, bias)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dit.dit_gemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), torch.from_numpy(bias).cuda(), C)
    g = from_dev(C)
    err = np.abs(g - ref)
    # Worst case of the five-slice split: per product, the dropped slice pairs
    # and the slicing remainders stay below 2^-32 of 2^(e_i + f_j) < 4 max|A_i| max|B_j|;
    # plus the final rounding to fp32.
    amax = np.abs(A).max(axis=1).astype(np.float64)
    bmax = np.abs(B).max(axis=1).astype(np.float64)
    bound = 2.0 ** -24 * np.abs(ref) * 1.0001 + K * 2.0 ** -30 * np.outer(amax, bmax) + 1e-30
    assert np.all(err <= bound)
    # and in practice within a correct rounding: rms error under half an fp32 ulp of the rms
    assert np.sqrt(np.mean(err ** 2)) <= 2.0 ** -24 * rms(ref)


@pytest.mark.parametrize("outlier_log2", [10, 14])
def test_gemm_f32_outlier_channels(dit, outlier_log2):
    """Rows whose range is dominated by one channel 2^10 or 2^14 above the rest.
    Each row is scaled by its max, so an element 2^k below the max keeps 35 - k
    bits of its five 7-bit slices: the rigorous bound (dropped slice pairs and
    remainders below K 2^-30 max|A_i| max|B_j|) still holds, but at k = 14 it
    is ~2^-16 of the typical product, beyond a correct fp32 rounding of an
    output whose terms are mostly the small elements.  The test checks the
    rigorous bound and reports the error against a correct rounding."""
    M, N, K = 172, 640, 2560
    rng = np.random.default_rng(50 + outlier_log2)
    A = rng.standard_normal((M, K)).astype(np.float32)
    A[:, 7] *= np.float32(2.0 ** outlier_log2)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ref = O.linear(A, B, np.zeros(N))
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dit.dit_gemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), None, C)
    g = from_dev(C)
    err = np.abs(g - ref)
    amax = np.abs(A).max(axis=1).astype(np.float64)
    bmax = np.abs(B).max(axis=1).astype(np.float64)
    bound = 2.0 ** -24 * np.abs(ref) * 1.0001 + K * 2.0 ** -30 * np.outer(amax, bmax)
    assert np.all(err <= bound)
    ulp_rms = np.sqrt(np.mean(err ** 2)) / (2.0 ** -24 * rms(ref))
    print(f"outlier 2^{outlier_log2}: rms error {ulp_rms:.3f} half-ulps of the output rms, "
          f"max err/bound {(err / bound).max():.3f}")


@pytest.mark.parametrize("M,N,K", [(37, 33, 64), (172, 2560, 2560), (172, 2560, 10240)])
def test_gemm_f32_nonfinite_rows_come_out_nan(dit, M, N, K):
    """A row of A holding a NaN, +Inf or -Inf has no int8 slicing: its output
    row must be NaN (never finite digits), on the direct and the split-K paths,
    and every other row keeps its value."""
    rng = np.random.default_rng(M + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    bad = {3: np.nan, 7: np.inf, 9: -np.inf}
    for r, v in bad.items():
        A[r, (r * 13) % K] = v
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dit.dit_gemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), torch.from_numpy(bias).cuda(), C)
    g = from_dev(C)
    good = [r for r in range(M) if r not in bad]
    for r in bad:
        assert np.isnan(g[r]).all(), f"row {r} not NaN"
    ref = O.linear(A[good], B, bias)
    assert np.isfinite(g[good]).all()
    assert_f32_close(g[good], ref, rel=2e-6, abs_=1e-6, what="finite rows beside non-finite ones")


def test_gemm_packed_equals_alone_bits(dit):
    rng = np.random.default_rng(1)
    A = _bf16_vals(rng, (700, 256))
    B = _bf16_vals(rng, (384, 256), 0.02)
    Ad, Bd = to_bf16_dev(A), to_bf16_dev(B)
    full = torch.empty(700, 384, dtype=torch.bfloat16, device="cuda")
    part = torch.empty(123, 384, dtype=torch.bfloat16, device="cuda")
    dit.dit_gemm(Ad, Bd, None, full)
    dit.dit_gemm(Ad[300:423].contiguous(), Bd, None, part)
    torch.cuda.synchronize()
    assert torch.equal(full[300:423], part)
    Af = torch.from_numpy(rng.standard_normal((172, 512)).astype(np.float32)).cuda()
    Bf = torch.from_numpy(rng.standard_normal((640, 512)).astype(np.float32)).cuda()
    f_full = torch.empty(172, 640, device="cuda")
    f_part = torch.empty(86, 640, device="cuda")
    dit.dit_gemm(Af, Bf, None, f_full)
    dit.dit_gemm(Af[86:].contiguous(), Bf, None, f_part)
    torch.cuda.synchronize()
    assert torch.equal(f_full[86:], f_part)
    # a wide fp32 GEMM (N 20480, K 2560): two row tiles against one
    As = torch.from_numpy(rng.standard_normal((300, 2560)).astype(np.float32)).cuda()
    Bs = torch.from_numpy((rng.standard_normal((20480, 2560)) * 0.02).astype(np.float32)).cuda()
    s_full = torch.empty(300, 20480, device="cuda")
    s_part = torch.empty(86, 20480, device="cuda")
    dit.dit_gemm(As, Bs, None, s_full)
    dit.dit_gemm(As[150:236].contiguous(), Bs, None, s_part)
    torch.cuda.synchronize()
    assert torch.equal(s_full[150:236], s_part)


# ----------------------------------------------------------------------------- modulate + norm

@pytest.mark.parametrize("norm", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,D", [(5, 128), (203, 2560), (77, 6144)])
def test_modnorm(dit, norm, dtype, N, D):
    rng = np.random.default_rng(N + D + norm)
    x = (rng.standard_normal((N, D)) * 2 + 0.5).astype(np.float32)
    n_cond = 3
    mod = (rng.standard_normal((n_cond, 6, D)) * 0.3).astype(np.float32)
    ci = rng.integers(0, n_cond, N).astype(np.int32)
    kind = "rms" if norm == 0 else "layer"
    for which, (ks, kc) in enumerate([(0, 1), (3, 4)]):
        ref = O.modulate(O.norm(x, kind, 1e-6), mod[ci, ks].astype(np.float64), mod[ci, kc].astype(np.float64))
        h = torch.empty(N, D, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
        dit.dit_modnorm(norm, 1e-6, torch.from_numpy(x).cuda(), torch.from_numpy(mod).cuda(), which,
                        torch.from_numpy(ci).cuda(), h)
        if dtype == "f32":
            assert_f32_close(from_dev(h), ref, what="modnorm f32")
        else:
            assert_bf16_rounded(from_dev(h), ref, "modnorm bf16")
    plain = torch.empty(N, D, dtype=torch.float32, device="cuda")
    dit.dit_modnorm(norm, 1e-6, torch.from_numpy(x).cuda(), None, 0, None, plain)
    assert_f32_close(from_dev(plain), O.norm(x, kind, 1e-6), what="plain norm")


@pytest.mark.parametrize("D,N", [(6144, 4103), (2560, 8195)])
@pytest.mark.parametrize("runs", ["random", "contiguous"])
def test_modnorm_many_rows(dit, D, N, runs):
    """Enough rows for the several-rows-per-workgroup launch, with a ragged
    last workgroup: parity with the oracle, and every row bit-identical to the
    same row normalised in a short call (one row per workgroup)."""
    rng = np.random.default_rng(D + N)
    x = (rng.standard_normal((N, D)) * 2 + 0.5).astype(np.float32)
    n_cond = 3
    mod = (rng.standard_normal((n_cond, 6, D)) * 0.3).astype(np.float32)
    if runs == "random":
        ci = rng.integers(0, n_cond, N).astype(np.int32)
    else:  # runs of odd lengths, the way packed segments lie
        bounds = np.sort(rng.choice(np.arange(1, N), 9, replace=False))
        ci = np.zeros(N, np.int32)
        for i, b in enumerate(bounds):
            ci[b:] = (i + 1) % n_cond
    xd, md, cd = torch.from_numpy(x).cuda(), torch.from_numpy(mod).cuda(), torch.from_numpy(ci).cuda()
    for norm in (0, 1):
        kind = "rms" if norm == 0 else "layer"
        ref = O.modulate(O.norm(x, kind, 1e-6), mod[ci, 3].astype(np.float64), mod[ci, 4].astype(np.float64))
        h = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
        dit.dit_modnorm(norm, 1e-6, xd, md, 1, cd, h)
        got = from_dev(h)
        assert_bf16_rounded(got, ref, "modnorm bf16 many rows")
        lo = N - 300
        hs = torch.empty(300, D, dtype=torch.bfloat16, device="cuda")
        dit.dit_modnorm(norm, 1e-6, xd[lo:].contiguous(), md, 1, cd[lo:].contiguous(), hs)
        torch.cuda.synchronize()
        assert torch.equal(hs, h[lo:])


# ----------------------------------------------------------------------------- RoPE + split

@pytest.mark.parametrize("dtype,N,H,hd,rot", [("f32", 160, 4, 32, 32), ("f32", 172, 3, 128, 64),
                                              ("bf16", 301, 5, 128, 128), ("bf16", 64, 2, 128, 64)])
def test_rope_split(dit, dtype, N, H, hd, rot):
    rng = np.random.default_rng(N + H)
    D = H * hd
    qkv = rng.standard_normal((N, 3 * D)).astype(np.float32)
    if dtype == "bf16":
        qkv = torch.from_numpy(qkv).to(torch.bfloat16).float().numpy()
    pos = rng.integers(0, 500, N).astype(np.float64)
    inv = np.array(O.rope_inv_freq(rot, 10000.0))
    cos = np.cos(np.outer(pos, inv)).astype(np.float32)
    sin = np.sin(np.outer(pos, inv)).astype(np.float32)
    tq = torch.from_numpy(qkv).cuda()
    if dtype == "bf16":
        tq = tq.to(torch.bfloat16)
    q, k, v = (torch.empty(H, N, hd, dtype=tq.dtype, device="cuda") for _ in range(3))
    dit.dit_rope_split(tq, H, hd, rot, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), q, k, v)
    for i, (t, rot_it) in enumerate([(q, True), (k, True), (v, False)]):
        src = qkv[:, i * D:(i + 1) * D].reshape(N, H, hd).astype(np.float64)
        ref = O.apply_rope(src, cos, sin, rot) if rot_it else src
        got = from_dev(t).transpose(1, 0, 2)
        if not rot_it:
            assert np.array_equal(got, ref)  # v is a bit-exact copy
        elif dtype == "f32":
            assert_f32_close(got, ref, what="rope f32")
        else:
            assert_bf16_rounded(got, ref, "rope bf16")
        if rot_it:
            assert np.array_equal(got[..., rot:], src[..., rot:])  # partial rotary passes the rest through


# ----------------------------------------------------------------------------- attention

@pytest.mark.parametrize("cu,H,hd", [([0, 64, 160], 4, 32), ([0, 86, 172], 3, 128), ([0, 1, 37, 100], 2, 64)])
def test_attention_f32(dit, cu, H, hd):
    rng = np.random.default_rng(cu[-1] + hd)
    N = cu[-1]
    q, k, v = (rng.standard_normal((H, N, hd)).astype(np.float32) for _ in range(3))
    ref = O.attention_varlen(*(a.transpose(1, 0, 2).astype(np.float64) for a in (q, k, v)), np.array(cu))
    o = torch.empty(N, H * hd, device="cuda")
    cut = torch.tensor(cu, dtype=torch.int32, device="cuda")
    dit.dit_attention(*(torch.from_numpy(a).cuda() for a in (q, k, v)), cut, int(np.diff(cu).max()), o)
    assert_f32_close(from_dev(o), ref.reshape(N, H * hd), what="attention f32")


@pytest.mark.parametrize("cu,H", [([0, 100, 357, 420], 2), ([0, 1, 129, 300], 3), ([0, 1024, 1536], 2)])
def test_attention_bf16(dit, cu, H):
    rng = np.random.default_rng(cu[-1])
    N, hd = cu[-1], 128
    q, k, v = (_bf16_vals(rng, (H, N, hd)) for _ in range(3))
    ref = O.attention_varlen(*(a.transpose(1, 0, 2).astype(np.float64) for a in (q, k, v)), np.array(cu))
    ref = ref.reshape(N, H * hd)
    o = torch.empty(N, H * hd, dtype=torch.bfloat16, device="cuda")
    cut = torch.tensor(cu, dtype=torch.int32, device="cuda")
    dit.dit_attention(*(to_bf16_dev(a) for a in (q, k, v)), cut, int(np.diff(cu).max()), o)
    got = from_dev(o)
    # the output is a bf16 rounding (half an ulp of each value) of a result whose
    # probabilities entered the PV product as bf16: a CPU emulation of exactly
    # that arithmetic differs from the fp64 oracle by up to 0.92% of rms
    assert_bf16_rounded(got, ref, "attention bf16", slack=1.2e-2)
    assert np.abs(got - ref).mean() / rms(ref) < 2e-3


@pytest.mark.parametrize("slope", [0.05, 0.4])
def test_attention_bf16_growing_max(dit, slope):
    """Scores that keep growing along the keys, so the running row max moves
    tile after tile (a few, or every, 64-key tile crosses the kernel's lazy
    max-refresh threshold)."""
    rng = np.random.default_rng(11)
    cu = [0, 700, 1300]
    N, H, hd = cu[-1], 2, 128
    q, k, v = (rng.standard_normal((H, N, hd)).astype(np.float32) for _ in range(3))
    q[:, :, 0] = 4.0
    k[:, :, 0] = slope * np.arange(N, dtype=np.float32)
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in (q, k, v))
    ref = O.attention_varlen(*(a.transpose(1, 0, 2).astype(np.float64) for a in (q, k, v)), np.array(cu))
    ref = ref.reshape(N, H * hd)
    o = torch.empty(N, H * hd, dtype=torch.bfloat16, device="cuda")
    cut = torch.tensor(cu, dtype=torch.int32, device="cuda")
    dit.dit_attention(*(to_bf16_dev(a) for a in (q, k, v)), cut, 700, o)
    got = from_dev(o)
    assert_bf16_rounded(got, ref, "attention bf16 growing max", slack=1.2e-2)
    assert np.abs(got - ref).mean() / rms(ref) < 2e-3


def test_attention_bf16_segmentation_bits(dit):
    rng = np.random.default_rng(7)
    cu = [0, 200, 333]
    N, H, hd = 333, 2, 128
    q, k, v = (_bf16_vals(rng, (H, N, hd)) for _ in range(3))
    cut = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o1 = torch.empty(N, H * hd, dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(*(to_bf16_dev(a) for a in (q, k, v)), cut, 200, o1)
    k2, v2 = k.copy(), v.copy()
    k2[:, 250] += 1.0
    v2[:, 300] -= 1.0
    o2 = torch.empty_like(o1)
    dit.dit_attention(to_bf16_dev(q), to_bf16_dev(k2), to_bf16_dev(v2), cut, 200, o2)
    alone = torch.empty(133, H * hd, dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(*(to_bf16_dev(np.ascontiguousarray(a[:, 200:])) for a in (q, k, v)),
                      torch.tensor([0, 133], dtype=torch.int32, device="cuda"), 133, alone)
    torch.cuda.synchronize()
    assert torch.equal(o1[:200], o2[:200])
    assert not torch.equal(o1[200:], o2[200:])
    assert torch.equal(o1[200:], alone)


# ----------------------------------------------------------------------------- SiLU gate, gated residual

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_silu_gate(dit, dtype):
    rng = np.random.default_rng(3)
    N, F = 37, 1024
    u = (rng.standard_normal((N, 2 * F)) * 3).astype(np.float32)
    t = torch.from_numpy(u).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        u = from_dev(t)
    m = torch.empty(N, F, dtype=t.dtype, device="cuda")
    dit.dit_silu_gate(t, m)
    ref = O.split_mlp(u.astype(np.float64), "gate_up", F)
    if dtype == "f32":
        assert_f32_close(from_dev(m), ref, what="silu f32")
    else:
        assert_bf16_rounded(from_dev(m), ref, "silu bf16")


def test_gated_residual(dit):
    rng = np.random.default_rng(4)
    N, D, n_cond = 99, 512, 4
    x = rng.standard_normal((N, D)).astype(np.float32)
    a = rng.standard_normal((N, D)).astype(np.float32)
    mod = rng.standard_normal((n_cond, 6, D)).astype(np.float32)
    ci = rng.integers(0, n_cond, N).astype(np.int32)
    for which, gk in ((0, 2), (1, 5)):
        xt = torch.from_numpy(x).cuda()
        dit.dit_gated_residual(xt, torch.from_numpy(a).cuda(), torch.from_numpy(mod).cuda(), which,
                               torch.from_numpy(ci).cuda())
        ref = x.astype(np.float64) + mod[ci, gk].astype(np.float64) * a
        assert_f32_close(from_dev(xt), ref, rel=1.2e-7, abs_=1e-7, what="gated residual")
    xt = torch.from_numpy(x).cuda()
    dit.dit_gated_residual(xt, torch.from_numpy(a).cuda(), torch.zeros(n_cond, 6, D, device="cuda"), 0,
                           torch.from_numpy(ci).cuda())
    torch.cuda.synchronize()
    assert torch.equal(xt.cpu(), torch.from_numpy(x))  # a zero gate leaves x bit-identical


def test_gated_residual_f64(dit):
    """The fp32 stream's residual in float64: gate * a is exact in fp64, so the
    update is the fp64 rounding of the exact sum."""
    rng = np.random.default_rng(5)
    N, D, n_cond = 77, 2560, 2
    x = rng.standard_normal((N, D)) * 3.0
    a = rng.standard_normal((N, D)).astype(np.float32)
    mod = rng.standard_normal((n_cond, 6, D)).astype(np.float32)
    ci = rng.integers(0, n_cond, N).astype(np.int32)
    for which, gk in ((0, 2), (1, 5)):
        xt = torch.from_numpy(x).cuda()
        dit.dit_gated_residual(xt, torch.from_numpy(a).cuda(), torch.from_numpy(mod).cuda(), which,
                               torch.from_numpy(ci).cuda())
        ref = x + mod[ci, gk].astype(np.float64) * a.astype(np.float64)
        assert np.array_equal(from_dev(xt), ref)  # numpy's fp64 a*b + x rounds the same way


@pytest.mark.parametrize("norm", [0, 1])
def test_modnorm_f64_residual(dit, norm):
    rng = np.random.default_rng(6 + norm)
    N, D, n_cond = 203, 2560, 3
    x = rng.standard_normal((N, D)) * 2 + 0.5 + rng.standard_normal((N, D)) * 1e-9  # below fp32 resolution
    mod = (rng.standard_normal((n_cond, 6, D)) * 0.3).astype(np.float32)
    ci = rng.integers(0, n_cond, N).astype(np.int32)
    kind = "rms" if norm == 0 else "layer"
    ref = O.modulate(O.norm(x, kind, 1e-6), mod[ci, 0].astype(np.float64), mod[ci, 1].astype(np.float64))
    h = torch.empty(N, D, dtype=torch.float32, device="cuda")
    dit.dit_modnorm(norm, 1e-6, torch.from_numpy(x).cuda(), torch.from_numpy(mod).cuda(), 0, torch.from_numpy(ci).cuda(), h)
    assert_f32_close(from_dev(h), ref, rel=2.0 ** -23, abs_=1e-12, what="modnorm f64 residual")
