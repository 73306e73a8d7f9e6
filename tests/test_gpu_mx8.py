"""The MXFP8 arm through the C ABI: the device re-quantization bit for bit
against the oracle's, the scaled fp8 GEMM against the oracle's product of the
dequantized operands, and whole bf16-stream blocks and forwards with their
four GEMMs on MXFP8 against the oracle's 'mxfp8' mode and its control arm."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import assert_bf16_parity, assert_bf16_rounded, from_dev, rms, to_bf16_dev
from synthetic.configs import Segment, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    from video_audio_gen_amd import dit as d
    d.load()
    return d


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _special_rows(rng, K):
    """Rows whose blocks hit the quantizer's edge cases."""
    rows = []
    base = rng.standard_normal(K)
    r = base.copy(); r[:32] = 0.0; r[5] = -0.0; rows.append(r)             # all-zero block with a -0
    r = base.copy(); r[32:64] = 0.0; r[40] = np.nan; rows.append(r)        # NaN block
    r = base.copy(); r[64:96] *= 0; r[70] = -np.inf; rows.append(r)        # Inf block
    r = base.copy(); r[0] = 1.75; r[1:32] = 0.01; rows.append(r)           # max mantissa exactly 1.75 (scale 2^-8)
    r = base.copy(); r[0] = 1.7578125; r[1:32] = 0.01; rows.append(r)      # next bf16 above: scale 2^-7
    r = base.copy(); r[:32] = np.exp2(-np.arange(32.0)); rows.append(r)    # a block reaching into E4M3 subnormals
    r = base.copy(); r[:32] *= 2.0 ** 100; r[32:64] *= 2.0 ** -120; rows.append(r)  # extreme scales
    # exact E4M3 ties after scaling: 448 sets the scale 2^0, then midpoints between codes
    r = base.copy(); r[0] = 448.0; r[1:8] = [1.0625, 1.1875, 3.0 * 2 ** -10, 2.0 ** -10, 232.0, 240.0 + 8, 13.5]
    rows.append(r)
    return np.array(rows)


@pytest.mark.parametrize("R,K", [(7, 32), (300, 6144), (64, 16384), (1, 128)])
def test_quantize_mx8_bit_exact(dit, R, K):
    rng = np.random.default_rng(R + K)
    x = rng.standard_normal((R, K)) * np.exp2(rng.integers(-30, 30, (R, 1)))
    if K >= 128:
        sp = _special_rows(rng, K)
        x[:len(sp)] = sp[:R]
    x = _bf16(x)
    codes_o, scales_o = O.quantize_mx8(x)
    xd = to_bf16_dev(x)
    codes = torch.empty(R, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(R, K // 32, dtype=torch.uint8, device="cuda")
    dit.dit_quantize_mx8(xd, codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), scales_o)
    assert np.array_equal(codes.cpu().numpy(), codes_o)


def test_quantize_mx8_every_bf16_value(dit):
    """Every bf16 bit pattern (NaNs and infinities included) through the device
    quantizer, bit for bit against the oracle: in blocks of 32 consecutive
    patterns (each block's values share a binade, so they land on the upper
    E4M3 codes), in blocks shifted by 16 patterns (straddling binades), and in
    a seeded shuffle (mixed magnitudes: the small values of a block fall into
    the E4M3 subnormals and to signed zeros).  The device encodes with the
    hardware fp8 conversion; this pins it to the nearest-even definition."""
    pats = np.arange(65536, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        vals = pats.view(np.float32).astype(np.float64)
    rng = np.random.default_rng(7)
    x = np.concatenate([vals, np.roll(vals, 16), vals[rng.permutation(65536)]]).reshape(-1, 128)
    codes_o, scales_o = O.quantize_mx8(x)
    xd = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(x.shape[0], x.shape[1] // 32, dtype=torch.uint8, device="cuda")
    dit.dit_quantize_mx8(xd, codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), scales_o)
    assert np.array_equal(codes.cpu().numpy(), codes_o)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (300, 320, 256), (513, 768, 384), (65, 97, 128),
                                   (26624 // 8, 18432 // 8, 6144), (200, 6144, 16384)])
def test_gemm_mx8(dit, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = _bf16(rng.standard_normal((M, K)))
    B = _bf16(rng.standard_normal((N, K)) * 0.02)
    bias = rng.standard_normal(N).astype(np.float32)
    ref = O.linear_mx8(A, B, bias)
    Ad, Bd = to_bf16_dev(A), to_bf16_dev(B)
    C32 = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dit.dit_gemm(Ad, Bd, torch.from_numpy(bias).cuda(), C32, mxfp8=True)
    g = from_dev(C32)
    # the products of E4M3 values times power-of-two scales are exact; the
    # matrix cores sum them in reduced precision: the error is measured
    # against the sum of the products' magnitudes
    Aq = O.dequantize_mx8(*O.quantize_mx8(A))
    Bq = O.dequantize_mx8(*O.quantize_mx8(B))
    mag = np.abs(Aq) @ np.abs(Bq).T
    e = np.abs(g - ref) / mag
    print(f"mx8 gemm {M}x{N}x{K}: max|d| {np.abs(g - ref).max():.3e} rms {rms(ref):.3e} "
          f"err/sum|ab|: max {e.max():.3e} mean {e.mean():.3e} (2^{np.log2(e.max()):.1f})")
    # the scaled fp8 instruction sums a step's 64 products on a grid well
    # below fp32 (measured 2^-16 of their magnitude sum at K 128 - 384)
    assert e.max() <= 2.0 ** -14
    C16 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dit.dit_gemm(Ad, Bd, torch.from_numpy(bias).cuda(), C16, mxfp8=True)
    # the bf16 epilogue rounds the same fp32 sum the fp32 epilogue stores
    assert torch.equal(C16, C32.to(torch.bfloat16))


def test_gemm_mx8_exact_on_small_integer_products(dit):
    """Operands whose values are small integers (each block's max 4 or 8, one
    power of two per block) and whose every partial sum is an integer below
    2^15: the product must come out exact whatever the accumulator's width (a
    wrong scale byte, block or lane half shows as a wrong integer)."""
    rng = np.random.default_rng(5)
    M, N, K = 96, 160, 256
    A = rng.integers(-3, 4, (M, K)).astype(np.float64)
    B = rng.integers(-3, 4, (N, K)).astype(np.float64)
    A[:, ::32] = 4.0
    B[:, ::32] = -4.0
    A *= np.exp2(rng.integers(0, 2, (M, K // 32))).repeat(32, axis=1)
    B *= np.exp2(rng.integers(0, 2, (N, K // 32))).repeat(32, axis=1)
    ref = A @ B.T
    assert (np.abs(A) @ np.abs(B).T).max() < 2 ** 15
    assert np.array_equal(O.linear_mx8(A, B, np.zeros(N)), ref)
    C = torch.empty(M, N, dtype=torch.float32, device="cuda")
    dit.dit_gemm(to_bf16_dev(A), to_bf16_dev(B), None, C, mxfp8=True)
    assert np.array_equal(from_dev(C), ref)


def test_gemm_mx8_packed_equals_alone_bits(dit):
    rng = np.random.default_rng(1)
    A = to_bf16_dev(_bf16(rng.standard_normal((700, 256))))
    B = to_bf16_dev(_bf16(rng.standard_normal((384, 256)) * 0.02))
    full = torch.empty(700, 384, dtype=torch.float32, device="cuda")
    part = torch.empty(123, 384, dtype=torch.float32, device="cuda")
    dit.dit_gemm(A, B, None, full, mxfp8=True)
    dit.dit_gemm(A[300:423].contiguous(), B, None, part, mxfp8=True)
    torch.cuda.synchronize()
    assert torch.equal(full[300:423], part)


def test_gemm_mx8_nonfinite_block_gives_nan_row(dit):
    rng = np.random.default_rng(2)
    A = _bf16(rng.standard_normal((40, 256)))
    A[3, 100] = np.nan
    A[9, 7] = np.inf
    B = _bf16(rng.standard_normal((64, 256)) * 0.02)
    C = torch.empty(40, 64, dtype=torch.float32, device="cuda")
    dit.dit_gemm(to_bf16_dev(A), to_bf16_dev(B), None, C, mxfp8=True)
    g = from_dev(C)
    assert np.isnan(g[3]).all() and np.isnan(g[9]).all()
    good = [r for r in range(40) if r not in (3, 9)]
    assert np.isfinite(g[good]).all()


# ----------------------------------------------------------------------------- whole blocks and forwards

@pytest.fixture(scope="module")
def H():
    import harness
    from video_audio_gen_amd import dit
    dit.load()
    return harness


def _stage(H, cfg, w):
    from video_audio_gen_amd import dit
    m = dit.Model(cfg)
    dit.dit_stage_weights(m, w, as_bf16=True)
    dit.dit_stage_finalize(m)
    return m


def _run(H, cfg):
    w = S.all_weights(cfg, 0, threads=8)
    r = H.Runner(cfg, 0, model=_stage(H, cfg, w))
    r.forward()
    return r, w, r.output_numpy()


def _oracle(cfg, w, inp, accum="fp64"):
    isl = {k: v for k, v in w.items() if not k.startswith("blocks.")}
    return O.forward(cfg, lambda b: w, isl, inp, threads=8, accum=accum)


# The control arm of the MXFP8 mode accumulates each 64-product step on a
# fixed-point grid 16 bits below its magnitude sum (oracle.linear, accum
# 'mx_step'): the precision class of the scaled fp8 instruction, which an fp32
# control would understate.
MX_CONTROL = "mx_step"


C3_MX_SMALL = scaled(S.get_config("c3_mxfp8"), segments=(Segment(0, (2, 8, 16), 0), Segment(1, (64,), 1)))
C4_MX_SMALL = scaled(S.get_config("c4_mxfp8"), n_blocks=2,
                     segments=(Segment(0, (1, 4, 8), 0), Segment(1, (24,), 1), Segment(0, (2, 2, 4), 2),
                               Segment(1, (40,), 3)))


def test_c3_block_mxfp8_parity(H):
    cfg = C3_MX_SMALL
    H.dit.dit_counters_reset()  # the launch counts below are this forward's alone
    r, w, got = _run(H, cfg)
    c = H.dit.dit_counters()
    # four block GEMMs per block on MXFP8 operands; one re-quantization launch
    # per block (the MLP-out input m: h, o and h2 come quantized from the
    # kernels that produce them)
    assert c["gemm_mx8"] == 4 * cfg.n_blocks and c["quantize_mx8"] == cfg.n_blocks
    ref = _oracle(cfg, w, r.inp)
    ctl = _oracle(cfg, w, r.inp, accum=MX_CONTROL)
    assert_bf16_parity(got["x"], ref["x"], ctl["x"], "c3 block mxfp8 (320 tokens)")
    # the arm is a different computation from the bf16 one: it moves the block by its fp8 rounding
    bf = _oracle(scaled(cfg, gemm="stream"), w, r.inp)
    d = np.abs(ref["x"] - bf["x"]).max() / rms(bf["x"])
    print(f"mxfp8 vs bf16 oracle: max|d|/rms {d:.3e}")
    assert d > 1e-3


def test_c4_io_mxfp8_parity(H):
    cfg = C4_MX_SMALL
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    ctl = _oracle(cfg, w, r.inp, accum=MX_CONTROL)
    for k in ref:
        assert_bf16_parity(got[k], ref[k], ctl[k], f"c4 mxfp8 small (2 blocks) {k}")


def test_mxfp8_zero_gate_identity_and_packed_equals_alone(H):
    cfg = C3_MX_SMALL
    w = S.all_weights(cfg, 0, threads=8)
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    mod = torch.randn(cfg.n_cond, 6, cfg.hidden, device="cuda")
    mod[:, 2] = 0
    mod[:, 5] = 0
    x = r.x_in.clone()
    H.dit.dit_block_forward(m, 0, x, mod, r.batch, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(x, r.x_in)
    r.forward()
    packed = r.output_numpy()["x"]
    lay = O.pack_layout(cfg)
    for i, seg in enumerate(cfg.segments):
        a, b = int(lay["cu_seqlens"][i]), int(lay["cu_seqlens"][i + 1])
        one = scaled(cfg, segments=(seg,))
        batch = H.dit.Batch(m, one.segments, H.cond_modality(cfg))
        ws = H.dit.workspace(batch)
        xi = r.x_in[a:b].contiguous()
        out = torch.empty_like(xi)
        H.dit.dit_forward(m, batch, xi, r.cond, out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), packed[a:b]), f"segment {i}"
