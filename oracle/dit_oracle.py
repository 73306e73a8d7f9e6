"""Plain, slow CPU oracle of the diffusion-transformer (DiT) block forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py, never by the library.  It shares no code,
table or constant generator with the HIP path; the only common module is the
seeded input generator in ``synthetic/``.

What it computes is the plain definition of a transformer block with adaptive
layer-norm (AdaLN) conditioning, written out step by step in numpy float64.  The
steps and their sources:

  * RMSNorm / LayerNorm and an indexed AdaLN modulate, a fused QKV GEMM with
    output order [q_all | k_all | v_all], NeoX rotate_half RoPE from a per-row
    cos/sin cache, non-causal packed attention over cu_seqlens, out projection,
    gated residual, gated-SiLU MLP, gated residual -- page "port the MiniMax-H3
    omni-modal video+audio DiT", section "The device-resident forward (W2b)",
    and the same page's update "Encoder vision block ported" for the qkv order;
  * LayerNorm, partial rotary, value*silu(gate) over a merged projection, 1x1
    convolutions as GEMMs on the frame-major activation -- page "the 2.4B fp32
    DiT onto the device, staged once", section "What moved, and onto what";
  * the position grid in fp64 feeding RoPE, and packed layout / patchify --
    page "port the MiniMax-H3 omni-modal video+audio DiT", section "Correctness
    gates" (table rows on the packed layout, the fp64 grid and patchify);
  * cos/sin built on the host before any kernel -- page "stream the ORIGINAL
    bf16 DiT to the device", section "What this enables";
  * rectified-flow time-shift sigma schedule, euler eta=0 with rf_v_to_x0 --
    page "port the MiniMax-H3 omni-modal video+audio DiT", update "quantized
    arms land" item 2 and milestone "the whole t2va path composes end to end";
  * the music model's loop of DiT forwards over two classifier-free-guidance
    branches per step -- page "the 2.4B fp32 DiT onto the device, staged
    once", opening paragraph (steps x 2 CFG branches x windows).

Where the pages leave a step open, the plainest reading is taken; each reading
is named in the docstring of the function that takes it.

Precision modes:
  'fp64'  -- every step in float64, no storage rounding (fp32 workloads);
  'bf16'  -- float64 math with round-to-nearest-even to bf16 at the storage
             points of a bf16 block stream with fp32 islands (listed in
             ``block_forward``).  The residual stream, the modulation table,
             the time embedding and the projections in and out stay fp32;
  'mxfp8' -- as 'bf16', with the four block GEMMs' operands re-quantized to
             MXFP8 (``quantize_mx8``) and dequantized before the product;
  'mxfp4' -- as 'mxfp8', with the four block GEMMs' weights re-quantized to
             MXFP4 (``quantize_mx4``) instead (activations stay MXFP8).

Pins: tests/test_oracle_pins.py checks every function here against closed
forms, invariants and brute force; tests/test_oracle_wiring_pins.py pins the
wiring between them -- q and k roles and the RoPE target (scores through the
relative position), the in/out projections and the final norm (closed form of
an islands-only forward), every bf16 storage point (a block rounded by hand)
and the timestep of each denoise step (hand fractions).  Each of those pins
was run against an oracle carrying the mutation it names.  The random-weight
forward as a whole has no printed value to meet: the pages' accuracy figures
belong to a model and inputs that are not available.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "round_bf16", "round_f32", "pack_layout", "token_positions", "rope_inv_freq", "rope_cache",
    "timestep_embedding", "cond_embeddings", "norm", "modulate", "linear", "apply_rope",
    "attention_varlen", "attention_dense_masked", "silu", "adaln_table", "block_forward",
    "patchify", "unpatchify", "forward", "sigma_schedule", "sigma_dt", "euler_step",
    "denoise_step_conditions", "denoise_loop", "split_mlp", "cfg_pairs", "cfg_combine",
    "cfg_denoise_loop", "e4m3_value", "e8m0_value", "e4m3_encode", "e4m3_encode_array", "quantize_mx8", "dequantize_mx8",
    "linear_mx8", "centered_rope_cache", "rms_affine", "vit_block_forward",
    "e2m1_value", "e2m1_encode", "e2m1_encode_array", "quantize_mx4", "dequantize_mx4", "pack_e2m1", "linear_mx4",
]


# ----------------------------------------------------------------------------- rounding

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps float32's 8-bit exponent and 7 stored mantissa bits, so in a
    float64 encoding the 45 low mantissa bits are rounded away.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64).copy()
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u += np.uint64((1 << 44) - 1) + lsb
    u &= ~np.uint64((1 << 45) - 1)
    return u.view(np.float64).reshape(x.shape)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _store(x: np.ndarray, mode: str) -> np.ndarray:
    """A bf16 storage point of the block stream (identity in 'fp64' mode)."""
    return round_bf16(x) if mode in ("bf16", "mxfp8", "mxfp4") else x


def _store_f32(x: np.ndarray, mode: str) -> np.ndarray:
    """An fp32 storage point of a bf16 stream (identity in 'fp64' mode)."""
    return round_f32(x) if mode in ("bf16", "mxfp8", "mxfp4") else x


# ----------------------------------------------------------------------------- MX block scaling (fp8)
#
# The low-precision GEMM path.  The pages' speed path is NVFP4 (FP4 values,
# one E4M3 scale per group of 16 along K plus an fp32 global scale; page "port
# the MiniMax-H3 omni-modal video+audio DiT", update "NVFP4 arm grounded" and
# "Not yet built -- honestly recorded").  The matrix cores of this GPU take
# the OCP microscaling (MX) formats instead: 32 consecutive K values share one
# power-of-two scale (E8M0), the values are OCP FP8 E4M3.  Reading taken: both
# operands of the four block GEMMs of a bf16 stream are re-quantized to MXFP8
# from their bf16 values (weights at staging, activations before each GEMM);
# the scale of a block is the smallest power of two 2^s with max|v| <= 448 2^s
# (so no value of the block saturates: the OCP rule 2^(floor(log2 max|v|) - 8)
# would clamp the block maximum by up to 1/8 whenever its leading digits
# exceed 1.75), each value divided by it is rounded to nearest-even E4M3;
# s is clamped to [-127, 127]; an all-zero block takes the smallest scale
# 2^-127 and a block holding a NaN or an Inf the NaN scale (byte 255).

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 byte: sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal (m 2^-9); S.1111.111 is NaN."""
    code = int(code) & 0xFF
    sgn = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sgn * m * 2.0 ** -9
    return sgn * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e8m0_value(byte: int) -> float:
    """Value of an E8M0 scale byte: 2^(byte - 127); 255 is NaN."""
    byte = int(byte) & 0xFF
    return float("nan") if byte == 255 else 2.0 ** (byte - 127)


def _half_even(x: float) -> int:
    """Nearest integer to x >= 0, ties to even."""
    f = math.floor(x)
    r = x - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        f += 1
    return int(f)


def e4m3_encode(y: float) -> int:
    """Round y to nearest-even OCP E4M3, clamped to +-448 (the sign of y kept, -0 included)."""
    sgn = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a >= E4M3_MAX:
        return sgn | 0x7E
    if a < 2.0 ** -6:                       # subnormal range: steps of 2^-9 (8 steps reach 2^-6, code 0x08)
        return sgn | _half_even(a * 2.0 ** 9)
    e = math.frexp(a)[1] - 1                # a = mant 2^e, mant in [1, 2)
    q = _half_even((a / 2.0 ** e - 1.0) * 8.0)
    if q == 8:
        e, q = e + 1, 0
    return sgn | ((e + 7) << 3) | q


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    """``e4m3_encode`` over an array (the same steps, vectorized: np.rint
    rounds half to even)."""
    y = np.asarray(y, np.float64)
    sgn = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.abs(y)
    sub = a < 2.0 ** -6
    e = np.frexp(np.where(sub, 1.0, a))[1] - 1
    q = np.rint((np.where(sub, 1.0, a) / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    mag = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), ((e + 7) << 3) | q)
    mag = np.where(a >= E4M3_MAX, 0x7E, mag)
    return (sgn | mag).astype(np.uint8)


def quantize_mx8(v: np.ndarray):
    """MXFP8 quantization of the rows of v [R, K] (K a multiple of 32):
    returns (codes uint8 [R, K], scales uint8 [R, K/32])."""
    v = np.asarray(v, np.float64)
    R, K = v.shape
    assert K % MX_BLOCK == 0
    blk = v.reshape(R, K // MX_BLOCK, MX_BLOCK)
    finite = np.isfinite(blk).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(blk), blk, 0.0)).max(axis=2), 0.0)
    e = np.frexp(amax)[1] - 1                                        # amax = m 2^e, m in [1, 2)
    over = amax / np.exp2(e.astype(np.float64)) > E4M3_MAX / 256.0     # m > 1.75: 2^(e-8) would clamp
    shared = np.clip(e - 8 + over, -127, 127)
    scales = np.where(amax > 0, shared + 127, 0)
    scales = np.where(finite, scales, 255).astype(np.uint8)
    X = np.exp2(np.where(amax > 0, shared, 0).astype(np.float64))[..., None]
    codes = e4m3_encode_array(np.where(finite[..., None], blk, 0.0) / X)
    # an all-zero block keeps each zero's sign; a non-finite block has zero codes
    codes = np.where(finite[..., None], codes, 0).astype(np.uint8)
    return codes.reshape(R, K), scales


_E4M3_TABLE = None


def dequantize_mx8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of MXFP8 rows: E4M3 value times its block's E8M0 scale."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], np.float64)
    vals = _E4M3_TABLE[np.asarray(codes, np.uint8)]
    sc = np.array([e8m0_value(b) for b in range(256)], np.float64)[np.asarray(scales, np.uint8)]
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)


def linear_mx8(x: np.ndarray, W: np.ndarray, b: np.ndarray, accum: str = "fp64") -> np.ndarray:
    """y = Q(x) Q(W)^T + b: both operands quantized to MXFP8 along K and
    dequantized, then the plain product (the scaled matrix cores' definition)."""
    xq = dequantize_mx8(*quantize_mx8(x))
    wq = dequantize_mx8(*quantize_mx8(W))
    return linear(xq, wq, b, accum)


# ----------------------------------------------------------------------------- MX block scaling (fp4 weights)
#
# The pages' FP4 path keeps the activations at 16 bits and quantizes the
# weights to 4-bit values with block scales (W4A16; page "port the
# MiniMax-H3 omni-modal video+audio DiT", update "NVFP4 arm grounded").  The
# matrix cores here multiply an FP4 operand only against another MX operand,
# so the reading taken: the four block GEMMs' weights re-quantized to MXFP4 at
# staging -- OCP E2M1 values, one E8M0 scale per 32 along K -- against the
# activations in MXFP8 as above (W4A8).  E2M1: a sign bit, two exponent bits
# (bias 1) and one mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no
# Inf or NaN.  The scale of a block is the smallest power of two 2^s with
# max|v| <= 6 2^s (the OCP rule 2^(floor(log2 max|v|) - 2) would clamp the
# block maximum whenever its leading digits exceed 1.5), each value divided
# by it is rounded to the nearest E2M1 value, ties to the even mantissa bit;
# the zero and non-finite blocks as for MXFP8.  Stored two values per byte,
# the value at even K in the low nibble.

E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of an OCP FP4 E2M1 nibble: sign (bit 3), 2 exponent bits (bias 1),
    1 mantissa bit; exponent 0 is subnormal (m / 2)."""
    code = int(code) & 0xF
    sgn = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    if e == 0:
        return sgn * m * 0.5
    return sgn * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e2m1_encode(y: float) -> int:
    """Round y to the nearest E2M1 value (ties to the even mantissa bit),
    clamped to +-6; the sign of y kept, -0 included."""
    sgn = 0x8 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a >= E2M1_MAX:
        return sgn | 0x7
    if a < 1.0:                             # subnormal range: steps of 0.5 (two steps reach 1.0, code 2)
        return sgn | _half_even(a * 2.0)
    e = math.frexp(a)[1] - 1                # a = mant 2^e, mant in [1, 2), e in {0, 1, 2}
    q = _half_even((a / 2.0 ** e - 1.0) * 2.0)
    if q == 2:
        e, q = e + 1, 0
    return sgn | ((e + 1) << 1) | q


def e2m1_encode_array(y: np.ndarray) -> np.ndarray:
    """``e2m1_encode`` over an array (the same steps, vectorized: np.rint
    rounds half to even)."""
    y = np.asarray(y, np.float64)
    sgn = np.where(np.signbit(y), 0x8, 0).astype(np.int64)
    a = np.abs(y)
    sub = a < 1.0
    e = np.frexp(np.where(sub, 1.0, a))[1] - 1
    q = np.rint((np.where(sub, 1.0, a) / np.exp2(e.astype(np.float64)) - 1.0) * 2.0).astype(np.int64)
    carry = q == 2
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    mag = np.where(sub, np.rint(a * 2.0).astype(np.int64), ((e + 1) << 1) | q)
    mag = np.where(a >= E2M1_MAX, 0x7, mag)
    return (sgn | mag).astype(np.uint8)


def quantize_mx4(v: np.ndarray):
    """MXFP4 quantization of the rows of v [R, K] (K a multiple of 32):
    returns (codes uint8 [R, K], one E2M1 code 0..15 per value, and
    scales uint8 [R, K/32])."""
    v = np.asarray(v, np.float64)
    R, K = v.shape
    assert K % MX_BLOCK == 0
    blk = v.reshape(R, K // MX_BLOCK, MX_BLOCK)
    finite = np.isfinite(blk).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(blk), blk, 0.0)).max(axis=2), 0.0)
    e = np.frexp(amax)[1] - 1                                        # amax = m 2^e, m in [1, 2)
    over = amax / np.exp2(e.astype(np.float64)) > E2M1_MAX / 4.0       # m > 1.5: 2^(e-2) would clamp
    shared = np.clip(e - 2 + over, -127, 127)
    scales = np.where(amax > 0, shared + 127, 0)
    scales = np.where(finite, scales, 255).astype(np.uint8)
    X = np.exp2(np.where(amax > 0, shared, 0).astype(np.float64))[..., None]
    codes = e2m1_encode_array(np.where(finite[..., None], blk, 0.0) / X)
    codes = np.where(finite[..., None], codes, 0).astype(np.uint8)
    return codes.reshape(R, K), scales


def dequantize_mx4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of MXFP4 rows: E2M1 value times its block's E8M0 scale."""
    vals = np.array([e2m1_value(c) for c in range(16)], np.float64)[np.asarray(codes, np.uint8) & 0xF]
    sc = np.array([e8m0_value(b) for b in range(256)], np.float64)[np.asarray(scales, np.uint8)]
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte, the code at even K in the low nibble: [R, K] -> [R, K/2]."""
    c = np.asarray(codes, np.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def linear_mx4(x: np.ndarray, W: np.ndarray, b: np.ndarray, accum: str = "fp64") -> np.ndarray:
    """y = Q8(x) Q4(W)^T + b: the activation quantized to MXFP8 and the weight
    to MXFP4 along K, both dequantized, then the plain product."""
    xq = dequantize_mx8(*quantize_mx8(x))
    wq = dequantize_mx4(*quantize_mx4(W))
    return linear(xq, wq, b, accum)


# ----------------------------------------------------------------------------- layout

def pack_layout(cfg) -> Dict[str, np.ndarray]:
    """Packed layout of a batch of segments (documents).

    Segments are laid end to end in the order given.  cu_seqlens holds the
    running token offsets; cond_idx names each token's modulation row; doc_id
    and modality name each token's segment and modality.  (Page "port the
    MiniMax-H3 omni-modal video+audio DiT", section "Correctness gates": the
    packed layout -- ids, tags, cu_seqlens, doc ids -- gated exact.)
    """
    cu = [0]
    cond, doc, mod = [], [], []
    for i, s in enumerate(cfg.segments):
        n = 1
        for g in s.grid:
            n *= g
        cu.append(cu[-1] + n)
        cond += [s.cond_row] * n
        doc += [i] * n
        mod += [s.modality] * n
    return {"cu_seqlens": np.array(cu, np.int32), "cond_idx": np.array(cond, np.int32),
            "doc_id": np.array(doc, np.int32), "modality": np.array(mod, np.int32)}


def token_positions(cfg) -> List[List[int]]:
    """Integer position of every packed token on each rope axis of its segment.

    Reading taken: positions restart at 0 in every document and run in raster
    order over the segment's grid with the last axis fastest, (t, h, w) for a
    3-axis grid and (i,) for a 1-axis grid -- an integer fp64 position grid.
    """
    out: List[List[int]] = []
    for s in cfg.segments:
        g = s.grid
        if len(g) == 1:
            out += [[i] for i in range(g[0])]
        elif len(g) == 3:
            for t in range(g[0]):
                for h in range(g[1]):
                    for w in range(g[2]):
                        out.append([t, h, w])
        else:
            raise ValueError("grid must have 1 or 3 axes")
    return out


def rope_inv_freq(axis_dim: int, theta: float) -> List[float]:
    """Inverse frequencies of one rope axis of sub-dimension ``axis_dim``.

    inv_freq[j] = 1 / theta^(2j / axis_dim), j < axis_dim/2, in fp64 (the
    standard NeoX/RoFormer spacing restricted to the axis' own sub-dimension).
    """
    return [1.0 / theta ** ((2 * j) / axis_dim) for j in range(axis_dim // 2)]


def rope_cache(cfg):
    """Per-row cos/sin cache [N, rot/2] (float32), built in fp64 on the host.

    For each token the angle vector is the concatenation over the segment's
    axes of pos_a * inv_freq_a; cos and sin are taken with scalar libm in fp64
    and rounded once to float32.  Reading taken for several axes: each axis
    owns a block of rot/2 frequencies and rotate_half pairs dimension i with
    i + rot/2, the same concatenate-then-tile-twice scheme the pages describe
    for their ND rotary embedding (page "port the MiniMax-H3 omni-modal
    video+audio DiT", update "video-VAE ViT3D decoder complete").
    """
    half = cfg.rot_dim // 2
    pos = token_positions(cfg)
    n = len(pos)
    cos = np.empty((n, half), np.float32)
    sin = np.empty((n, half), np.float32)
    freqs = [[rope_inv_freq(d, cfg.theta) for d in m.rope_axes] for m in cfg.modalities]
    two_pi = 2.0 * math.pi
    row = 0
    for s in cfg.segments:
        fr = freqs[s.modality]
        centered = getattr(cfg.modalities[s.modality], "rope_grid", "integer") == "centered"
        assert len(fr) == len(s.grid), "segment grid must have one extent per rope axis"
        assert sum(len(f) for f in fr) == half
        for _ in range(s.n_tokens):
            p = pos[row]
            col = 0
            for a, fa in enumerate(fr):
                pa = float(p[a])
                for f in fa:
                    if centered:  # the ND rotary embedding's coordinates (``centered_rope_cache``)
                        ang = (two_pi * ((2.0 * pa + 1.0) / s.grid[a] - 1.0)) * f
                    else:
                        ang = pa * f
                    cos[row, col] = math.cos(ang)
                    sin[row, col] = math.sin(ang)
                    col += 1
            row += 1
    return cos, sin


# ----------------------------------------------------------------------------- conditioning

def timestep_embedding(t: float, dim: int) -> np.ndarray:
    """Sinusoidal timestep embedding, float32 values.

    Reading taken (the pages name a time embedder but print no formula):
    [cos(t f_j) for j < dim/2] ++ [sin(t f_j) for j < dim/2] with
    f_j = 10000^(-j/(dim/2)), t unscaled in [0, 1], no SiLU after it; computed
    in fp64 with scalar libm and rounded once to float32 (an fp32 island).
    """
    h = dim // 2
    t = float(np.float32(t))
    e = np.empty(dim, np.float32)
    for j in range(h):
        f = 10000.0 ** (-j / h)
        e[j] = math.cos(t * f)
        e[h + j] = math.sin(t * f)
    return e


def cond_embeddings(cfg, t_rows: Optional[Sequence[float]] = None,
                    cond: Optional[np.ndarray] = None) -> np.ndarray:
    """[n_cond, cond_dim] conditioning vectors that feed the AdaLN linears.

    Timestep conditioning: row c embeds the timestep of its request (or the
    explicit per-row ``t_rows``).  Vector conditioning (the music model's
    conditional / unconditional CFG branches): row c is conditioning vector
    ``source``.
    """
    out = np.empty((cfg.n_cond, cfg.cond_dim), np.float64)
    for c, r in enumerate(cfg.cond_rows):
        if cfg.cond_kind == "timestep":
            out[c] = timestep_embedding(t_rows[c], cfg.cond_dim)
        else:
            out[c] = cond[r.source]
    return out


def adaln_table(cfg, bw: Dict[str, np.ndarray], b: int, emb: np.ndarray, mode: str) -> np.ndarray:
    """Modulation rows [n_cond, 6, D] of block ``b``: W_ada[m] . e_c + bias_ada[m].

    Row c uses the AdaLN linear of its modality ("two indexed AdaLN modulates",
    page "port the MiniMax-H3 omni-modal video+audio DiT", section "The
    device-resident forward (W2b)").  Reading taken for the order of the six
    vectors: shift_msa, scale_msa, gate_msa, shift_mlp, scale_mlp, gate_mlp.
    The table is stored in fp32 in a bf16 stream.
    """
    D = cfg.hidden
    out = np.empty((cfg.n_cond, 6, D), np.float64)
    for c, r in enumerate(cfg.cond_rows):
        W = bw[f"blocks.{b}.adaln.{r.modality}.weight"].astype(np.float64)
        bias = bw[f"blocks.{b}.adaln.{r.modality}.bias"].astype(np.float64)
        out[c] = (W @ emb[c] + bias).reshape(6, D)
    return _store_f32(out, mode)


# ----------------------------------------------------------------------------- block pieces

def norm(x: np.ndarray, kind: str, eps: float) -> np.ndarray:
    """Row normalisation without affine weights (AdaLN supplies scale and shift).

    RMS: x / sqrt(mean(x^2) + eps).  Layer: (x - mean) / sqrt(var + eps) with
    the population variance.
    """
    x = np.asarray(x, np.float64)
    if kind == "rms":
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if kind == "layer":
        mu = np.mean(x, axis=-1, keepdims=True)
        d = x - mu
        return d / np.sqrt(np.mean(d * d, axis=-1, keepdims=True) + eps)
    raise ValueError(kind)


def modulate(y: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """AdaLN modulate y * (1 + scale) + shift (reading taken: the DiT form, in
    which zero modulation passes the normalised value through)."""
    return y * (1.0 + scale) + shift


def linear(x: np.ndarray, W: np.ndarray, b: np.ndarray, accum: str = "fp64") -> np.ndarray:
    """y = x W^T + b with W in nn.Linear layout [out, in] (MatmulBT plus a rank-1 bias add,
    page "the 2.4B fp32 DiT onto the device, staged once", section "What moved").

    accum='fp32' runs the product in float32 (numpy's sgemm) instead: the
    control arm, a second valid accumulation order used to measure how far two
    correct implementations drift apart through the storage roundings.
    """
    if accum == "fp32":
        y = np.asarray(x, np.float32) @ np.asarray(W, np.float32).T
        return y.astype(np.float64) + np.asarray(b, np.float64)
    if accum == "mx_step":
        return _linear_step_grid(x, W, b)
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64).T + np.asarray(b, np.float64)


def _linear_step_grid(x: np.ndarray, W: np.ndarray, b: np.ndarray, step: int = 64, bits: int = 16) -> np.ndarray:
    """Control-arm accumulation for the MXFP8 mode only: K in steps of 64; each
    step's products summed exactly, then rounded to the grid 2^(floor(log2 M) -
    bits), M the step's sum of |products|; the steps accumulated in float32.
    This is a second valid accumulation of the same exact products at the
    precision class of a matrix core that adds a step's 64 products on an
    aligned fixed-point grid (the op-level GPU test bounds the scaled fp8
    instruction's error by 2^-14 of that magnitude sum)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    acc = np.zeros((x.shape[0], W.shape[0]), np.float32)
    for k0 in range(0, x.shape[1], step):
        xs, ws = x[:, k0:k0 + step], W[:, k0:k0 + step]
        p = xs @ ws.T
        mag = np.abs(xs) @ np.abs(ws).T
        q = np.exp2(np.frexp(np.where(mag > 0, mag, 1.0))[1] - 1.0 - bits)
        acc = (acc + (np.rint(p / q) * q).astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64) + np.asarray(b, np.float64)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, rot: int) -> np.ndarray:
    """NeoX rotate_half RoPE on the first ``rot`` dims of each head.

    x: [n, H, hd]; cos, sin: [n, rot/2].  With x1 = x[:rot/2], x2 = x[rot/2:rot]:
    out1 = x1 cos - x2 sin, out2 = x2 cos + x1 sin.  Dims >= rot pass through
    (partial rotary).
    """
    half = rot // 2
    c = np.asarray(cos, np.float64)[:, None, :]
    s = np.asarray(sin, np.float64)[:, None, :]
    out = np.array(x, np.float64, copy=True)
    x1 = x[..., :half]
    x2 = x[..., half:rot]
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rot] = x2 * c + x1 * s
    return out


def _attn_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, chunk: int) -> np.ndarray:
    """softmax(q k^T * scale) v for one head of one document, queries in chunks."""
    o = np.empty_like(q)
    kt = np.ascontiguousarray(k.T)
    for i in range(0, q.shape[0], chunk):
        s = (q[i:i + chunk] @ kt) * scale
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[i:i + chunk] = p @ v
    return o


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: np.ndarray,
                     threads: int = 1, chunk: int = 2048) -> np.ndarray:
    """Non-causal packed attention: within each document, softmax(q k^T / sqrt(hd)) v.

    q, k, v: [N, H, hd].  No term crosses a document boundary; the softmax scale
    is 1/sqrt(head_dim) also under partial rotary (reading taken).  (Page "port
    the MiniMax-H3 omni-modal video+audio DiT", section "Correctness gates",
    the note that attention is a packed varlen non-causal block attention.)
    """
    N, H, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    o = np.empty((N, H, hd), np.float64)
    jobs = []
    for d in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[d]), int(cu_seqlens[d + 1])
        if b > a:
            for h in range(H):
                jobs.append((a, b, h))

    def run(job):
        a, b, h = job
        o[a:b, h] = _attn_one(q[a:b, h], k[a:b, h], v[a:b, h], scale, chunk)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return o


def attention_dense_masked(q, k, v, cu_seqlens):
    """Brute force: one dense N x N score matrix with a block-diagonal mask (tiny N only)."""
    N, H, hd = q.shape
    doc = np.empty(N, np.int64)
    for d in range(len(cu_seqlens) - 1):
        doc[cu_seqlens[d]:cu_seqlens[d + 1]] = d
    same = doc[:, None] == doc[None, :]
    o = np.zeros((N, H, hd))
    for h in range(H):
        s = q[:, h] @ k[:, h].T / math.sqrt(hd)
        s = np.where(same, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, h] = p @ v[:, h]
    return o


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def split_mlp(u: np.ndarray, mlp: str, F: int) -> np.ndarray:
    """Gated MLP activation from the merged projection, read in its original layout.

    'gate_up' ([gate | up], SwiGLU): silu(gate) * up.
    'value_gate' ([value | gate], the music model's merged ff projection):
    value * silu(gate).  (Page "the 2.4B fp32 DiT onto the device, staged once",
    sections "What moved" and "Correctness": the halves are swapped at stage
    time to feed silu(first) * second.)
    """
    a, b = u[:, :F], u[:, F:]
    if mlp == "gate_up":
        return silu(a) * b
    if mlp == "value_gate":
        return a * silu(b)
    raise ValueError(mlp)


def block_forward(cfg, x: np.ndarray, mod: np.ndarray, bw: Dict[str, np.ndarray], b: int,
                  layout: Dict[str, np.ndarray], cos: np.ndarray, sin: np.ndarray, mode: str,
                  threads: int = 1, trace: Optional[Dict[str, np.ndarray]] = None,
                  accum: str = "fp64") -> np.ndarray:
    """One DiT block on the packed residual stream x [N, D]; returns the new x.

    h  = norm(x) * (1 + scale_msa[c]) + shift_msa[c]          (bf16 store)
    qkv = h W_qkv^T + b, split [q_all | k_all | v_all]          (bf16 store)
    q, k = RoPE(q), RoPE(k); v unchanged                        (bf16 store)
    o  = varlen non-causal attention                            (bf16 store)
    x  = x + gate_msa[c] * (o W_o^T + b)                        (fp32 store)
    h2 = norm(x) * (1 + scale_mlp[c]) + shift_mlp[c]            (bf16 store)
    u  = h2 W_in^T + b                                          (bf16 store)
    m  = gated SiLU of u                                        (bf16 store)
    x  = x + gate_mlp[c] * (m W_2^T + b)                        (fp32 store)

    c = cond_idx of the token.  The storage points apply in 'bf16', 'mxfp8'
    and 'mxfp4' mode; in 'mxfp8' mode the four GEMMs run on MXFP8 re-quantized
    operands (``linear_mx8``), in 'mxfp4' mode on MXFP8 activations against
    MXFP4 weights (``linear_mx4``).  ``accum`` selects the GEMM accumulation (see
    ``linear``).
    Reading taken: the residual stream and both projection outputs feeding it
    stay fp32, because a bf16 rounding of those values alone moves a block's
    output by more than the bf16 tolerance.
    """
    D, H, hd, F = cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.ffn
    N = x.shape[0]
    ci = layout["cond_idx"]
    m_tok = mod[ci]  # [N, 6, D]
    p = f"blocks.{b}."
    W = lambda n: bw[p + n]  # noqa: E731
    gemm = linear_mx8 if mode == "mxfp8" else linear_mx4 if mode == "mxfp4" else linear
    lin = lambda a, w, bias: gemm(a, w, bias, accum)  # noqa: E731

    h = _store(modulate(norm(x, cfg.norm, cfg.norm_eps), m_tok[:, 0], m_tok[:, 1]), mode)
    qkv = _store(lin(h, W("attn.qkv.weight"), W("attn.qkv.bias")), mode)
    q = qkv[:, 0:D].reshape(N, H, hd)
    k = qkv[:, D:2 * D].reshape(N, H, hd)
    v = qkv[:, 2 * D:3 * D].reshape(N, H, hd)
    q = _store(apply_rope(q, cos, sin, cfg.rot_dim), mode)
    k = _store(apply_rope(k, cos, sin, cfg.rot_dim), mode)
    o = _store(attention_varlen(q, k, v, layout["cu_seqlens"], threads).reshape(N, D), mode)
    a = lin(o, W("attn.out.weight"), W("attn.out.bias"))
    x = _store_f32(x + m_tok[:, 2] * a, mode)
    if trace is not None:
        trace.update(h=h, qkv=qkv, q=q, k=k, v=v, o=o, a=a, x_mid=x)
    h2 = _store(modulate(norm(x, cfg.norm, cfg.norm_eps), m_tok[:, 3], m_tok[:, 4]), mode)
    u = _store(lin(h2, W("mlp.in.weight"), W("mlp.in.bias")), mode)
    mm = _store(split_mlp(u, cfg.mlp, F), mode)
    a2 = lin(mm, W("mlp.out.weight"), W("mlp.out.bias"))
    x = _store_f32(x + m_tok[:, 5] * a2, mode)
    if trace is not None:
        trace.update(h2=h2, u=u, m=mm, a2=a2, x_out=x)
    return x


# ----------------------------------------------------------------------------- ViT-style block variant
#
# The video VAE's decoder block (page "port the MiniMax-H3 omni-modal
# video+audio DiT", updates "video-VAE decoder block ported" and "video-VAE
# ViT3D decoder complete"), fp32 throughout:
#   h += scale1 * Attention(RMSNorm(h)),  h += scale2 * GatedSiLU_FF(RMSNorm(h))
# with affine RMSNorms, learned per-channel residual scales, a per-head RMS norm
# of q and k without affine weights, a fused qkv projection laid out per head
# ([head0 q | head0 k | head0 v | head1 q | ...]) and a 3-axis rotary
# embedding on length-normalized token coordinates.

def centered_rope_cache(grid, axis_dims, theta: float):
    """cos/sin [T*H*W, sum(axis_dims)/2] of a (t, h, w) token grid, raster order.

    Per axis a of extent n_a, token index i has the coordinate
    c = (2i + 1)/n_a - 1 (the centre of cell i of [-1, 1) split in n_a), and
    the angle of frequency j is (2 pi c) f_aj with f_aj = 1/theta^(2j/d_a),
    j < d_a/2; the axes' blocks are concatenated (t, h, w) and paired with
    rotate_half as in the integer-grid cache.  fp64, scalar libm, rounded to
    float32.  (Readings taken: the axes share the rotary width equally -- the
    caller passes d_a -- and the frequency spacing is the standard one.)
    """
    n_tok = 1
    for g in grid:
        n_tok *= g
    half = sum(axis_dims) // 2
    cos = np.empty((n_tok, half), np.float32)
    sin = np.empty((n_tok, half), np.float32)
    freqs = [rope_inv_freq(d, theta) for d in axis_dims]
    two_pi = 2.0 * math.pi
    row = 0
    for t in range(grid[0]):
        for h in range(grid[1]):
            for w in range(grid[2]):
                idx = (t, h, w)
                col = 0
                for a in range(3):
                    c = (2.0 * idx[a] + 1.0) / grid[a] - 1.0
                    for f in freqs[a]:
                        ang = (two_pi * c) * f
                        cos[row, col] = math.cos(ang)
                        sin[row, col] = math.sin(ang)
                        col += 1
                row += 1
    return cos, sin


def rms_affine(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with a per-channel weight: x / sqrt(mean(x^2) + eps) * g."""
    return norm(x, "rms", eps) * np.asarray(g, np.float64)


def vit_block_forward(x: np.ndarray, w: Dict[str, np.ndarray], n_heads: int, rot: int, eps: float,
                      cu_seqlens: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """One ViT-style decoder block on x [N, D] in fp64.

    w: 'norm1.weight' [D], 'attn.qkv.weight' [3D, D] + bias (rows per head:
    [q | k | v] of head 0, then head 1, ...), 'attn.out.weight' [D, D] + bias,
    'scale1' [D], 'norm2.weight' [D], 'ff.w1.weight' [2F, D] + bias ([gate |
    up], reading taken for the gated SiLU), 'ff.w2.weight' [D, F] + bias,
    'scale2' [D].  The q/k norm is an RMS norm over each head's dims with the
    block's eps and no weight; RoPE acts on the first ``rot`` dims of q and k.
    """
    N, D = x.shape
    hd = D // n_heads
    h = rms_affine(x, w["norm1.weight"], eps)
    qkv = linear(h, w["attn.qkv.weight"], w["attn.qkv.bias"]).reshape(N, n_heads, 3, hd)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    q = norm(q, "rms", eps)
    k = norm(k, "rms", eps)
    q = apply_rope(q, cos, sin, rot)
    k = apply_rope(k, cos, sin, rot)
    o = attention_varlen(q, k, v, cu_seqlens).reshape(N, D)
    x = x + np.asarray(w["scale1"], np.float64) * linear(o, w["attn.out.weight"], w["attn.out.bias"])
    h2 = rms_affine(x, w["norm2.weight"], eps)
    u = linear(h2, w["ff.w1.weight"], w["ff.w1.bias"])
    F = u.shape[1] // 2
    m = silu(u[:, :F]) * u[:, F:]
    return x + np.asarray(w["scale2"], np.float64) * linear(m, w["ff.w2.weight"], w["ff.w2.bias"])


# ----------------------------------------------------------------------------- patch islands

def patchify(latent: np.ndarray, mod) -> np.ndarray:
    """Latent -> tokens of one segment.

    'patch3d': [C, T pt, H ph, W pw] -> [T H W, pt ph pw C], tokens in raster
    (t, h, w) order, vector order (pt, ph, pw, c) with c fastest -- a
    convolution whose kernel equals its stride is a linear map of the flattened
    patch (page "port the MiniMax-H3 omni-modal video+audio DiT", update
    "Encoder complete").  'channel_major': [C, L] -> [L, C], the frame-major
    view under which a 1x1 convolution is a GEMM (page "the 2.4B fp32 DiT onto
    the device, staged once", section "What moved").
    """
    if mod.io == "patch3d":
        C, Tp, Hp, Wp = latent.shape
        pt, ph, pw = mod.patch
        T, Hh, Ww = Tp // pt, Hp // ph, Wp // pw
        z = latent.reshape(C, T, pt, Hh, ph, Ww, pw)
        z = z.transpose(1, 3, 5, 2, 4, 6, 0)
        return np.ascontiguousarray(z.reshape(T * Hh * Ww, pt * ph * pw * C))
    if mod.io == "channel_major":
        return np.ascontiguousarray(latent.T)
    raise ValueError(mod.io)


def unpatchify(tokens: np.ndarray, mod, grid) -> np.ndarray:
    """Inverse of ``patchify``."""
    if mod.io == "patch3d":
        T, Hh, Ww = grid
        pt, ph, pw = mod.patch
        C = mod.channels
        z = tokens.reshape(T, Hh, Ww, pt, ph, pw, C)
        z = z.transpose(6, 0, 3, 1, 4, 2, 5)
        return np.ascontiguousarray(z.reshape(C, T * pt, Hh * ph, Ww * pw))
    if mod.io == "channel_major":
        return np.ascontiguousarray(tokens.T)
    raise ValueError(mod.io)


# ----------------------------------------------------------------------------- whole forward

def forward(cfg, weights: Callable[[int], Dict[str, np.ndarray]], islands: Dict[str, np.ndarray],
            inp: Dict[str, np.ndarray], mode: Optional[str] = None,
            t_rows: Optional[Sequence[float]] = None, threads: int = 1,
            block_hook: Optional[Callable[[int, np.ndarray], None]] = None,
            accum: str = "fp64") -> Dict[str, np.ndarray]:
    """The DiT forward.

    ``weights(b)`` returns block b's tensors (regenerated block by block so a
    60 GB model never sits in host memory at once).  With in/out projections:
    per segment patchify -> fp32 in-projection -> scatter to its packed rows;
    the blocks; a final norm without modulation (reading taken: the pages name
    only the fp32 output heads) -> gather -> fp32 out-projection -> unpatchify.
    Without: tokens in, tokens out.  Returns {'latent.{i}' or 'x': array}.
    """
    gemm_fmt = getattr(cfg, "gemm", "stream")
    mode = mode or ("fp64" if cfg.stream != "bf16" else (gemm_fmt if gemm_fmt in ("mxfp8", "mxfp4") else "bf16"))
    layout = pack_layout(cfg)
    cos, sin = rope_cache(cfg)
    cu = layout["cu_seqlens"]
    if t_rows is None and cfg.cond_kind == "timestep":
        t_rows = [float(inp["t"][r.source]) for r in cfg.cond_rows]
    emb = cond_embeddings(cfg, t_rows, inp.get("cond"))

    if cfg.io:
        x = np.empty((cfg.n_tokens, cfg.hidden), np.float64)
        for i, s in enumerate(cfg.segments):
            m = s.modality
            tok = patchify(inp[f"latent.{i}"].astype(np.float64), cfg.modalities[m])
            x[cu[i]:cu[i + 1]] = linear(tok, islands[f"in.{m}.weight"], islands[f"in.{m}.bias"])
        x = _store_f32(x, mode)
    else:
        x = inp["x"].astype(np.float64)

    for b in range(cfg.n_blocks):
        bw = weights(b)
        mod = adaln_table(cfg, bw, b, emb, mode)
        x = block_forward(cfg, x, mod, bw, b, layout, cos, sin, mode, threads, accum=accum)
        if block_hook is not None:
            block_hook(b, x)
        del bw

    if not cfg.io:
        return {"x": x}
    y = _store_f32(norm(x, cfg.norm, cfg.norm_eps), mode)
    out = {}
    for i, s in enumerate(cfg.segments):
        m = s.modality
        v = linear(y[cu[i]:cu[i + 1]], islands[f"out.{m}.weight"], islands[f"out.{m}.bias"])
        out[f"latent.{i}"] = unpatchify(_store_f32(v, mode), cfg.modalities[m], s.grid)
    return out


# ----------------------------------------------------------------------------- denoise loop

def sigma_schedule(shift: float, n_steps: int) -> np.ndarray:
    """Rectified-flow time-shifted sigmas, fp64, n_steps + 1 values from 1 to 0.

    Reading taken (the pages name a time-shift schedule with shifts 12 and 3
    but print no formula): s_i = 1 - i/n, sigma_i = shift s_i / (1 + (shift-1) s_i).
    """
    out = np.empty(n_steps + 1, np.float64)
    for i in range(n_steps + 1):
        s = 1.0 - i / n_steps
        out[i] = shift * s / (1.0 + (shift - 1.0) * s)
    return out


def sigma_dt(sig: np.ndarray) -> np.ndarray:
    """Per-step dt = sigma_{i+1} - sigma_i, computed in fp64 and rounded to float32."""
    return np.array([np.float32(sig[i + 1] - sig[i]) for i in range(len(sig) - 1)], np.float32)


def euler_step(x: np.ndarray, v: np.ndarray, dt: np.float32) -> np.ndarray:
    """x + dt v in float32 without contraction: fl32(x + fl32(dt * v)).

    With eta = 0 the ancestral step injects no noise and steps to sigma_next;
    with x0 = x - sigma v (rf_v_to_x0) the update
    x' = (sigma'/sigma) x + (1 - sigma'/sigma) x0 equals x + (sigma' - sigma) v.
    """
    x = np.asarray(x, np.float32)
    v = np.asarray(v, np.float32)
    prod = (np.float32(dt) * v).astype(np.float32)
    return (x + prod).astype(np.float32)


def denoise_loop(cfg, weights, islands, latents: Dict[str, np.ndarray], n_steps: int,
                 mode: Optional[str] = None, threads: int = 1, accum: str = "fp64") -> Dict[str, np.ndarray]:
    """n_steps Euler steps from the given latents: at step i every row's
    timestep is sigma_m(i) of its modality and each segment moves by
    dt_m(i) * v (float32 state, as the loop keeps it)."""
    lat = {k: np.asarray(v, np.float32) for k, v in latents.items()}
    for i in range(n_steps):
        t_rows, dts = denoise_step_conditions(cfg, i)
        v = forward(cfg, weights, islands, lat, mode, t_rows=t_rows, threads=threads, accum=accum)
        for j, seg in enumerate(cfg.segments):
            lat[f"latent.{j}"] = euler_step(lat[f"latent.{j}"], v[f"latent.{j}"].astype(np.float32),
                                            dts[seg.modality])
    return lat


def denoise_step_conditions(cfg, step: int):
    """Per conditioning row: the fp32 timestep sigma_m(step) and the fp32 dt of its modality."""
    t_rows, dts = [], {}
    for m in range(cfg.n_mod):
        sig = sigma_schedule(cfg.shifts[m], cfg.denoise_steps)
        dts[m] = sigma_dt(sig)[step]
    for r in cfg.cond_rows:
        sig = sigma_schedule(cfg.shifts[r.modality], cfg.denoise_steps)
        t_rows.append(float(np.float32(sig[step])))
    return t_rows, dts


# ----------------------------------------------------------------------------- CFG denoise loop

def cfg_pairs(cfg) -> int:
    """Number P of guidance pairs in a packed batch of 2P segments.

    Reading taken (the pages give the branch count, not the packing): the
    first P segments are the conditional branches, segment j + P is the
    unconditional branch of segment j, with the same modality and grid, and
    both branches of a pair see the same latent.
    """
    n = len(cfg.segments)
    if n % 2:
        raise ValueError("a guided batch holds an even number of segments")
    P = n // 2
    for j in range(P):
        a, b = cfg.segments[j], cfg.segments[j + P]
        if a.modality != b.modality or tuple(a.grid) != tuple(b.grid):
            raise ValueError(f"segments {j} and {j + P} do not pair")
    return P


def cfg_combine(v_cond: np.ndarray, v_uncond: np.ndarray, w: float) -> np.ndarray:
    """Classifier-free guidance v = v_u + w (v_c - v_u), float32 operations in
    that order, each rounded (no contraction).

    Reading taken (the pages name the two branches but print no formula): the
    standard guidance form in which w = 0 is the unconditional velocity and
    w = 1 the conditional one.
    """
    vc = np.asarray(v_cond, np.float32)
    vu = np.asarray(v_uncond, np.float32)
    d = (vc - vu).astype(np.float32)
    return (vu + (np.float32(w) * d).astype(np.float32)).astype(np.float32)


def cfg_denoise_loop(cfg, weights, islands, latents: Dict[str, np.ndarray], cond_steps: np.ndarray,
                     dts: np.ndarray, w: float, n_steps: int, mode: Optional[str] = None,
                     threads: int = 1, accum: str = "fp64") -> Dict[str, np.ndarray]:
    """n_steps guided Euler steps of a vector-conditioned model.

    ``latents`` holds the P shared latents ('latent.{j}', j < P).  Step i runs
    one forward over all 2P segments -- segment j and j + P both read latent
    j, each with its own conditioning row taken from ``cond_steps[i]``
    ([n_sources, cond_dim]; the per-step rows carry whatever the sampler folds
    into them, the timestep included) -- combines each pair with
    ``cfg_combine`` and moves latent j by ``dts[i][modality]`` times the
    guided velocity (``euler_step``).
    """
    P = cfg_pairs(cfg)
    lat = {f"latent.{j}": np.asarray(latents[f"latent.{j}"], np.float32) for j in range(P)}
    for i in range(n_steps):
        inp = {f"latent.{j}": lat[f"latent.{j % P}"] for j in range(2 * P)}
        inp["cond"] = np.asarray(cond_steps[i])
        v = forward(cfg, weights, islands, inp, mode, threads=threads, accum=accum)
        for j in range(P):
            g = cfg_combine(v[f"latent.{j}"].astype(np.float32), v[f"latent.{j + P}"].astype(np.float32), w)
            lat[f"latent.{j}"] = euler_step(lat[f"latent.{j}"], g, np.float32(dts[i][cfg.segments[j].modality]))
    return lat
