"""CPU checks of the C ABI: the library loads and exports every declared symbol,
the host table builders equal the oracle bit for bit, and the host-side error
paths return the documented status codes (no GPU needed, no device call made).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import synthetic as S
from synthetic.configs import Segment, scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dit():
    from video_audio_gen_amd import dit as d
    d.load()
    return d


def test_exports_every_declared_symbol(dit):
    hdr = open(os.path.join(ROOT, "include", "dit.h")).read()
    names = set(re.findall(r"^\s*(?:int|void|size_t|const char\*)\s+(dit_\w+)\s*\(", hdr, re.M))
    assert len(names) >= 30
    lib = dit.load()
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_pack_layout_bit_exact(dit, name):
    cfg = S.get_config(name)
    got, ref = dit.dit_pack_layout(cfg), O.pack_layout(cfg)
    for k in ("cu_seqlens", "cond_idx", "doc_id"):
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_rope_cache_bit_exact(dit, name):
    cfg = S.get_config(name)
    c, s = dit.dit_rope_cache_build(cfg)
    oc, os_ = O.rope_cache(cfg)
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))


def test_timestep_embedding_and_sigma_bit_exact(dit):
    t = np.random.default_rng(0).random(7).astype(np.float32)
    for dim in (128, 256):
        got = dit.dit_timestep_embedding(t, dim)
        ref = np.stack([O.timestep_embedding(x, dim) for x in t])
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    for shift in (1.0, 3.0, 12.0):
        sig, dt = dit.dit_sigma_schedule(shift, 50)
        osig = O.sigma_schedule(shift, 50)
        assert np.array_equal(sig, osig)
        assert np.array_equal(dt, O.sigma_dt(osig))


def _fake_model(dit, cfg):
    c = dit.make_config(cfg)
    nbytes = ctypes.c_size_t()
    assert dit.load().dit_weight_bytes(ctypes.byref(c), ctypes.byref(nbytes)) == 0
    h = ctypes.c_void_p()
    fake = 1 << 40  # never dereferenced: only host-side validation runs in these tests
    assert dit.load().dit_model_create(ctypes.byref(c), fake, nbytes.value, ctypes.byref(h)) == 0
    return h, nbytes.value


def _stage_one(dit, h, name, arr, dtype=None):
    v = (dit.dit_weight_view * 1)()
    v[0].name = name.encode()
    v[0].dtype = dtype if dtype is not None else dit.DIT_F32
    v[0].ndim = arr.ndim
    for d in range(arr.ndim):
        v[0].shape[d] = arr.shape[d]
    v[0].host = arr.ctypes.data
    return dit.load().dit_stage_weights(h, v, 1, None)


def test_weight_bytes_match_the_contract(dit):
    cfg = S.get_config("c4")
    c = dit.make_config(cfg)
    nbytes = ctypes.c_size_t()
    assert dit.load().dit_weight_bytes(ctypes.byref(c), ctypes.byref(nbytes)) == 0
    D, F, dt = 6144, 16384, 256
    block = 2 * (4 * D * D + 3 * D * F) + 2 * (6 * D * dt * 2) + 4 * (3 * D + D + 2 * F + D + 2 * 6 * D)
    assert abs(nbytes.value - 64 * block) < 64 * 20 * 256 + 10 ** 7  # alignment + islands
    assert 60e9 < nbytes.value < 61.5e9  # ~30B parameters in bf16


def test_staging_errors_are_named(dit):
    cfg = S.get_config("c1")
    h, _ = _fake_model(dit, cfg)
    lib = dit.load()
    assert _stage_one(dit, h, "blocks.0.attn.nope.weight", np.zeros((4, 4), np.float32)) == 3
    assert b"blocks.0.attn.nope.weight" in lib.dit_last_error()
    assert _stage_one(dit, h, "blocks.0.attn.qkv.weight", np.zeros((128, 384), np.float32)) == 4
    assert _stage_one(dit, h, "blocks.0.attn.qkv.weight", np.zeros((384, 128), np.float32), dtype=7) == 5
    assert lib.dit_stage_finalize(h) == 6
    assert b"missing weight" in lib.dit_last_error()
    lib.dit_model_destroy(h)


def test_config_validation(dit):
    lib = dit.load()
    bad = [scaled(S.get_config("c1"), hidden=130), scaled(S.get_config("c1"), rot_dim=40),
           scaled(S.get_config("c3"), head_dim=64, n_heads=96),  # bf16 attention is head_dim 128 only
           scaled(S.get_config("c1"), norm_eps=0.0),
           scaled(S.get_config("c1"), ffn=24580),  # the fp32 stream's SiLU row kernel: ffn <= 24576
           scaled(S.get_config("c1"), ffn=514)]    # ffn a multiple of 4
    for cfg in bad:
        c = dit.make_config(cfg)
        n = ctypes.c_size_t()
        assert lib.dit_weight_bytes(ctypes.byref(c), ctypes.byref(n)) != 0
        assert len(lib.dit_last_error()) > 0


def test_layout_rejects_malformed_segments(dit):
    cfg = S.get_config("c1")
    with pytest.raises(dit.DitError) as e:
        dit.dit_pack_layout(cfg, [Segment(0, (4, 0, 4), 0)])
    assert e.value.status == "DIT_E_INVALID"
    with pytest.raises(dit.DitError):
        dit.dit_pack_layout(cfg, [Segment(3, (4, 4, 4), 0)])  # no modality 3
    with pytest.raises(dit.DitError, match="cond_row"):
        dit.dit_pack_layout(cfg, [Segment(0, (4, 4, 4), -1)])  # modulation row out of range


def test_forward_requires_finalized_model(dit):
    cfg = S.get_config("c1")
    h, _ = _fake_model(dit, cfg)
    lib = dit.load()
    rc = lib.dit_forward(h, None, 1, 1, 1, None, 0, None)
    assert rc == 1  # null batch is rejected before anything else
    rc = lib.dit_block_forward(None, 0, 1, 1, None, None, 0, None)
    assert rc == 1
    lib.dit_model_destroy(h)


def test_gemm_splits_query(dit):
    lib = dit.load()
    n = ctypes.c_int()
    # fp32 GEMM split count: a positive count for valid shapes, errors otherwise
    assert lib.dit_gemm_splits(dit.DIT_F32, 2560, 10240, ctypes.byref(n)) == 0 and n.value >= 1
    assert lib.dit_gemm_splits(dit.DIT_BF16, 2560, 10240, ctypes.byref(n)) == 1
    assert lib.dit_gemm_splits(dit.DIT_F32, 0, 10240, ctypes.byref(n)) == 1
    assert lib.dit_gemm_splits(dit.DIT_F32, 2560, 10240, None) == 1


@pytest.mark.parametrize("n,k", [(7680, 2560), (2560, 2560), (20480, 2560), (2560, 10240), (256, 256), (1000, 4000)])
def test_gemm_split_groups_query(dit, n, k):
    # the two column groups agree with the slot count: columns [0, col_split)
    # in s_lo splits, the rest in s_hi >= s_lo, and the slot count is the larger
    lo, hi, cb = dit.dit_gemm_split_groups(n, k)
    assert 1 <= lo <= hi and 0 < cb <= n and (cb == n or cb % 64 == 0)
    assert max(lo, hi) == dit.dit_gemm_splits(n, k)
    if cb == n:
        assert lo == hi


def test_gemm_split_groups_rejects_bad_arguments(dit):
    lib = dit.load()
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.dit_gemm_split_groups(dit.DIT_BF16, 2560, 2560, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 1
    assert lib.dit_gemm_split_groups(dit.DIT_F32, 0, 2560, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 1
    assert lib.dit_gemm_split_groups(dit.DIT_F32, 2560, 2560, None, ctypes.byref(b), ctypes.byref(c)) == 1


def test_nonfinite_fp32_gemm_weight_is_rejected_by_name(dit):
    # an fp32 GEMM weight is cut into int8 slices on the host; a NaN or an Inf
    # has no slicing and must fail the call (before any device copy), not
    # stage as finite digits
    cfg = S.get_config("c1")
    lib = dit.load()
    for bad in (np.nan, np.inf, -np.inf):
        h, _ = _fake_model(dit, cfg)
        w = np.zeros((384, 128), np.float32)
        w[77, 5] = bad
        assert _stage_one(dit, h, "blocks.0.attn.qkv.weight", w) == 1
        msg = lib.dit_last_error()
        assert b"blocks.0.attn.qkv.weight" in msg and b"row 77" in msg, msg
        lib.dit_model_destroy(h)


def test_batch_beyond_the_gemm_offsets_is_rejected_before_any_device_call(dit):
    # the music model's fp32 GEMMs address 5 bytes of slices per element of an
    # [N, 10240] operand in 32 bits: N = 50,000 tokens is beyond them
    cfg = S.get_config("c2")
    h, _ = _fake_model(dit, cfg)
    lib = dit.load()
    segs = dit.make_segments([Segment(0, (50000,), 0)])
    cond_mod = (ctypes.c_int * 1)(0)
    out = ctypes.c_void_p()
    fake_tables = 1 << 41  # never dereferenced: the check comes before the copy
    rc = lib.dit_batch_create(h, segs, 1, 1, cond_mod, fake_tables, 1 << 40, None, ctypes.byref(out))
    assert rc == 9, lib.dit_last_error()
    assert b"32-bit" in lib.dit_last_error()
    lib.dit_model_destroy(h)


def test_centered_rope_cache_bit_exact(dit):
    # the ViT decoder's centred 3-axis coordinates: the library's table equals
    # the oracle's, and a single segment equals the stand-alone definition
    cfg = S.get_config("vit")
    c, s = dit.dit_rope_cache_build(cfg)
    oc, os_ = O.rope_cache(cfg)
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    g = cfg.segments[0].grid
    cc, ss = O.centered_rope_cache(g, cfg.modalities[0].rope_axes, cfg.theta)
    n = cfg.segments[0].n_tokens
    assert np.array_equal(cc.view(np.uint32), c[:n].view(np.uint32))
    assert np.array_equal(ss.view(np.uint32), s[:n].view(np.uint32))


def test_vit_config_validation(dit):
    lib = dit.load()
    good = S.get_config("vit")
    c = dit.make_config(good)
    n = ctypes.c_size_t()
    assert lib.dit_weight_bytes(ctypes.byref(c), ctypes.byref(n)) == 0
    for bad in (scaled(good, stream="bf16"),          # the q/k norm runs in the fp32 stream only
                scaled(good, head_dim=48, n_heads=32, hidden=1536, rot_dim=48)):  # head lanes not a power of two
        c = dit.make_config(bad)
        assert lib.dit_weight_bytes(ctypes.byref(c), ctypes.byref(n)) != 0


def test_graph_and_mx4_calls_reject_bad_arguments_on_the_host(dit):
    """The captured-forward and MXFP4 calls refuse bad arguments by status
    before any device call: a null output handle or batch, a null graph, a K
    that is not a multiple of 32 for the MXFP4 quantizer, an MXFP4 model
    whose widths are not multiples of 128, or one with an fp32 stream."""
    lib = dit.load()
    cfg = S.get_config("c1")
    h, _ = _fake_model(dit, cfg)
    assert lib.dit_forward_graph_create(h, None, 1, 1, 1, None, 0, None) == 1       # null output handle
    out = ctypes.c_void_p()
    assert lib.dit_forward_graph_create(h, None, 1, 1, 1, None, 0, ctypes.byref(out)) == 1  # null batch
    assert out.value is None
    lib.dit_model_destroy(h)
    assert lib.dit_graph_launch(None, None) == 1
    n = ctypes.c_size_t()
    assert lib.dit_graph_nodes(None, ctypes.byref(n)) == 1
    lib.dit_graph_destroy(None)                                                         # no-op
    assert lib.dit_quantize_mx4(4, 48, 16, 16, 16, None) == 1                           # K % 32
    assert lib.dit_quantize_mx4(0, 64, None, None, None, None) == 0                     # nothing to do
    for bad in (scaled(S.get_config("c3_mxfp4"), ffn=16384 + 64),
                scaled(S.get_config("c1"), gemm="mxfp4")):
        c = dit.make_config(bad)
        nb = ctypes.c_size_t()
        assert lib.dit_weight_bytes(ctypes.byref(c), ctypes.byref(nb)) == 9  # DIT_E_UNSUPPORTED
        assert b"MX GEMMs" in lib.dit_last_error()
    # the weight contract of an MXFP4 model: half a byte per weight plus a scale byte per 32
    c = dit.make_config(S.get_config("c3_mxfp4"))
    c8 = dit.make_config(S.get_config("c3_mxfp8"))
    n4, n8 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.dit_weight_bytes(ctypes.byref(c), ctypes.byref(n4)) == 0
    assert lib.dit_weight_bytes(ctypes.byref(c8), ctypes.byref(n8)) == 0
    D, F = 6144, 16384
    per_block = 3 * D * D + D * D + 2 * F * D + D * F
    assert 0 < n8.value - n4.value and abs((n8.value - n4.value) - per_block / 2) < 1 << 20
