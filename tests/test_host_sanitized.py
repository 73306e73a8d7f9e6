"""The library's host table builders (host_builders.cpp) rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer (plain g++, CPU only) and run
on every workload's layout and rope cache, on malformed segments, on the
timestep and sigma tables and on the int8 slicing of an fp32 weight with a
ragged K and a non-finite row.  Any sanitizer report fails the run; the
outputs must equal the shipped library's bit for bit."""

import ctypes
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import synthetic as S
from synthetic.configs import Segment

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_audio_gen_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("asan") / "host_builders_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "host_builders.cpp"), os.path.join(ROOT, "tests", "host_check", "host_builders_check.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_host_builders_under_sanitizers(checker, tmp_path):
    from video_audio_gen_amd import dit
    cases = [(S.get_config(n), None) for n in ("c1", "c2", "c3", "c4", "c5")]
    c1 = S.get_config("c1")
    cases += [(c1, [Segment(0, (4, 0, 4), 0)]),     # empty extent: rejected
              (c1, [Segment(2, (4, 4, 4), 0)]),     # no such modality: rejected
              (c1, [Segment(0, (1, 1, 1), 0)])]     # a one-token document
    rejected = {5, 6}
    req = bytearray(struct.pack("i", len(cases)))
    for cfg, segs in cases:
        segs = list(cfg.segments) if segs is None else segs
        req += bytes(dit.make_config(cfg))
        req += struct.pack("i", len(segs)) + bytes(dit.make_segments(segs))
    t = np.random.default_rng(0).random(5).astype(np.float32)
    req += struct.pack("i", len(t)) + t.tobytes() + struct.pack("i", 256)
    shifts = [1.0, 3.0, 12.0]
    req += struct.pack("i", len(shifts)) + np.asarray(shifts, np.float64).tobytes() + struct.pack("i", 50)
    R, K, bad_row = 37, 70, 20
    X = (np.random.default_rng(1).standard_normal((R, K)) * np.exp2(np.arange(R) % 9 - 4)[:, None]).astype(np.float32)
    X[bad_row, 11] = np.nan
    req += struct.pack("qq", R, K) + X.tobytes()
    rq, rs = tmp_path / "req.bin", tmp_path / "res.bin"
    rq.write_bytes(bytes(req))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([checker, str(rq), str(rs)], capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    buf = memoryview(rs.read_bytes())
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(buf, dtype, n, off)
        off += a.nbytes
        return a

    for i, (cfg, segs) in enumerate(cases):
        rc = int(take(np.int32, 1)[0])
        segs_ = list(cfg.segments) if segs is None else segs
        if i in rejected:
            assert dit.STATUS[rc] == "DIT_E_INVALID"
            continue
        assert rc == 0
        N = int(take(np.int32, 1)[0])
        lay = dit.dit_pack_layout(cfg, segs_)
        cos, sin = dit.dit_rope_cache_build(cfg, segs_)
        half = cfg.rot_dim // 2
        assert np.array_equal(take(np.int32, len(segs_) + 1), lay["cu_seqlens"])
        assert np.array_equal(take(np.int32, N), lay["cond_idx"])
        assert np.array_equal(take(np.int32, N), lay["doc_id"])
        assert np.array_equal(take(np.float32, N * half).view(np.uint32), cos.reshape(-1).view(np.uint32))
        assert np.array_equal(take(np.float32, N * half).view(np.uint32), sin.reshape(-1).view(np.uint32))
    emb = take(np.float32, len(t) * 256)
    assert np.array_equal(emb.view(np.uint32), dit.dit_timestep_embedding(t, 256).reshape(-1).view(np.uint32))
    for sh in shifts:
        sig, dt = dit.dit_sigma_schedule(sh, 50)
        assert np.array_equal(take(np.float64, 51), sig)
        assert np.array_equal(take(np.float32, 50), dt)
    Kp = (K + 31) // 32 * 32
    plane = R * Kp
    sl = take(np.int8, ((5 * plane + 255) & ~255) + 4 * R)
    assert int(take(np.int64, 1)[0]) == bad_row
    # rows before the non-finite one are complete: their digits and exponents
    # reconstruct each value to within 2^-35 of the row's scale
    E = sl[((5 * plane + 255) & ~255):].view(np.int32)
    digits = sl[:5 * plane].reshape(5, Kp // 32, R, 32).transpose(0, 2, 1, 3).reshape(5, R, Kp).astype(np.float64)
    w = np.exp2(-7.0 * (np.arange(5) + 1))[:, None, None]
    recon = (digits * w).sum(axis=0)[:, :K] * np.exp2(E.astype(np.float64))[:, None]
    for r in range(bad_row):
        scale = np.exp2(float(E[r]))
        assert np.abs(X[r].astype(np.float64)).max() < scale
        assert np.abs(recon[r] - X[r]).max() <= scale * 2.0 ** -35
    assert off == len(buf)
