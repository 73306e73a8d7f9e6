"""bench.py's algorithmic byte counts for the fp32 stream's row kernels (host
logic, no GPU): a GEMM result reaches the kernel after it as fp64 split-K
partials, 8 bytes per split and value, except for column groups of one split,
which the GEMM hands over finished as 4-byte floats."""

import bench
import synthetic as S


def _groups(table):
    return lambda n, k: table[(n, k)]


def test_silu_slice_bytes_count_one_split_columns_at_four_bytes():
    cfg = S.get_config("c2")
    N, D, F, L = cfg.n_tokens, cfg.hidden, cfg.ffn, cfg.n_blocks
    plan = {(3 * D, D): (2, 2, 3 * D), (D, D): (6, 6, D), (2 * F, D): (1, 4, 16384), (D, F): (6, 6, D)}
    w = bench.family_work(cfg, _groups(plan))
    # MLP-in result [N, 2F]: 16,384 finished columns, 4,096 columns of four partials; m sliced (5 bytes)
    part = N * (16384 * 4 + (2 * F - 16384) * 4 * 8)
    assert w["silu_slice"] == (L * (part + 5 * N * F), "byte")
    # QKV result: two partials everywhere; q, k, v written as fp32; cos/sin rows read
    assert w["rope_split"] == (L * (N * 3 * D * 2 * 8 + 3 * N * D * 4 + N * cfg.rot_dim * 4), "byte")


def test_all_one_split_plans_count_four_bytes_per_value():
    cfg = S.get_config("c2")
    N, D, F, L = cfg.n_tokens, cfg.hidden, cfg.ffn, cfg.n_blocks
    one = {(3 * D, D): (1, 1, 3 * D), (D, D): (1, 1, D), (2 * F, D): (1, 1, 2 * F), (D, F): (1, 1, D)}
    many = {k: (3, 3, v[2]) for k, v in one.items()}
    w1 = bench.family_work(cfg, _groups(one))
    w3 = bench.family_work(cfg, _groups(many))
    # the silu kernel's partial bytes: 4 per value with one split, 24 with three
    slices = L * 5 * N * F
    assert (w1["silu_slice"][0] - slices) * 6 == w3["silu_slice"][0] - slices
