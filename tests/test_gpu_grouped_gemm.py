"""GPU parity of the grouped (mixture-of-experts) blockwise GEMM against the
oracle: each row uses its group's weight; empty groups, groups smaller than
a tile, rows past the last boundary (left untouched) and a malformed
boundary table (clamped, no access outside the operands)."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import gemm
from tests.gpu_util import check_gemm_output, host_f32, say

pytestmark = pytest.mark.gpu


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _case(gpu, G, M, N, K, ends, od, seed, sample=None):
    rng = np.random.default_rng(seed)
    a = _codes(rng, (M, K))
    b = np.stack([_codes(rng, (N, K)) for _ in range(G)])
    ra = rng.uniform(1e-3, 2e-3, (M, K // 128)).astype(np.float32)
    rb = rng.uniform(1e-3, 2e-3, (G, -(-N // 128), K // 128)).astype(np.float32)
    dt = torch.bfloat16 if od == "bf16" else torch.float32
    out = torch.full((M, N), float("nan"), dtype=dt, device=gpu)
    ra_d = torch.from_numpy(np.ascontiguousarray(ra.T)).to(gpu).t()
    # per-group column-major scale grids, groups side by side
    rb_d = torch.from_numpy(np.ascontiguousarray(rb.transpose(0, 2, 1))).to(gpu).transpose(1, 2)
    say("grouped gemm", G, M, N, K, od, list(ends)[:8])
    fp8.fp8_scaled_grouped_gemm_blockwise(
        torch.from_numpy(a).to(gpu), ra_d, torch.from_numpy(b).to(gpu), rb_d,
        torch.tensor(ends, dtype=torch.int32, device=gpu), out=out)
    torch.cuda.synchronize()
    got = host_f32(out)
    rows = np.arange(M) if sample is None else sample
    bounds = np.minimum(np.maximum.accumulate(np.clip(np.asarray(ends, np.int64), 0, M)), M)
    refs, bnds, keep = [], [], []
    for m in rows:
        g = int(np.searchsorted(bounds, m, side="right"))
        if g >= G:
            assert np.all(np.isnan(got[m])), f"row {m} past the last group was written"
            continue
        ref, S = gemm.blockwise_gemm(a[[m]], ra[[m]], b[g], rb[g], "128x128", with_bound=True)
        refs.append(ref)
        bnds.append(S)
        keep.append(m)
    # one check over all written rows (the Frobenius bar is a whole-output bar)
    check_gemm_output(got[keep], np.concatenate(refs), np.concatenate(bnds), K // 128, od,
                      f"grouped {G}x{M}x{N}x{K}")
    return got


def test_grouped_ragged_groups_and_unwritten_tail(gpu):
    _case(gpu, 4, 1024, 512, 1024, [300, 300, 700, 1000], "bf16", seed=50)


def test_grouped_single_group_equals_plain_gemm(gpu):
    rng = np.random.default_rng(51)
    M, N, K = 640, 384, 512
    got = _case(gpu, 1, M, N, K, [M], "f32", seed=51, sample=np.r_[0, 1, 255, 256, 639])
    assert np.isfinite(got).all()
    del rng


def test_grouped_narrow_n_uses_the_256x128_tiles(gpu):
    _case(gpu, 3, 520, 128, 768, [17, 260, 520], "f32", seed=52)


def test_grouped_moe_like_sampled(gpu):
    rng = np.random.default_rng(53)
    G, M, N, K = 16, 8192, 2048, 2048
    sizes = rng.multinomial(M, np.ones(G) / G)
    ends = np.cumsum(sizes)
    sample = np.unique(np.r_[ends[:-1] - 1, ends[:-1], 0, M - 1, rng.integers(0, M, 24)])
    _case(gpu, G, M, N, K, ends, "bf16", seed=53, sample=sample)


@pytest.mark.parametrize("mn", [(200, 384), (520, 64), (100, 96)])
def test_grouped_small_problems_use_the_small_tiles(gpu, mn):
    """Fewer rows than a 256-row tile, or fewer columns than 128: the
    small-tile kernel runs the groups (loads clamped to each group's rows),
    with an empty group and a group smaller than a tile."""
    M, N = mn
    ends = [M // 4, M // 4, M // 2 + 3, M]
    _case(gpu, 4, M, N, 512, ends, "f32", seed=56 + M)


@pytest.mark.parametrize("od", ["bf16", "f32"])
def test_grouped_last_tile_remainders(gpu, od):
    """Groups whose last 256-row tile holds 1, 63, 64, 65, 128, 129 or 255
    rows, or none: at most 128 rows go to the 64x64 second launch, more stay
    on the large tiles; groups smaller than a tile, and an empty group."""
    sizes = [256 + 1, 512 + 63, 64, 256 + 65, 128, 0, 256 + 129, 255, 512]
    ends = np.cumsum(sizes)
    _case(gpu, len(sizes), int(ends[-1]), 512, 256, list(ends), od, seed=57)


@pytest.mark.parametrize("od", ["bf16", "f32"])
def test_grouped_split_launch_when_it_saves_a_round(gpu, od):
    """16 whole 256-row tiles x 16 column tiles fill one round of 256 CUs;
    the groups' small last tiles (1, 64, 65, 128 and 10 rows) would need a
    second round, so they run in the 64-row second launch (on MI355X's 256
    CUs; with another count the same table may run in one launch, which the
    check covers as well).  Sampled rows: every group's first and last rows
    and random ones."""
    sizes = [4 * 256 + 1, 4 * 256 + 64, 0, 4 * 256 + 65, 10, 4 * 256 + 128]
    ends = np.cumsum(sizes)
    M = int(ends[-1])
    rng = np.random.default_rng(58)
    starts = np.r_[0, ends[:-1]]
    sample = np.unique(np.r_[starts[np.array(sizes) > 0], ends[np.array(sizes) > 0] - 1,
                             ends[np.array(sizes) > 0] - 2, rng.integers(0, M, 24)])
    _case(gpu, len(sizes), M, 4096, 256, list(ends), od, seed=58, sample=sample)


def test_grouped_many_groups_one_launch(gpu):
    """More groups than the two-launch split takes (80 > 64): every row in
    one large-tile launch, groups of 0 .. 120 rows."""
    rng = np.random.default_rng(59)
    sizes = rng.integers(0, 121, 80)
    ends = np.cumsum(sizes)
    M = int(ends[-1])
    sample = np.unique(np.r_[ends[sizes > 0] - 1, rng.integers(0, M, 40)])
    _case(gpu, 80, M, 512, 256, list(ends), "bf16", seed=59, sample=sample)


def test_grouped_malformed_table_is_clamped(gpu):
    """Decreasing ends and ends past M are clamped to [previous end, M]."""
    _case(gpu, 4, 512, 256, 256, [200, 100, 9999, 50], "f32", seed=54)


def test_grouped_benchmark_configuration_sampled(gpu):
    """The configuration the benchmark times: the 16640 tokens of the
    forward shape split over 8 experts with the same seeded multinomial
    sizes, N 5120, K 8192, bf16 out; sampled rows (every group's first and
    last row, and random ones) against the oracle."""
    G, M, N, K = 8, 16640, 5120, 8192
    sizes = np.random.default_rng(0).multinomial(M, np.ones(G) / G)
    ends = np.cumsum(sizes)
    rng = np.random.default_rng(55)
    starts = np.r_[0, ends[:-1]]
    sample = np.unique(np.r_[starts, ends - 1, rng.integers(0, M, 16)])
    _case(gpu, G, M, N, K, ends, "bf16", seed=55, sample=sample)


@pytest.mark.parametrize("od", ["bf16", "f32"])
def test_grouped_large_tiles_ragged_windows(gpu, od):
    """More than two rounds of 256x256 tiles on a group table whose groups
    end at every kind of offset inside a tile: a group's last tile loads a
    window that runs past the group's end (or, at the end of A, starts
    before the tile) and stores only its own rows; groups of 129-255
    leftover rows stay on the large tiles, an empty group, a first group
    whose last tile reaches into the next group.  Sampled rows: every
    group's first and last rows, the rows around each 256-row tile boundary
    inside a group, and random ones."""
    sizes = [3 * 256 + 200, 255, 129, 5 * 256 + 1, 0, 8 * 256 + 130, 2 * 256 + 250,
             4 * 256 + 64, 300]
    ends = np.cumsum(sizes)
    M = int(ends[-1])
    starts = np.r_[0, ends[:-1]]
    rng = np.random.default_rng(60)
    rows = [0, M - 1]
    for s0, n in zip(starts, sizes):
        if n == 0:
            continue
        rows += [s0, s0 + n - 1]
        for t in range(256, n, 256):
            rows += [s0 + t - 1, s0 + t]
    sample = np.unique(np.r_[rows, rng.integers(0, M, 40)])
    _case(gpu, len(sizes), M, 4096, 256, list(ends), od, seed=60, sample=sample)
