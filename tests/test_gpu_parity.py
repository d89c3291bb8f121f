"""GPU parity: the HIP library against the CPU oracle, element by element.

Runs through the binding (and so through the C ABI).  Integer-grid workloads
must match bit for bit; Gaussian ones within the stated tolerance (see
gpu_util).  Full-size workloads run in the launch configuration the benchmark
times and are compared on sampled rows, which the oracle computes one by one.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_scores_close, assert_topk_match, dev_problem, gpu_score, gpu_select, to_np)
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_problem

import sparse_attention_indexer_csa_amd as csa

pytestmark = pytest.mark.gpu

PLANS = ["row_tiles", "split_rows"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()
    oracle.build(force=False)


def _check_full(P, plan, exact, with_scores=True):
    s_o, i_o = oracle.select(P)
    idx, sc = gpu_select(P, plan=plan, return_scores=True)
    sc2 = gpu_score(P, plan=plan)
    idx_only = gpu_select(P, plan=plan)
    assert_scores_close(to_np(sc).reshape(P.rows, P.W), s_o, exact=exact, what=f"{P.name} select scores")
    assert_scores_close(to_np(sc2).reshape(P.rows, P.W), s_o, exact=exact, what=f"{P.name} score")
    assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=exact, what=f"{P.name} select")
    # the fused selection without a score output is the same selection
    np.testing.assert_array_equal(to_np(idx_only), to_np(idx))
    return s_o, i_o


# --- the named workloads -------------------------------------------------------------

@pytest.mark.parametrize("plan", PLANS)
def test_tiny_integer_grid_exact(plan):
    _check_full(make_config("c1"), plan, exact=True)


def test_mid_integer_grid_exact():
    _check_full(make_config("c2int"), "auto", exact=True)


def test_mid_gaussian_tolerance():
    _check_full(make_config("c2"), "auto", exact=False)


def _sample_rows(S, B=1, extra=()):
    rows = set()
    for b in range(B):
        for i in list(range(0, 8)) + list(range(2040, 2060)) + list(np.linspace(0, S - 1, 24).astype(int)) + \
                [S - 2, S - 1] + list(extra):
            if 0 <= i < S:
                rows.add(b * S + int(i))
    return np.array(sorted(rows), dtype=np.int64)


def test_long_prefill_full_size_sampled():
    """seq-16384 prefill in the benchmark's launch configuration: fused select
    (no score output) and the scores-only call, checked on sampled rows."""
    P = make_config("c3")
    d = dev_problem(P)
    idx = to_np(gpu_select(P, dev=d)).reshape(P.rows, -1)
    sc = to_np(gpu_score(P, dev=d)).reshape(P.rows, P.W)
    rows = _sample_rows(P.S)
    s_o, i_o = oracle.select(P, rows)
    assert_scores_close(sc[rows], s_o, what="c3 score")
    assert_topk_match(idx[rows], i_o, s_o, what="c3 select")
    # every row: count of selected = min(k, visible), no -1 before the end
    nvis = np.minimum((np.arange(P.S) + 1) // P.m, P.W)
    cnt = (idx >= 0).sum(axis=1)
    np.testing.assert_array_equal(cnt, np.minimum(nvis, P.top_k))


@pytest.mark.parametrize("name", ["c4", "c4aligned"])
def test_packed_segments_full_size_sampled(name):
    P = make_config(name)
    d = dev_problem(P)
    idx = to_np(gpu_select(P, dev=d)).reshape(P.rows, -1)
    sc = to_np(gpu_score(P, dev=d)).reshape(P.rows, P.W)
    rows = _sample_rows(P.S, P.B, extra=np.where(np.diff(P.q_seg[0]) != 0)[0].tolist())
    s_o, i_o = oracle.select(P, rows)
    assert_scores_close(sc[rows], s_o, what=f"{name} score")
    assert_topk_match(idx[rows], i_o, s_o, what=f"{name} select")


def test_decode_full():
    """B=64 decode rows over a 32768-entry cache, all rows checked."""
    P = make_config("c5")
    d = dev_problem(P)
    assert csa.resolve_plan(d["q"], d["k"], d["w"], P.m) == "split_rows"
    s_o, i_o = oracle.select(P)
    idx = to_np(gpu_select(P, dev=d)).reshape(P.rows, -1)
    idx2, sc = gpu_select(P, dev=d, return_scores=True)
    assert_scores_close(to_np(sc).reshape(P.rows, P.W), s_o, what="c5 scores")
    assert_topk_match(idx, i_o, s_o, what="c5 select")
    np.testing.assert_array_equal(to_np(idx2).reshape(P.rows, -1), idx)
    # the row-tile plan computes the very same bits
    idx_rt = to_np(gpu_select(P, plan="row_tiles", dev=d)).reshape(P.rows, -1)
    np.testing.assert_array_equal(idx_rt, idx)


# --- selection given scores, and fused == two-pass ----------------------------------------

def test_topk_exact_on_oracle_scores():
    """The top-k kernel is exact on any fp32 input: on the oracle's own scores
    it reproduces the oracle's selection bit for bit (ties, -0, -inf, NaN)."""
    P = make_config("c2")
    s_o, i_o = oracle.select(P)
    got = to_np(csa.topk(torch.from_numpy(s_o).cuda(), P.top_k))
    np.testing.assert_array_equal(got, i_o)
    rng = np.random.default_rng(3)
    s = rng.choice(np.array([-2.0, -0.0, 0.0, 0.5, 0.5, 1.0, 3.0], np.float32), size=(300, 1500))
    s[rng.random(s.shape) < 0.2] = -np.inf
    s[rng.random(s.shape) < 0.01] = np.nan
    s[5] = -np.inf
    for k in (1, 7, 64, 512, 700, 2048):
        np.testing.assert_array_equal(to_np(csa.topk(torch.from_numpy(s).cuda(), k)), oracle.topk(s, k), err_msg=f"k={k}")


@pytest.mark.parametrize("dist", ["ties", "one_bucket", "gauss"])
def test_topk_long_rows_exact(dist):
    """Long rows (the workgroup-per-row kernel with its coarse-histogram
    prefilter) stay exact: heavy ties, scores that all share one coarse bucket
    (the prefilter cannot narrow them down, so more than 2048 candidates send
    the row down the streaming path), -inf/NaN holes, odd lengths."""
    rng = np.random.default_rng(11)
    W = 20000
    if dist == "ties":
        s = rng.integers(-3, 4, size=(9, W)).astype(np.float32)
    elif dist == "one_bucket":
        s = (1.0 + rng.random((9, W)) * 2.0 ** -10).astype(np.float32)
    else:
        s = rng.standard_normal((9, W)).astype(np.float32)
    s[rng.random(s.shape) < 0.1] = -np.inf
    s[rng.random(s.shape) < 0.01] = np.nan
    s[1, :] = -np.inf
    s[2, 100:] = -np.inf          # fewer valid entries than k
    s[3, :] = 0.0                 # all ties
    s[3, ::7] = -0.0
    # k not a multiple of 64 as well; 1200 and 1700 leave between 1025 and
    # 2048 candidates on Gaussian rows (the widest in-LDS sort)
    for k in (1, 100, 300, 512, 1200, 1700, 2048):
        np.testing.assert_array_equal(to_np(csa.topk(torch.from_numpy(s).cuda(), k)), oracle.topk(s, k),
                                      err_msg=f"{dist} k={k}")
    # a row length that is not a multiple of 4 or of 64
    s2 = np.ascontiguousarray(s[:, :W - 37])
    np.testing.assert_array_equal(to_np(csa.topk(torch.from_numpy(s2).cuda(), 512)), oracle.topk(s2, 512),
                                  err_msg=f"{dist} ragged")
    # lengths that leave each thread of the in-LDS path 4-5, 8-9 and 15-16
    # blocks of four keys
    for w2 in (9001, 16390, 31000):
        s3 = np.ascontiguousarray(np.concatenate([s, s], axis=1)[:, :w2])
        np.testing.assert_array_equal(to_np(csa.topk(torch.from_numpy(s3).cuda(), 300)), oracle.topk(s3, 300),
                                      err_msg=f"{dist} W={w2}")


def test_topk_large_k_two_pass():
    """k whose streaming fallback does not fit one workgroup's LDS: the
    in-LDS path takes the rows it can, marks the others, and one wave per row
    selects those (tied rows); rows packed into one coarse bucket go through
    the split of that bucket by the next key bits."""
    rng = np.random.default_rng(17)
    W = 32768
    s = rng.standard_normal((7, W)).astype(np.float32)
    s[1] = rng.integers(-2, 3, size=W).astype(np.float32)      # ties: handed over
    s[2] = (1.0 + rng.random(W) * 2.0 ** -10).astype(np.float32)  # one coarse bucket
    s[3, 5000:] = -np.inf
    s[4, :] = -np.inf                                          # nothing selectable
    s[5, ::3] = np.nan
    for k in (512, 1700, 1920, 1921):
        np.testing.assert_array_equal(to_np(csa.topk(torch.from_numpy(s).cuda(), k)), oracle.topk(s, k),
                                      err_msg=f"k={k}")


@pytest.mark.parametrize("name,plan", [("c2", "auto"), ("c4", "auto"), ("c5", "auto"), ("c5", "row_tiles")])
def test_fused_select_equals_topk_of_scores(name, plan):
    P = make_config(name)
    d = dev_problem(P)
    sc = gpu_score(P, plan=plan, dev=d)
    two_pass = to_np(csa.topk(sc, P.top_k))
    fused = to_np(gpu_select(P, plan=plan, dev=d))
    np.testing.assert_array_equal(fused, two_pass)


# --- invariants on the GPU -------------------------------------------------------------------

@pytest.mark.parametrize("dist", ["int", "gauss"])
def test_decode_row_equals_last_prefill_row(dist):
    S, H, D, W, m, k = 1024, 64, 128, 256, 4, 64
    P = make_problem(3, S, H, D, W, m, k, dist=dist, seed=31)
    idx, sc = gpu_select(P, return_scores=True)
    Q = make_problem(3, 1, H, D, W, m, k, dist=dist, seed=31)
    Q.q = np.ascontiguousarray(P.q[:, :, S - 1:S])
    Q.w = np.ascontiguousarray(P.w[:, S - 1:S])
    Q.k = P.k.copy()
    Q.q_offset = np.full(3, S - 1, np.int32)
    for plan in PLANS:
        idx1, sc1 = gpu_select(Q, plan=plan, return_scores=True)
        np.testing.assert_array_equal(to_np(sc1)[:, 0], to_np(sc)[:, S - 1])
        np.testing.assert_array_equal(to_np(idx1)[:, 0], to_np(idx)[:, S - 1])


def test_future_keys_are_never_read():
    """Keys past a row's visible prefix are poisoned; the outputs of rows that
    cannot see them do not change (bitwise)."""
    P = make_config("c2")
    d = dev_problem(P)
    idx, sc = gpu_select(P, dev=d, return_scores=True)
    J0 = 600
    kk = bf16_bits_to_f32(P.k).copy()
    kk[0, J0:] = 30.0
    d2 = dict(d)
    d2["k"] = torch.from_numpy(f32_to_bf16_bits(kk).view(np.int16)).view(torch.bfloat16).cuda()
    idx2, sc2 = gpu_select(P, dev=d2, return_scores=True)
    rows = np.where(np.minimum((np.arange(P.S) + 1) // P.m, P.W) <= J0)[0]
    np.testing.assert_array_equal(to_np(sc2)[0, rows], to_np(sc)[0, rows])
    np.testing.assert_array_equal(to_np(idx2)[0, rows], to_np(idx)[0, rows])


def test_deterministic():
    P = make_config("c2")
    d = dev_problem(P)
    a1, s1 = gpu_select(P, dev=d, return_scores=True)
    a2, s2 = gpu_select(P, dev=d, return_scores=True)
    np.testing.assert_array_equal(to_np(a1), to_np(a2))
    assert np.array_equal(to_np(s1).view(np.uint32), to_np(s2).view(np.uint32))


def test_power_of_two_scale_is_exact():
    P = make_problem(1, 512, 64, 128, 128, 4, 32, dist="gauss", seed=41)
    _, s1 = gpu_select(P, return_scores=True)
    P.scale = 0.25
    i2, s2 = gpu_select(P, return_scores=True)
    a, b = to_np(s1), to_np(s2)
    fin = np.isfinite(a)
    np.testing.assert_array_equal(b[fin], a[fin] * np.float32(0.25))
    s_o, i_o = oracle.select(P)
    assert_topk_match(to_np(i2).reshape(P.rows, -1), i_o, s_o, what="scaled")


# --- layouts and edge shapes (integer grid: bitwise) --------------------------------------

EDGE = [
    # (B, S, H, D, W, m, top_k, q_offset)
    (1, 13, 4, 32, 8, 4, 3, None),          # ragged rows, short
    (2, 77, 1, 32, 19, 4, 5, None),         # one head
    (1, 200, 20, 64, 50, 4, 16, None),      # heads not a multiple of 16
    (1, 130, 100, 128, 40, 3, 7, None),     # 100 heads, compress rate 3
    (1, 96, 128, 128, 24, 4, 8, None),      # 128 heads
    (2, 150, 8, 128, 150, 1, 33, None),     # compress rate 1 (W = S)
    (1, 64, 16, 32, 16, 4, 1, None),        # top_k = 1
    (1, 64, 16, 32, 16, 4, 40, None),       # top_k > W
    (2, 40, 16, 64, 300, 4, 20, [-9, 2000]),  # offsets: before the start / past the cache
    (1, 9, 16, 128, 4096, 2, 2048, [6000]),  # top_k = 2048, buffer compactions
    (3, 5, 16, 32, 0, 4, 4, None),          # empty cache
]


@pytest.mark.parametrize("case", EDGE, ids=[str(c[:7]) for c in EDGE])
@pytest.mark.parametrize("plan", PLANS)
def test_edge_shapes_exact(case, plan):
    B, S, H, D, W, m, k, off = case
    P = make_problem(B, S, H, D, W, m, k, dist="int", seed=sum(case[:7]),
                     q_offset=None if off is None else np.array(off, np.int32))
    s_o, i_o = oracle.select(P)
    idx, sc = gpu_select(P, plan=plan, return_scores=True)
    assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=True, what=str(case))
    # without a score output the split plan takes its balanced kernel
    assert_topk_match(to_np(gpu_select(P, plan=plan)).reshape(P.rows, -1), i_o, s_o, exact=True,
                      what=f"{case} select only")
    if W > 0:
        assert_scores_close(to_np(sc).reshape(P.rows, W), s_o, exact=True, what=str(case))
        assert_scores_close(to_np(gpu_score(P, plan=plan)).reshape(P.rows, W), s_o, exact=True, what=str(case))


@pytest.mark.parametrize("W,plans", [(65536, ("row_tiles", "split_rows")), (65537, ("auto",))])
def test_widest_row_tile_cache(W, plans):
    """The row-tile plan keeps entry numbers in 16 bits: W = 65536 is its
    widest cache (the last entry is 65535); one more entry goes to the split
    plan, and forcing the row-tile plan there is refused."""
    P = make_problem(1, 3, 16, 32, W, 1, 2048, dist="int", seed=W, q_offset=np.array([W + 5], np.int32))
    # the last entry duplicates row 0's best one, so it is selected
    best = int(oracle.select(P)[1][0, 0])
    P.k[0, W - 1] = P.k[0, best]
    s_o, i_o = oracle.select(P)
    assert (i_o[0] == W - 1).any()
    for plan in plans:
        idx = gpu_select(P, plan=plan)
        assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=True, what=f"W={W} {plan}")
    if W > 65536:
        with pytest.raises(csa.CsaUnsupportedError):
            gpu_select(P, plan="row_tiles")


@pytest.mark.parametrize("plan", PLANS)
def test_chunked_prefill_equals_unchunked(plan):
    """Chunked prefill through q_offset (each chunk of query rows passes its
    absolute start position and the whole compressed cache) selects exactly
    what the unchunked call selects for those rows, on Gaussian inputs: the
    score of a pair does not depend on how the rows were batched."""
    P = make_problem(2, 768, 64, 128, 192, 4, 64, dist="gauss", seed=31)
    full = to_np(gpu_select(P, plan=plan)).reshape(P.B, P.S, -1)
    for c0, c1 in ((0, 256), (256, 320), (320, 767), (767, 768)):
        Pc = dataclasses.replace(P, S=c1 - c0, q=np.ascontiguousarray(P.q[:, :, c0:c1]),
                                 w=np.ascontiguousarray(P.w[:, c0:c1]),
                                 q_offset=np.full(P.B, c0, np.int32))
        got = to_np(gpu_select(Pc, plan=plan)).reshape(P.B, c1 - c0, -1)
        np.testing.assert_array_equal(got, full[:, c0:c1], err_msg=f"rows {c0}:{c1}")


@pytest.mark.parametrize("dist", ["int", "gauss"])
def test_compress_rate_one(dist):
    """compress_rate = 1 (one compressed entry per token, W = S: the
    uncompressed indexer): every plan against the oracle."""
    P = make_problem(1, 1536, 64, 128, 1536, 1, 512, dist=dist, seed=41)
    s_o, i_o = oracle.select(P)
    for plan in PLANS:
        idx, sc = gpu_select(P, plan=plan, return_scores=True)
        assert_scores_close(to_np(sc).reshape(P.rows, P.W), s_o, exact=dist == "int", what=f"{dist} {plan}")
        assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=dist == "int", what=f"{dist} {plan}")


def test_empty_batch_and_rows():
    for B, S in ((0, 10), (2, 0)):
        P = make_problem(B, S, 4, 32, 8, 4, 3, dist="int", seed=1)
        idx = gpu_select(P)
        assert tuple(idx.shape) == (B, S, 3)


def test_segments_exact_integer_grid():
    P = make_problem(3, 300, 16, 64, 75, 4, 12, dist="int", seed=5, segments="random")
    for plan in PLANS:
        s_o, i_o = oracle.select(P)
        idx, sc = gpu_select(P, plan=plan, return_scores=True)
        assert_scores_close(to_np(sc).reshape(P.rows, P.W), s_o, exact=True, what=f"segments {plan}")
        assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=True, what=f"segments {plan}")


def test_sequence_major_q_and_padded_k_rows():
    """q given as a permuted [B,S,H,D] tensor and k with a row pitch wider
    than D give the same bits as dense head-major inputs."""
    P = make_problem(2, 96, 16, 64, 24, 4, 6, dist="gauss", seed=8)
    d = dev_problem(P)
    ref_i, ref_s = gpu_select(P, dev=d, return_scores=True)
    d2 = dev_problem(P, layout="seq_major")
    assert d2["q"].stride(1) == P.D and d2["q"].stride(2) == P.H * P.D
    kb = torch.zeros(P.B, P.W, P.D + 8, dtype=torch.bfloat16, device="cuda")
    kb[:, :, :P.D] = d["k"]
    d2["k"] = kb[:, :, :P.D]
    i2, s2 = gpu_select(P, dev=d2, return_scores=True)
    np.testing.assert_array_equal(to_np(i2), to_np(ref_i))
    assert np.array_equal(to_np(s2).view(np.uint32), to_np(ref_s).view(np.uint32))
    # every kernel takes the strides: row tiles, and the split plan's
    # chunked (with scores) and balanced (selection only) kernels
    for plan in ("row_tiles", "split_rows"):
        np.testing.assert_array_equal(to_np(gpu_select(P, dev=d2, plan=plan)), to_np(ref_i))
        i3, s3 = gpu_select(P, dev=d2, plan=plan, return_scores=True)
        np.testing.assert_array_equal(to_np(i3), to_np(ref_i))
        assert np.array_equal(to_np(s3).view(np.uint32), to_np(ref_s).view(np.uint32))


BALANCED = [
    # B, S, H, D, W, m, top_k, lengths lo..hi, segments
    (256, 1, 64, 128, 4096, 4, 512, (0, 4096), None),    # most rows the balanced split takes, empty rows among them
    (37, 1, 32, 64, 2500, 4, 100, (1, 2500), None),      # ragged tails, one head block
    (5, 40, 16, 32, 3000, 2, 64, None, "random"),        # several rows per sequence, segments
    (3, 1, 128, 128, 9000, 4, 2048, (8000, 9000), None), # four head blocks, top_k = 2048
]


@pytest.mark.parametrize("case", BALANCED, ids=[str(c[:7]) for c in BALANCED])
def test_balanced_split_exact(case):
    """The split plan without a score output divides the rows' visible
    entries evenly over the waves (ranges cross row ends); every selection
    equals the oracle's on the integer grid, and equals the chunked kernel's
    (the select with a score output) bit for bit."""
    B, S, H, D, W, m, k, lens, segs = case
    P = make_problem(B, S, H, D, W, m, k, dist="int", seed=sum(case[:7]), decode_lengths=lens,
                     segments=segs)
    d = dev_problem(P)
    s_o, i_o = oracle.select(P)
    idx = to_np(gpu_select(P, plan="split_rows", dev=d)).reshape(P.rows, -1)
    assert_topk_match(idx, i_o, s_o, exact=True, what=f"{case}")
    idx2, _ = gpu_select(P, plan="split_rows", dev=d, return_scores=True)
    np.testing.assert_array_equal(to_np(idx2).reshape(P.rows, -1), idx)


# --- key strides below the row width, one-entry caches ----------------------------------------

@pytest.mark.parametrize("plan", PLANS)
def test_one_entry_cache_exact(plan):
    """W = 1: the binding passes the stride of a size-1 dimension as 0, so the
    key tile covers a single 2*D-byte entry; scores and selections equal the
    oracle's bit for bit."""
    for B, S, H, D in ((2, 9, 16, 32), (1, 40, 64, 128)):
        P = make_problem(B, S, H, D, 1, 1, 3, dist="int", seed=B * S + H)
        s_o, i_o = oracle.select(P)
        idx, sc = gpu_select(P, plan=plan, return_scores=True)
        assert_scores_close(to_np(sc).reshape(P.rows, 1), s_o, exact=True, what=f"W=1 {plan}")
        assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=True, what=f"W=1 {plan}")
        assert_scores_close(to_np(gpu_score(P, plan=plan)).reshape(P.rows, 1), s_o, exact=True, what="W=1 score")
        assert_topk_match(to_np(gpu_select(P, plan=plan)).reshape(P.rows, -1), i_o, s_o, exact=True,
                          what=f"W=1 {plan} select only")


@pytest.mark.parametrize("plan", PLANS)
def test_overlapping_key_rows_exact(plan):
    """Entry j of k read at j * k_sw with k_sw (8 or 0 elements) below D: the
    entries overlap in memory.  The oracle gets the same entries written out
    densely; every kernel must read exactly those bytes."""
    B, S, H, D, W, m, k = 2, 64, 16, 32, 24, 2, 6
    for k_sw in (8, 0):
        P = make_problem(B, S, H, D, W, m, k, dist="int", seed=70 + k_sw)
        flat = P.k.reshape(B, -1)[:, :(W - 1) * k_sw + D]
        P.k = np.ascontiguousarray(np.stack([np.stack([flat[b, j * k_sw:j * k_sw + D] for j in range(W)])
                                             for b in range(B)]))
        s_o, i_o = oracle.select(P)
        d = dev_problem(P)
        base = torch.from_numpy(np.ascontiguousarray(flat).view(np.int16)).view(torch.bfloat16).cuda()
        d["k"] = torch.as_strided(base, (B, W, D), (base.stride(0), k_sw, 1))
        idx, sc = gpu_select(P, plan=plan, dev=d, return_scores=True)
        assert_scores_close(to_np(sc).reshape(P.rows, W), s_o, exact=True, what=f"k_sw={k_sw} {plan}")
        assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=True, what=f"k_sw={k_sw} {plan}")
        assert_topk_match(to_np(gpu_select(P, plan=plan, dev=d)).reshape(P.rows, -1), i_o, s_o, exact=True,
                          what=f"k_sw={k_sw} {plan} select only")


def test_short_segment_ids_refused():
    P = make_problem(1, 64, 16, 32, 16, 4, 4, dist="int", seed=3, segments="random")
    d = dev_problem(P)
    d["k_seg"] = d["k_seg"][:, :-1].contiguous()
    with pytest.raises(ValueError, match="k_seg"):
        gpu_select(P, dev=d)


def test_sort_of_full_buffer_with_lowest_bucket_last():
    """A row with exactly 512 selectable entries and k = 512 is sorted by the
    32-bit composite sort with nine position bits.  Its last entry holds a key
    in the lowest truncated bucket, just above the smallest key: its composite
    is 0 and the truncation check must still compare it with its neighbour,
    so the output order is exact."""
    s = (100.0 + np.arange(512)).astype(np.float32)
    s[0] = 1.0
    s[511] = np.float32(1.0) + np.float32(3 * 2.0 ** -23)
    rows = np.stack([s, s[::-1].copy()])
    want = oracle.topk(rows, 512)
    assert want[0, -2] == 511 and want[0, -1] == 0
    np.testing.assert_array_equal(to_np(csa.topk(torch.from_numpy(rows).cuda(), 512)), want)


# --- scales other than 1, compared element-wise with the oracle --------------------------------

@pytest.mark.parametrize("scale", [0.08838835, -1.0, 3.7])
@pytest.mark.parametrize("plan", PLANS)
def test_scale_elementwise(scale, plan):
    """The scale is one fp32 multiply after the head sum: on the integer grid
    the unscaled sum is exact, so the oracle's scaled scores (1/sqrt(128),
    -1, 3.7) and selections are matched bit for bit; on Gaussian inputs
    within the tolerance."""
    for dist in ("int", "gauss"):
        P = make_problem(2, 300, 64, 128, 75, 4, 24, dist=dist, seed=57, scale=scale)
        s_o, i_o = oracle.select(P)
        idx, sc = gpu_select(P, plan=plan, return_scores=True)
        exact = dist == "int"
        assert_scores_close(to_np(sc).reshape(P.rows, P.W), s_o, exact=exact, what=f"{dist} scale={scale}")
        assert_topk_match(to_np(idx).reshape(P.rows, -1), i_o, s_o, exact=exact, what=f"{dist} scale={scale}")
        assert_topk_match(to_np(gpu_select(P, plan=plan)).reshape(P.rows, -1), i_o, s_o, exact=exact,
                          what=f"{dist} scale={scale} select only")


def test_long_prefill_integer_grid_sampled():
    """The seq-16384 prefill shape (S=16384, H=64, D=128, W=4096, k=512) on the
    integer grid (seed 33), in the benchmark's launch configuration (fused
    select without a score output).  Rows past 6144 see more than the 1536
    pairs the row kernel's buffer holds, so its mid-stream compactions run,
    here under heavy ties: 72 sampled rows must equal the oracle bit for bit,
    scores (from the score call) and selections."""
    P = make_problem(1, 16384, 64, 128, 4096, 4, 512, dist="int", seed=33, name="c3int")
    d = dev_problem(P)
    assert csa.resolve_plan(d["q"], d["k"], d["w"], P.m) == "row_tiles"
    idx = to_np(gpu_select(P, dev=d)).reshape(P.rows, -1)
    sc = to_np(gpu_score(P, dev=d)).reshape(P.rows, P.W)
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([[3, 4, 2047, 2048, 6143, 6144, 6147, 16382, 16383],
                                     rng.choice(np.arange(6148, 16382), 48, replace=False),
                                     rng.choice(np.arange(5, 6143), 16, replace=False)])).astype(np.int64)
    assert len(rows) >= 64
    s_o, i_o = oracle.select(P, rows)
    assert_scores_close(sc[rows], s_o, exact=True, what="c3int score")
    assert_topk_match(idx[rows], i_o, s_o, exact=True, what="c3int select")
