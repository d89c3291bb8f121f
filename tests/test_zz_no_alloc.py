"""The no-allocation entry point (csa_index_select_noalloc) against the
fused select with a caller-provided workspace (csa_index_select).

Both run the same kernels; the no-allocation call takes its workspace from
the library's fixed per-GPU scratch buffer.  Two calls in a row, the second
on a smaller problem, must each equal the regular entry point's output bit
for bit (the scratch keeps the first call's contents, which the second must
not depend on), and a problem whose workspace exceeds the scratch is refused
before any launch.
"""

import numpy as np
import pytest
import torch

from gpu_util import dev_problem, to_np
from synth import make_config, make_problem

import sparse_attention_indexer_csa_amd as csa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


def _both(P, d, return_scores=False):
    ref = csa.select(d["q"], d["k"], d["w"], P.top_k, P.m, scale=P.scale, q_offset=d["q_offset"],
                     q_seg=d["q_seg"], k_seg=d["k_seg"], return_scores=return_scores)
    out = torch.full((P.B, P.S, P.top_k), -7, dtype=torch.int32, device="cuda")
    sc = torch.empty((P.B, P.S, P.W), dtype=torch.float32, device="cuda") if return_scores else None
    got = csa.select_noalloc(d["q"], d["k"], d["w"], P.top_k, P.m, out, scale=P.scale, q_offset=d["q_offset"],
                             q_seg=d["q_seg"], k_seg=d["k_seg"], scores=sc)
    assert got is out
    if return_scores:
        ref_i, ref_s = ref
        np.testing.assert_array_equal(to_np(out), to_np(ref_i))
        assert np.array_equal(to_np(sc).view(np.uint32), to_np(ref_s).view(np.uint32))
    else:
        np.testing.assert_array_equal(to_np(out), to_np(ref))


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    # decode over a 32768-entry cache: the split plan, 8 MiB of workspace
    P = make_config("c5")
    d = dev_problem(P)
    assert csa.resolve_plan(d["q"], d["k"], d["w"], P.m) == "split_rows"
    assert 0 < csa.workspace_size(d["q"], d["k"], d["w"], P.top_k, P.m) <= csa.NOALLOC_SCRATCH_BYTES
    _both(P, d)
    # a smaller decode problem next: the scratch still holds the first call's scores
    Q = make_problem(8, 1, 64, 128, 4096, 4, 100, dist="gauss", seed=77, decode_lengths=(100, 4096))
    dq = dev_problem(Q)
    assert csa.resolve_plan(dq["q"], dq["k"], dq["w"], Q.m) == "split_rows"
    _both(Q, dq)
    # integer grid, several rows per sequence with segments, forced split plan
    R = make_problem(3, 40, 16, 32, 3000, 2, 64, dist="int", seed=5, segments="random")
    dr = dev_problem(R)
    ref = csa.select(dr["q"], dr["k"], dr["w"], R.top_k, R.m, q_seg=dr["q_seg"], k_seg=dr["k_seg"],
                     plan="split_rows")
    out = torch.empty((R.B, R.S, R.top_k), dtype=torch.int32, device="cuda")
    csa.select_noalloc(dr["q"], dr["k"], dr["w"], R.top_k, R.m, out, q_seg=dr["q_seg"], k_seg=dr["k_seg"],
                       plan="split_rows")
    np.testing.assert_array_equal(to_np(out), to_np(ref))


def test_without_workspace_and_with_scores():
    # the row-tile plan needs no workspace; a score output replaces it on the split plan
    P = make_problem(1, 512, 64, 128, 128, 4, 32, dist="gauss", seed=8)
    _both(P, dev_problem(P), return_scores=True)
    _both(P, dev_problem(P))
    Q = make_problem(4, 1, 64, 128, 8192, 4, 512, dist="gauss", seed=9, decode_lengths=(4000, 8192))
    _both(Q, dev_problem(Q), return_scores=True)


def test_oversized_workspace_is_refused():
    # 128 rows x 40000 entries of fp32 scores = 20.5 MB > 16 MiB of scratch
    P = make_problem(128, 1, 4, 32, 40000, 4, 16, dist="zeros", seed=1, decode_lengths=(39000, 40000))
    d = dev_problem(P)
    assert csa.workspace_size(d["q"], d["k"], d["w"], P.top_k, P.m) > csa.NOALLOC_SCRATCH_BYTES
    out = torch.empty((P.B, 1, P.top_k), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        csa.select_noalloc(d["q"], d["k"], d["w"], P.top_k, P.m, out, q_offset=d["q_offset"])
