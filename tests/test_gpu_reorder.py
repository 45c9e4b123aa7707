"""GPU parity of the channel reordering (msq_reorder_channels) with the oracle."""
import numpy as np
import pytest

from oracle import msq_reorder as R
from block_wise_mixed_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


@pytest.mark.parametrize("N,K,rows", [(256, 512, True), (1024, 8192, True), (28672, 1024, True),
                                      (8192, 8192, False), (64, 128, True)])
def test_integer_saliency_exact(msq, N, K, rows):
    """Small-integer saliency: every row and column sum is exact in fp32 in any order,
    so the permutations must equal the oracle's, ties (many) by index."""
    print(f"reorder int {N}x{K} rows={rows}", flush=True)
    S = synth.draw_saliency(N, K, N + K, integer=True)
    pr, pc = msq.reorder_channels(S, reorder_rows=rows)
    torch.cuda.synchronize()
    rr, rc = R.reorder_channels(S, reorder_rows=rows)
    assert np.array_equal(pr.cpu().numpy(), rr)
    assert np.array_equal(pc.cpu().numpy(), rc)


@pytest.mark.parametrize("N,K", [(2048, 4096), (512, 28672)])
def test_real_saliency_sorted(msq, N, K):
    """Activation-aware saliency: valid permutations, ordered by the oracle's fp64 scores
    up to fp32 summation error, and reproducible."""
    print(f"reorder real {N}x{K}", flush=True)
    S = synth.draw_saliency(N, K, 7)
    pr, pc = msq.reorder_channels(S)
    pr2, pc2 = msq.reorder_channels(S)
    torch.cuda.synchronize()
    assert torch.equal(pr, pr2) and torch.equal(pc, pc2)
    pr, pc = pr.cpu().numpy(), pc.cpu().numpy()
    assert sorted(pr.tolist()) == list(range(N)) and sorted(pc.tolist()) == list(range(K))
    r, c = R.channel_scores(S)
    for perm, s in ((pr, r), (pc, c)):
        d = np.diff(s[perm])
        assert (d <= 1e-5 * s.max()).all()
