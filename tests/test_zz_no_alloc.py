"""msq_gemm_noalloc (the entry point that allocates nothing: its workspace is the
library's static device scratch) against msq_gemm (a caller-provided workspace):
bit-identical y through the C ABI, on consecutive calls of shrinking size, the
second call smaller than the first, for the decode (M = 1 with and without a K
split, M = 16) and the prefill kernel (M = 200, split K)."""
import numpy as np
import pytest

from block_wise_mixed_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _bf16_cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


# (N, K, M), each pair run big then small
CASES = [((4096, 8192, 1), (512, 1024, 1)),        # decode, one K range, then a small one
         ((2048, 14336, 1), (256, 4096, 1)),       # decode with K split (counters), then small
         ((4096, 4096, 16), (1024, 2048, 16)),     # decode M = 16, K split (arrival counters)
         ((4096, 8192, 200), (1024, 1024, 130))]   # prefill, split K, then smaller


@pytest.mark.parametrize("big,small", CASES)
def test_noalloc_matches_gemm(msq, big, small):
    for seed, (N, K, M) in enumerate((big, small)):
        c = synth.random_case(N, K, 300 + seed, dist={0: .05, 1: .1, 2: .4, 3: .2, 4: .15, 8: .1})
        pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
        x = _bf16_cuda(c.x(M))
        ref = msq.gemm(x, pw)
        y = msq.gemm_noalloc(x, pw)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"N={N} K={K} M={M}"
        # again, right after: the scratch keeps the last call's contents
        y2 = msq.gemm_noalloc(x, pw)
        torch.cuda.synchronize()
        assert torch.equal(y2, ref)


def test_noalloc_rejects_oversize(msq):
    """A prefill whose workspace exceeds the scratch is refused before any launch."""
    c = synth.random_case(64, 16384, 310, dist={2: 1.0})
    pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    M = 4096  # gathered x alone: 4096 * 16384 * 2 = 128 MiB
    assert msq.workspace_bytes(M, c.N, c.K) > msq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, c.K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msq.MsqError) as e:
        msq.gemm_noalloc(x, pw)
    assert e.value.status == 5
