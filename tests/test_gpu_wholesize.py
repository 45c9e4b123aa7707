"""Whole-matrix GPU parity on every full-size workload, in the launch configuration
bench.py times (msq_gemm's automatic kernel choice, msq_gemm_group for the layer's
grouped linears).

For every matrix: block offsets, codes, scales (bit patterns) and zero points of
EVERY block row are compared bit for bit with the oracle, and y of every output row
at every M the workload names is compared within the 2e-3 tolerance against the
oracle's fp64 product.  The oracle runs in chunks of block rows (each chunk is one
call of oracle.quantize on those rows) so that memory stays bounded; the chunking
changes nothing in what it computes (rows are independent in the quantizer, and the
product of a chunk is its own rows of y).
"""
import numpy as np
import pytest

import oracle
from block_wise_mixed_amd import synth

from test_gpu_parity import TOL, _log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CHUNK_BLOCK_ROWS = 32


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _bf16_cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def compare_whole(msq, c, Ms, ys_gpu=None, pw=None):
    """Pack c on the GPU (unless pw is given) and compare every block row with the
    oracle; y at each M in Ms (GPU y computed by msq.gemm unless ys_gpu[M] is given)."""
    if pw is None:
        pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    xs = {M: c.x(M) for M in Ms}
    if ys_gpu is None:
        ys_gpu = {M: msq.gemm(_bf16_cuda(xs[M]), pw) for M in Ms}
    torch.cuda.synchronize()
    got = pw.to_numpy()
    ys = {M: y.cpu().numpy() for M, y in ys_gpu.items()}
    off_ref, cb = oracle.block_offsets(c.bits)
    assert pw.code_bytes == cb
    assert np.array_equal(got["block_offset"], off_ref), "block offsets differ"
    oracle.validate(c.N, c.K, c.bits, c.perm_row, c.perm_col)
    NBr = c.N // 64
    err = {M: 0.0 for M in Ms}
    scale = {M: 0.0 for M in Ms}
    for r0 in range(0, NBr, CHUNK_BLOCK_ROWS):
        brs = np.arange(r0, min(NBr, r0 + CHUNK_BLOCK_ROWS))
        ref = oracle.quantize(c.W, c.bits, c.perm_row, c.perm_col, block_rows=brs, check=False)
        assert np.array_equal(got["scale"][brs].view(np.uint32), ref["scale"].view(np.uint32)), \
            f"scales differ in block rows {brs[0]}..{brs[-1]}"
        assert np.array_equal(got["zero"][brs], ref["zero"]), \
            f"zero points differ in block rows {brs[0]}..{brs[-1]}"
        qb = oracle.msq_oracle.blocks_of(ref["q"])
        for b in oracle.SEGMENT_ORDER:
            ii, cc = np.nonzero(ref["bits"] == b)
            if ii.size == 0:
                continue
            want = oracle.pack_blocks(qb[ii, cc], b)
            starts = off_ref[brs[ii], cc].astype(np.int64) * 1024
            have = got["codes"][starts[:, None] + np.arange(1024 * b)[None, :]]
            assert np.array_equal(have, want), \
                f"codes differ for {b}-bit blocks in block rows {brs[0]}..{brs[-1]}"
        cols = c.perm_row[ref["rows"]]  # original output rows of this chunk
        # the oracle's product of the chunk's reordered rows (column t of yref is
        # reordered row ref["rows"][t], i.e. original row cols[t]), whether or not
        # the chunk covers the whole matrix
        What = oracle.dequantize(ref["q"], ref["s"], ref["z"], ref["bits"])
        for M in Ms:
            yref = oracle.matmul(oracle.bf16_to_f32(xs[M]), What, c.perm_col)
            yg = ys[M][:, cols].astype(np.float64)
            assert np.isfinite(yg).all()
            err[M] = max(err[M], float(np.abs(yg - yref).max()))
            scale[M] = max(scale[M], float(np.abs(yref).max()))
        del ref, qb, What
    for M in Ms:
        rel = err[M] / scale[M] if scale[M] > 0 else err[M]
        _log(f"   {c.name} {c.N}x{c.K} M={M}: rel err {rel:.3e} over all {c.N} rows")
        assert rel <= TOL
    return pw


SINGLE = [("llama3-8b-q_proj", "q_proj"), ("llama3-8b-mlp", "gate_proj"),
          ("llama3-8b-mlp", "up_proj"), ("llama3-8b-mlp", "down_proj"),
          ("llama3-8b-down_proj-prefill", "down_proj"), ("llama3-70b-layer", "o_proj"),
          ("llama3-70b-layer", "down_proj")]


@pytest.mark.parametrize("workload,matrix", SINGLE)
def test_whole_matrix(msq, workload, matrix):
    c = synth.matrix_inputs(workload, matrix)
    _log(f"whole {workload} {matrix} {c.N}x{c.K}")
    compare_whole(msq, c, synth.WORKLOADS[workload].ms)
    torch.cuda.empty_cache()


# the layer's grouped linears, as bench.py calls them (one shared activation each)
GROUPS = [("q_proj", "k_proj", "v_proj"), ("gate_proj", "up_proj")]


@pytest.mark.parametrize("names", GROUPS, ids=["qkv", "gate_up"])
def test_whole_layer_group(msq, names):
    wl = "llama3-70b-layer"
    cases = [synth.matrix_inputs(wl, n) for n in names]
    pws = [msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col) for c in cases]
    Ms = synth.WORKLOADS[wl].ms
    # one shared activation per M: the first matrix's (all share K)
    xs = {M: cases[0].x(M) for M in Ms}
    ys = {}
    for M in Ms:
        x = _bf16_cuda(xs[M])
        ys[M] = msq.gemm_group([x] * len(pws), pws)
    for i, c in enumerate(cases):
        _log(f"whole {wl} {c.name} {c.N}x{c.K} (grouped)")
        c.x = (lambda M, _x=xs: _x[M])  # the activation the group used
        compare_whole(msq, c, Ms, ys_gpu={M: ys[M][i] for M in Ms}, pw=pws[i])
    del pws, ys
    torch.cuda.empty_cache()
