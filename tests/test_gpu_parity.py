"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

* Block offsets, codes, scales (as bit patterns) and zero points: bit-exact.
* y: max|y - y_ref| / max|y_ref| <= 2e-3 per (matrix, M), the tolerance the
  method is held to; y_ref is the oracle's fp64 product with the oracle's own
  dequantized weights.  With max|y_ref| == 0, y must be exactly 0.
* Integer lattice (s = 1, integer x): y must equal y_ref exactly.
* Full-size workloads run in the same launch configuration as bench.py
  (msq_gemm's automatic kernel choice) and are compared on sampled block rows
  that the oracle computes one by one.
"""
import os

import numpy as np
import pytest

import oracle
from block_wise_mixed_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _log(msg):
    print(msg, flush=True)


def check_pack(msq, case, block_rows=None):
    """Pack on the GPU and compare with the oracle (all block rows or the listed ones)."""
    _log(f"pack {case.name} {case.N}x{case.K}")
    pw = msq.quantize_pack(case.W, case.bits, case.perm_row, case.perm_col)
    torch.cuda.synchronize()
    got = pw.to_numpy()
    off_ref, cb = oracle.block_offsets(case.bits)
    assert pw.code_bytes == cb
    assert np.array_equal(got["block_offset"], off_ref)
    ref = oracle.quantize(case.W, case.bits, case.perm_row, case.perm_col, block_rows=block_rows,
                          check=block_rows is None)
    brs = ref["block_rows"]
    assert np.array_equal(got["scale"][brs].view(np.uint32), ref["scale"].view(np.uint32))
    assert np.array_equal(got["zero"][brs], ref["zero"])
    qb = oracle.msq_oracle.blocks_of(ref["q"])  # [len(brs)][NBc][64][128]
    bits_sub = case.bits[brs]
    for b in oracle.SEGMENT_ORDER:
        ii, cc = np.nonzero(bits_sub == b)
        if ii.size == 0:
            continue
        want = oracle.pack_blocks(qb[ii, cc], b)
        starts = off_ref[brs[ii], cc].astype(np.int64) * 1024
        have = got["codes"][starts[:, None] + np.arange(1024 * b)[None, :]]
        assert np.array_equal(have, want), f"codes differ for {b}-bit blocks"
    return pw, ref


def check_y(msq, pw, case, ref, M, kernel="auto", exact=False, x=None):
    x = case.x(M) if x is None else x
    _log(f"gemm {case.name} {case.N}x{case.K} M={M} kernel={kernel}")
    y = msq.gemm(x, pw, kernel=kernel)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    yref = oracle.reference_gemm(x, ref, case.perm_row, case.perm_col)
    if yref.shape[1] != case.N:
        y = y[:, case.perm_row[ref["rows"]]]
    assert np.isfinite(y).all()
    if exact:
        assert np.array_equal(y, yref)
        return 0.0
    scale = np.abs(yref).max() if yref.size else 0.0
    if scale == 0:
        assert (y == 0).all()
        return 0.0
    err = float(np.abs(y - yref).max() / scale)
    _log(f"   rel err {err:.3e}")
    assert err <= TOL
    return err


SMALL_DIST = {0: .1, 1: .15, 2: .3, 3: .2, 4: .15, 8: .1}


@pytest.mark.parametrize("N,K,seed", [(64, 128, 0), (192, 384, 1), (320, 640, 2), (256, 4096, 3),
                                      (1024, 256, 4)])
def test_pack_bit_exact_small(msq, N, K, seed):
    check_pack(msq, synth.random_case(N, K, seed, dist=SMALL_DIST))


@pytest.mark.parametrize("b", [0, 1, 2, 3, 4, 8])
def test_pack_uniform_bitwidth(msq, b):
    pw, ref = check_pack(msq, synth.random_case(192, 512, 10 + b, dist={b: 1.0}))
    if b == 0:
        assert pw.code_bytes == 0


def test_pack_edge_values(msq):
    """All-zero groups, signed zeros, one-signed groups, tiny (subnormal) and huge values."""
    c = synth.random_case(128, 512, 20, dist=SMALL_DIST)
    W = oracle.bf16_to_f32(c.W).copy()
    Wr = W[np.ix_(c.perm_row, c.perm_col)]
    Wr[0, :128] = 0.0
    Wr[1, :128] = -0.0
    Wr[2, 128:256] = np.abs(Wr[2, 128:256])
    Wr[3, 256:384] = -np.abs(Wr[3, 256:384])
    Wr[4, :128] = np.float32(1e-40)  # fp32/bf16 subnormal
    Wr[5, :128] *= np.float32(1e-38)
    Wr[6, 128:256] *= np.float32(1e30)
    Wr[70, 384:] = np.float32(1.5e38)
    Wr[71, 384:] = np.linspace(-1, 1, 128, dtype=np.float32)
    W[np.ix_(c.perm_row, c.perm_col)] = Wr
    c.W = synth.f32_to_bf16_bits(W)
    check_pack(msq, c)


@pytest.mark.parametrize("kernel", ["auto", "gemm"])
def test_smoke_workload_256x512(msq, kernel):
    c = synth.matrix_inputs("linear-256x512", 0)
    pw, ref = check_pack(msq, c)
    for M in synth.WORKLOADS["linear-256x512"].ms:
        check_y(msq, pw, c, ref, M, kernel=kernel)


@pytest.mark.parametrize("N,K,seed", [(512, 1024, 30), (320, 4096, 31)])
def test_m_boundary_sweep(msq, N, K, seed):
    c = synth.random_case(N, K, seed, dist=SMALL_DIST)
    pw, ref = check_pack(msq, c)
    for M in (1, 2, 15, 16, 17, 63, 64, 65, 511, 512, 513):
        check_y(msq, pw, c, ref, M, kernel="auto")
        if M <= 64:
            check_y(msq, pw, c, ref, M, kernel="gemm")
            check_y(msq, pw, c, ref, M, kernel="gemv")


@pytest.fixture(scope="module")
def shape_cases(msq):
    """256 x 8192 matrices (64 block columns per block row) with mixed, all 1-bit and all
    8-bit blocks, packed once for the launch-shape sweep."""
    out = {}
    for name, dist, seed in (("mixed", SMALL_DIST, 50), ("1bit", {1: 1.0}, 51), ("8bit", {8: 1.0}, 52)):
        c = synth.random_case(256, 8192, seed, dist=dist)
        out[name] = (c,) + check_pack(msq, c)
    return out


@pytest.mark.parametrize("split,waves", [(1, 8), (1, 4), (1, 16), (2, 8), (3, 8), (5, 4), (16, 16),
                                         (64, 8)])
@pytest.mark.parametrize("name", ["mixed", "1bit", "8bit"])
def test_decode_launch_shapes(msq, shape_cases, monkeypatch, name, split, waves):
    """M = 1 decode in every launch shape the tuning knobs reach: full 64-column ranges
    (wavefronts then stream more chunks than their ring holds), ragged last ranges, one
    column per range, 4 to 16 wavefronts per workgroup."""
    c, pw, ref = shape_cases[name]
    monkeypatch.setenv("MSQ_GEMV_SPLIT", str(split))
    monkeypatch.setenv("MSQ_GEMV_WAVES", str(waves))
    check_y(msq, pw, c, ref, 1)
    if split > 1:
        # again: the split counters of the last-workgroup reduction start from zero each call
        check_y(msq, pw, c, ref, 1)


def _bf16_cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("waves", [8, 16])
@pytest.mark.parametrize("N,K,seed", [(256, 8192, 70), (192, 1024, 71), (64, 128, 72),
                                      (320, 640, 73)])
def test_decode_gather_matches_prep(msq, monkeypatch, N, K, seed, waves):
    """M = 1 without a K split: the decode workgroups reorder x themselves (no prep
    launch).  The result equals the prep-kernel path bit for bit (the reordered values
    are copies and the k-step sums use the same addition tree) and the oracle within
    tolerance; 64, 8, 1 and 5 block columns per row (ragged perm_col loads)."""
    c = synth.random_case(N, K, seed, dist=SMALL_DIST)
    pw, ref = check_pack(msq, c)
    monkeypatch.setenv("MSQ_GEMV_SPLIT", "1")
    monkeypatch.setenv("MSQ_GEMV_WAVES", str(waves))
    x = _bf16_cuda(c.x(1))
    monkeypatch.setenv("MSQ_M1_GATHER", "0")
    y_prep = msq.gemm(x, pw)
    monkeypatch.setenv("MSQ_M1_GATHER", "1")
    y_gather = msq.gemm(x, pw)
    y_again = msq.gemm(x, pw)
    torch.cuda.synchronize()
    assert torch.equal(y_gather, y_prep)
    assert torch.equal(y_again, y_prep)
    check_y(msq, pw, c, ref, 1)


def test_group_decode_gather_mixed(msq, group_cases, monkeypatch):
    """A grouped M = 1 call whose jobs split between gathering workgroups (one K range)
    and the prep launch (a 16384-wide matrix needs two K ranges; placed first, in the
    middle and last): every output equals its single call on the prep path bit for
    bit, twice in a row, and the oracle within tolerance."""
    monkeypatch.setenv("MSQ_GEMV_SPLIT", "1")
    wide = synth.random_case(128, 16384, 74, dist=SMALL_DIST)
    cases = list(group_cases) + [(wide,) + check_pack(msq, wide)]
    xs_all = [_bf16_cuda(c.x(1)) for c, _, _ in cases]
    for order in ((4, 0, 1, 2, 3), (0, 1, 4, 2, 3), (0, 1, 2, 3, 4)):
        sel = [cases[i] for i in order]
        xs = [xs_all[i] for i in order]
        pws = [pw for _, pw, _ in sel]
        _log(f"group decode, job order {order}")
        for rep in range(2):
            monkeypatch.setenv("MSQ_M1_GATHER", "1")
            outs = msq.gemm_group(xs, pws)
            monkeypatch.setenv("MSQ_M1_GATHER", "0")
            singles = [msq.gemm(x, pw) for x, pw in zip(xs, pws)]
            torch.cuda.synchronize()
            for (c, _, _), y, s in zip(sel, outs, singles):
                assert torch.equal(y, s), c.name
    for c, pw, ref in cases:
        check_y(msq, pw, c, ref, 1)


@pytest.mark.parametrize("N,K,seed", [(192, 512, 0), (512, 4096, 1)])
def test_integer_lattice_is_exact(msq, N, K, seed):
    c, xgen = synth.lattice_case(N, K, seed, dist={0: .1, 1: .2, 2: .2, 3: .2, 4: .2, 8: .1})
    pw, ref = check_pack(msq, c)
    assert (ref["s"][np.repeat(c.bits, 64, axis=0) > 0] == 1).all()
    for M, kernel in ((1, "auto"), (5, "auto"), (64, "auto"), (1, "gemm"), (130, "gemm")):
        check_y(msq, pw, c, ref, M, kernel=kernel, exact=True, x=xgen(M))


def test_all_pruned_gives_zero(msq):
    c = synth.random_case(128, 256, 40, dist={0: 1.0})
    pw, ref = check_pack(msq, c)
    for M, kernel in ((1, "auto"), (3, "auto"), (100, "auto"), (2, "gemm")):
        y = msq.gemm(c.x(M), pw, kernel=kernel)
        torch.cuda.synchronize()
        assert (y.cpu().numpy() == 0).all()


def test_empty_batch(msq):
    c = synth.random_case(128, 256, 41)
    pw, _ = check_pack(msq, c)
    y = msq.gemm(np.zeros((0, 256), np.uint16), pw)
    assert tuple(y.shape) == (0, 128)


def test_deterministic(msq):
    c = synth.random_case(512, 4096, 42, dist=SMALL_DIST)
    pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    pw2 = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    torch.cuda.synchronize()
    assert torch.equal(pw.codes[:pw.code_bytes], pw2.codes[:pw2.code_bytes])
    for M in (1, 16, 300):
        x = c.x(M)
        a = msq.gemm(x, pw)
        b = msq.gemm(x, pw)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_rejects_wrong_x_shape(msq):
    c = synth.random_case(64, 128, 43)
    pw, _ = check_pack(msq, c)
    with pytest.raises(ValueError):
        msq.gemm(np.zeros((2, 256), np.uint16), pw)
    with pytest.raises(msq.MsqError):
        msq.gemm(c.x(65), pw, kernel="gemv")


# ---- full-size workloads, sampled rows --------------------------------------------------

def _sample_block_rows(NBr, seed):
    g = np.random.default_rng(seed)
    pick = {0, NBr - 1} | set(int(v) for v in g.choice(NBr, size=min(NBr, 3), replace=False))
    return np.array(sorted(pick))


FULL = [(w, m.name) for w in ("llama3-8b-q_proj", "llama3-8b-mlp", "llama3-8b-down_proj-prefill",
                              "llama3-70b-layer")
        for m in synth.WORKLOADS[w].matrices]


@pytest.mark.parametrize("workload,matrix", FULL)
def test_full_size_sampled(msq, workload, matrix):
    c = synth.matrix_inputs(workload, matrix)
    brs = _sample_block_rows(c.N // 64, 7)
    pw, ref = check_pack(msq, c, block_rows=brs)
    for M in synth.WORKLOADS[workload].ms:
        check_y(msq, pw, c, ref, M)
    del pw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("split", ["auto", "1"])
def test_graph_replay_matches_eager(msq, monkeypatch, split):
    """The decode and prefill calls are captured in HIP graphs by bench.py: every replay,
    with eager work in between, must equal the eager result bit for bit (at M = 1 with
    the automatic K split and with one K range, where the decode workgroups reorder x
    themselves)."""
    if split != "auto":
        monkeypatch.setenv("MSQ_GEMV_SPLIT", split)
    c = synth.random_case(1024, 4096, 50, dist=SMALL_DIST)
    pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    for M in (1, 16, 200):
        x = torch.from_numpy(c.x(M).view(np.int16)).view(torch.bfloat16).cuda()
        ws = torch.empty(max(msq.workspace_bytes(M, c.N, c.K), 256), dtype=torch.uint8, device="cuda")
        y_eager = msq.gemm(x, pw)
        y = torch.empty_like(y_eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            msq.gemm(x, pw, out=y, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            msq.gemm(x, pw, out=y, workspace=ws)
        other = (-x).contiguous()
        for rep in range(3):
            y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_eager), f"replay {rep} differs at M={M}"
            msq.gemm(other, pw, workspace=ws)  # eager work between replays, same workspace
            torch.cuda.synchronize()


@pytest.fixture(scope="module")
def group_cases(msq):
    """Four matrices of different shapes and bit mixes for the grouped call; the
    first three share K (one activation, as q, k, v of a layer do)."""
    out = []
    for N, K, seed, dist in ((512, 4096, 60, SMALL_DIST), (128, 4096, 61, {2: .7, 3: .3}),
                             (256, 4096, 62, {8: .5, 1: .5}), (192, 1024, 63, SMALL_DIST)):
        c = synth.random_case(N, K, seed, dist=dist)
        out.append((c,) + check_pack(msq, c))
    return out


@pytest.mark.parametrize("M", [1, 3, 200])
def test_group_matches_single_calls(msq, group_cases, monkeypatch, M):
    """Each output of the grouped call equals the single call bit for bit (the same
    kernels, launch plan and summation order) and the oracle within tolerance; at
    M == 1 with several K splits (the shapes here force them) as well, and at a
    prefill M of two row tiles, the second ragged, with four matrices in one launch."""
    monkeypatch.setenv("MSQ_GEMV_SPLIT", "3")
    pws = [pw for _, pw, _ in group_cases]
    x_shared = group_cases[0][0].x(M)
    xs = [x_shared, x_shared, x_shared, group_cases[3][0].x(M)]
    _log(f"group of {len(pws)} M={M}")
    for rep in range(2):  # twice: the split counters start from zero every call
        outs = msq.gemm_group(xs, pws)
        torch.cuda.synchronize()
        for (c, pw, ref), x, y in zip(group_cases, xs, outs):
            single = msq.gemm(x, pw)
            torch.cuda.synchronize()
            assert torch.equal(y, single), c.name
            check_y(msq, pw, c, ref, M, x=x)


def test_group_prefill_one_launch(msq):
    """Two 4096 x 1024 matrices at M = 1024 have enough tiles for the one grouped GEMM
    launch (smaller groups run as split-K single calls): each output equals its single
    call bit for bit and the oracle within tolerance."""
    cases = []
    for seed, dist in ((64, SMALL_DIST), (65, {2: .5, 4: .3, 8: .2})):
        c = synth.random_case(4096, 1024, seed, dist=dist)
        cases.append((c,) + check_pack(msq, c))
    M = 1024
    x = cases[0][0].x(M)
    outs = msq.gemm_group([x, x], [pw for _, pw, _ in cases])
    torch.cuda.synchronize()
    for (c, pw, ref), y in zip(cases, outs):
        single = msq.gemm(x, pw)
        torch.cuda.synchronize()
        assert torch.equal(y, single), c.name
        check_y(msq, pw, c, ref, M, x=x)


@pytest.mark.parametrize("split", [1, 2, 3, 5, 8])
def test_gemm_split_k(msq, monkeypatch, split):
    """The GEMM with its K range cut into `split` pieces (ragged last piece for 3 and 5;
    partials summed in split order by the reduction): oracle within tolerance at a
    one-tile and a two-tile M, and reproducible."""
    c = synth.random_case(256, 8192, 66, dist=SMALL_DIST)
    pw, ref = check_pack(msq, c)
    monkeypatch.setenv("MSQ_GEMM_SPLIT", str(split))
    for M in (16, 130):
        x = c.x(M)
        check_y(msq, pw, c, ref, M, kernel="gemm", x=x)
        a = msq.gemm(x, pw, kernel="gemm")
        b = msq.gemm(x, pw, kernel="gemm")
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("M", [1, 130])
def test_group_sizes(msq, group_cases, M):
    """One matrix, and the largest group: the same matrix eight times."""
    c, pw, ref = group_cases[1]
    x = c.x(M)
    (y1,) = msq.gemm_group([x], [pw])
    ys = msq.gemm_group([x] * msq.GROUP_MAX, [pw] * msq.GROUP_MAX)
    single = msq.gemm(x, pw)
    torch.cuda.synchronize()
    assert torch.equal(y1, single)
    for y in ys:
        assert torch.equal(y, single)
    with pytest.raises(ValueError):
        msq.gemm_group([x] * (msq.GROUP_MAX + 1), [pw] * (msq.GROUP_MAX + 1))


@pytest.mark.parametrize("split", ["auto", "1"])
def test_group_graph_replay_matches_eager(msq, group_cases, monkeypatch, split):
    """bench.py captures grouped decode calls in HIP graphs: every replay, with eager
    work in between on the same workspace, must equal the eager result bit for bit;
    with the automatic split (prep launch, split counters) and with one K range (the
    workgroups reorder x themselves)."""
    if split != "auto":
        monkeypatch.setenv("MSQ_GEMV_SPLIT", split)
    pws = [pw for _, pw, _ in group_cases]
    x_shared = torch.from_numpy(group_cases[0][0].x(1).view(np.int16)).view(torch.bfloat16).cuda()
    x_last = torch.from_numpy(group_cases[3][0].x(1).view(np.int16)).view(torch.bfloat16).cuda()
    xs = [x_shared, x_shared, x_shared, x_last]
    ws = torch.empty(max(msq.group_workspace_bytes(1, pws), 256), dtype=torch.uint8, device="cuda")
    eager = [y.clone() for y in msq.gemm_group(xs, pws)]
    outs = [torch.empty_like(y) for y in eager]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        msq.gemm_group(xs, pws, outs=outs, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        msq.gemm_group(xs, pws, outs=outs, workspace=ws)
    others = [(-x).contiguous() for x in xs]
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"
        msq.gemm_group(others, pws, workspace=ws)  # eager work between replays
        torch.cuda.synchronize()
