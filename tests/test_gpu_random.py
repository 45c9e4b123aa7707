"""GPU parity on seeded random problems: shapes, bit mixes (pruned, 16-bit and
single-width maps among them), batch sizes on both sides of every automatic
kernel choice (M = 1, 2..16, 17..64, 65..299) and explicit launch options
(K splits, wavefront counts, the GEMM at small M), each compared with the CPU
oracle: packing bit for bit, y within 2e-3 of the oracle's fp64 product."""
import numpy as np
import pytest

import oracle
from block_wise_mixed_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3

torch = pytest.importorskip("torch")

DISTS = [{2: 1.0}, {1: .5, 2: .5}, {0: .1, 1: .15, 2: .3, 3: .2, 4: .15, 8: .1}, {3: .5, 8: .5},
         {0: .05, 1: .1, 2: .3, 3: .15, 4: .1, 8: .15, 16: .15}, {4: 1.0}, {0: .9, 2: .1},
         {16: .5, 2: .5}]


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _bf16_cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _cases(n, seed):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = 64 * int(g.integers(1, 80))
        K = 128 * int(g.integers(1, 72))
        dist = DISTS[i % len(DISTS)]
        Ms = (1, int(g.integers(2, 17)), int(g.integers(17, 65)), int(g.integers(65, 300)))
        opts = {1: {"gemv_split": int(g.integers(1, 5)), "gemv_waves": int(g.choice([4, 8, 16]))},
                Ms[1]: {"gemv_split": int(g.integers(1, 5))},
                Ms[2]: {"gemv_split": int(g.integers(1, 5))},
                Ms[3]: {"gemm_split": int(g.integers(1, 4))}}
        out.append((N, K, dist, 500 + i, Ms, opts))
    return out


@pytest.mark.parametrize("N,K,dist,seed,Ms,opts", _cases(40, 2024))
def test_random_problem(msq, N, K, dist, seed, Ms, opts):
    c = synth.random_case(N, K, seed, dist=dist)
    print(f"random case {N}x{K} seed {seed} dist {sorted(dist)} M {Ms}", flush=True)
    pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    ref = oracle.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    torch.cuda.synchronize()
    got = pw.to_numpy()
    assert np.array_equal(got["block_offset"], ref["block_offset"])
    assert np.array_equal(got["codes"], ref["codes"])
    assert np.array_equal(got["scale"].view(np.uint32), ref["scale"].view(np.uint32))
    assert np.array_equal(got["zero"], ref["zero"])
    for M in Ms:
        x = c.x(M)
        yref = oracle.reference_gemm(x, ref, c.perm_row, c.perm_col)
        scale = float(np.abs(yref).max())
        runs = [("auto", None), ("auto", opts[M])]
        if 2 <= M <= 64:
            runs.append(("gemm", None))
        for kernel, opt in runs:
            y = msq.gemm(_bf16_cuda(x), pw, kernel=kernel, options=opt)
            torch.cuda.synchronize()
            y = y.cpu().numpy().astype(np.float64)
            assert np.isfinite(y).all()
            if scale == 0.0:
                assert (y == 0).all()
                continue
            err = float(np.abs(y - yref).max() / scale)
            assert err <= TOL, f"M={M} kernel={kernel} options={opt}: {err:.3e}"
