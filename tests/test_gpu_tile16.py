"""GPU parity with 16-bit (bf16 passthrough) blocks beside quantized ones: packing
bit-exact, y against the oracle within tolerance through every kernel path, exact on
the integer lattice, and bitwise identical between the single and grouped calls."""
import numpy as np
import pytest

import oracle
from block_wise_mixed_amd import synth

from test_gpu_parity import TOL, check_pack, check_y, _bf16_cuda

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MIX16 = {0: .05, 1: .1, 2: .3, 3: .15, 4: .1, 8: .15, 16: .15}
TQ = {8: .7, 16: .3}  # tiles at 8 or 16 bits only, as the pages' 16/8 variant


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


@pytest.mark.parametrize("N,K,dist,seed", [(256, 1024, MIX16, 80), (192, 384, TQ, 81),
                                           (64, 128, {16: 1.0}, 82), (512, 8192, MIX16, 83)])
def test_pack_and_products(msq, N, K, dist, seed):
    c = synth.random_case(N, K, seed, dist=dist)
    pw, ref = check_pack(msq, c)
    assert pw.tile16_blocks == int((c.bits == 16).sum())
    for M, kernel in ((1, "auto"), (4, "auto"), (4, "gemm"), (64, "gemv"), (130, "auto")):
        check_y(msq, pw, c, ref, M, kernel=kernel)
    check_y(msq, pw, c, ref, 1, options={"gemv_split": 1})  # the workgroups reorder x


def test_integer_lattice_exact(msq):
    """Integer x and small integer W (bf16-exact in the 16-bit blocks): every product
    and sum is exact, so y must equal the oracle exactly."""
    c, _ = synth.lattice_case(192, 512, 84, dist={16: .5, 1: .25, 4: .25})
    W = oracle.bf16_to_f32(c.W).copy()
    Wr = W[np.ix_(c.perm_row, c.perm_col)]
    pt = np.repeat(np.repeat(c.bits == 16, 64, axis=0), 128, axis=1)
    Wr[pt] = np.random.default_rng(84).integers(-8, 8, int(pt.sum())).astype(np.float32)
    W[np.ix_(c.perm_row, c.perm_col)] = Wr
    c.W = synth.f32_to_bf16_bits(W)
    pw, ref = check_pack(msq, c)
    g = np.random.default_rng(5)
    for M in (1, 3, 70):
        x = synth.f32_to_bf16_bits(g.integers(-8, 9, (M, 512)).astype(np.float32))
        check_y(msq, pw, c, ref, M, exact=True, x=x)


def test_group_matches_single(msq):
    cases = [synth.random_case(256, 2048, 85 + i, dist=d) for i, d in enumerate((MIX16, TQ))]
    packed = [check_pack(msq, c)[0] for c in cases]
    for M in (1, 4, 200):  # M = 4: the grouped decode launches, then each 16-bit pass
        xs = [_bf16_cuda(cases[0].x(M))] * 2
        outs = msq.gemm_group(xs, packed)
        for x, pw, y in zip(xs, packed, outs):
            assert torch.equal(y, msq.gemm(x, pw))


def test_group_one_launch_with_16bit_blocks(msq):
    """Groups that reach the one grouped GEMM launch (two 4096 x 1024 matrices at
    M = 1024: 512 tiles): with 16-bit blocks in both (the 16-chunk kernel variant
    k_gemm_group<16>), and mixing a matrix with them and one without (the whole
    launch then takes the 16-chunk variant).  Each output equals its single call bit
    for bit and the oracle within tolerance."""
    M = 1024
    plain = synth.random_case(4096, 1024, 87, dist={1: .2, 2: .5, 4: .2, 8: .1})
    mix = synth.random_case(4096, 1024, 88, dist=MIX16)
    tq = synth.random_case(4096, 1024, 89, dist=TQ)
    packed = {c.name: (c,) + check_pack(msq, c) for c in (plain, mix, tq)}
    x = _bf16_cuda(mix.x(M))
    for names in ((mix.name, tq.name), (plain.name, mix.name)):
        sel = [packed[n] for n in names]
        outs = msq.gemm_group([x, x], [pw for _, pw, _ in sel])
        torch.cuda.synchronize()
        for (c, pw, ref), y in zip(sel, outs):
            single = msq.gemm(x, pw)
            torch.cuda.synchronize()
            assert torch.equal(y, single), c.name
            check_y(msq, pw, c, ref, M, x=mix.x(M))

