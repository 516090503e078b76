"""GEMM shapes on both sides of every kernel-selection threshold, against the oracle.

The library picks one of several kernels for a problem from its shape alone (split-K aside):
the large-problem kernel on 256 x 256 or 256 x 224 tiles when 256 x 256 tiles give more than half
the CUs a workgroup and K % 512 == 0, the step-wise kernel on 256 x 256 tiles when K is not such
a multiple, 128 x 128 tiles when those still fill the CUs, the kernel that copies a 64 x 64 tile's
whole K into LDS when K % 256 == 0, K <= 1024 and one wave of 64 x 64 tiles suffices, the
step-wise 64 x 64 kernel otherwise; both operands MXFP4 with M <= 64 take the skinny scaled-FP4
kernel.  Each case below sits one tile, one K chunk or one row on either side of such a rule
(`pick` restates the rule for one MI355X, and the case names the kernel it expects), so that a
mistake at a boundary of the selection, or in the tails a kernel sees only there, shows as an
output outside |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k|.
"""
import pytest

from block_scaled_precision_act_amd import synth

from test_gpu_gemm import check_workload

pytestmark = pytest.mark.gpu

CUS = 256


def pick(a_kind, M, N, K, batch=1):
    """The kernel the library selects for an unsplit problem on one MI355X (256 CUs)."""
    if a_kind == "fp4_fp4" and M <= 64:
        return "skinny"

    def tiles(bm, bn):
        return -(-M // bm) * -(-N // bn) * batch
    if 2 * tiles(256, 256) > CUS:
        if K % 512 == 0:
            waves = lambda bn: -(-tiles(256, bn) // CUS)
            return "large224" if waves(224) * 224 < waves(256) * 256 else "large256"
        return "step256"
    if tiles(128, 128) >= CUS:
        return "step128"
    if K % 256 == 0 and K <= 1024 and tiles(64, 64) <= CUS:
        return "whole_k64"
    return "step64"


# (M, N, K, batch, expected kernel)
EDGES = [
    (2048, 4096, 512, 1, "step128"),     # 128 tiles of 256 x 256: exactly half the CUs
    (2048, 4097, 512, 1, "large224"),    # one column more: 136 tiles, the large kernel
    (2048, 4097, 544, 1, "step256"),     # same tiles, K not a multiple of 512
    (4096, 4096, 512, 1, "large256"),    # 256 tiles of 256 x 256: one full wave
    (1024, 4097, 512, 2, "large224"),    # batched: 2 x 68 tiles
    (2048, 2048, 256, 1, "step128"),     # 256 tiles of 128 x 128
    (1920, 2048, 256, 1, "step64"),      # 240 tiles of 128 x 128, 960 of 64 x 64
    (1024, 1024, 1024, 1, "whole_k64"),  # 256 tiles of 64 x 64, K of four chunks
    (1024, 1025, 1024, 1, "step64"),     # one column more: 272 tiles
    (1024, 1024, 1280, 1, "step64"),     # K of five chunks
    (1000, 1000, 992, 1, "step64"),      # K not a multiple of 256
    (999, 1000, 768, 1, "whole_k64"),    # ragged M and N tails
]


@pytest.mark.parametrize("kind", ["fp8_fp4", "fp8_fp8"])
@pytest.mark.parametrize("M,N,K,batch,kernel", EDGES)
def test_selection_edges(mx, kind, M, N, K, batch, kernel):
    assert pick(kind, M, N, K, batch) == kernel
    b_kind = "fp4" if kind == "fp8_fp4" else "fp8"
    with_bias = (M + N + K) % 2 == 1
    w = synth.gemm_inputs("fp8", b_kind, M, N, K, seed=5 * M + 3 * N + K + batch,
                          batch=None if batch == 1 else batch, with_bias=with_bias)
    check_workload(mx, w)


@pytest.mark.parametrize("M,N,K,kernel", [(64, 300, 256, "skinny"), (65, 300, 256, "whole_k64"),
                                          (64, 1000, 1056, "skinny"), (65, 1000, 1056, "step64")])
@pytest.mark.parametrize("with_bias", [False, True])
def test_fp4_fp4_skinny_edge(mx, M, N, K, kernel, with_bias):
    assert pick("fp4_fp4", M, N, K) == kernel
    w = synth.gemm_inputs("fp4", "fp4", M, N, K, seed=11 * M + N + K + with_bias,
                          with_bias=with_bias)
    check_workload(mx, w)
