"""The residual epilogue of the large-problem GEMM kernel, whose residual tile is copied into LDS
during the last K steps (tiles inside the matrix with 16-byte aligned residual rows).

Each case runs twice: with the residual at a 16-byte aligned address, which takes the copy
during the last K steps for every tile inside the matrix, and with the same values one element
past such an address, which sends every tile through the epilogue's own element loads.  Both
compute the same fp32 sum + bias + residual and round it once, so the outputs must agree bit for
bit; the aligned one is also checked against the float64 reference, |out - ref| <= 2^-7 |ref| +
2^-20 sum_k |a_k b_k| with ref = sum a*b + bias + residual.  The shapes take every copy plan the
kernel has: 256 x 224 and 256 x 256 tiles; copy slots fewer than, equal to, and more than a
slice's copies (E4M3 x E2M1, E2M1 x E2M1, E4M3 x E4M3); K of one 8-step group only, and of several;
ragged M and N edges; a batch sharing one residual; the residual being the output itself.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16
from test_gpu_gemm import assert_within
from test_gpu_gemm_epilogue import operands

pytestmark = pytest.mark.gpu

CUS = 256


def large_kernel_tile_n(M, N, K, batch=1):
    """The library's rule for the large-problem kernel and its tile width (None: not taken)."""
    def tiles(bn):
        return -(-M // 256) * -(-N // bn) * batch
    if not (2 * tiles(256) > CUS and K % 512 == 0):
        return None
    waves = lambda bn: -(-tiles(bn) // CUS)
    return 224 if waves(224) * 224 < waves(256) * 256 else 256


def misaligned_copy(t: torch.Tensor) -> torch.Tensor:
    """The values of bf16 tensor t in a buffer that starts 2 bytes past a 16-byte boundary."""
    n = t.numel()
    raw = torch.empty(n + 8, dtype=torch.bfloat16, device="cuda")
    out = raw[1:1 + n].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 == 2
    return out


def run_residual(mx, kind, args, res: torch.Tensor, bias, shape):
    c = poison_bf16(shape)
    getattr(mx, f"mx_gemm_{kind}_bias_residual")(*args, res, c, bias=bias)
    torch.cuda.synchronize()
    return host_bf16_bits(c)


# (a_kind, b_kind, M, N, K, batch, tile width the library picks)
CASES = [("acts", "fp4", 4096, 7168, 2048, None, 224),   # the headline shape: 6 slots, 7 copies
         ("acts", "fp4", 4096, 4096, 1024, None, 256),   # 256 x 256: 6 slots, 8 copies
         ("fp4", "fp4", 2048, 7168, 1024, None, 224),    # 4 slots, 7 copies
         ("acts", "fp8", 2000, 7000, 512, None, 224),    # 8 slots, 7 copies; K of one group;
                                                          # ragged M and N
         ("acts", "fp8", 4000, 4096, 1024, None, 256),   # 8 slots, 8 copies; ragged M
         ("fp4", "fp4", 4096, 4096, 1024, None, 256),    # 4 slots, 8 copies
         ("acts", "fp4", 1024, 7000, 512, 2, 224)]       # a batch sharing one residual


@pytest.mark.parametrize("a_kind,b_kind,M,N,K,batch,tile_n", CASES)
def test_prefetched_residual_matches_element_loads_and_oracle(mx, a_kind, b_kind, M, N, K, batch,
                                                              tile_n):
    assert large_kernel_tile_n(M, N, K, batch or 1) == tile_n
    w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=M + 7 * N + K, batch=batch,
                          with_bias=True)
    a, a_s, kind, A, B, bias = operands(w)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    shape = (M, N) if batch is None else (batch, M, N)
    res_bits = synth.bf16_normal(synth.rng_for(M + N), (M, N))     # one residual for every batch
    res = dev_bf16(res_bits)
    assert res.data_ptr() % 16 == 0
    bias_t = dev_bf16(w.bias)
    note(f"gemm {kind} residual {shape}x{K} (aligned: copied during the last K steps)")
    out = run_residual(mx, kind, args, res, bias_t, shape)
    note(f"gemm {kind} residual {shape}x{K} (misaligned: epilogue element loads)")
    out_ref_path = run_residual(mx, kind, args, misaligned_copy(res), bias_t, shape)
    diff = np.count_nonzero(out != out_ref_path)
    assert diff == 0, f"{diff} outputs differ between the two residual paths"
    ref, S = O.gemm_residual_ref(A, B, bias, res_bits)
    assert_within(out, ref, S, f"{kind} residual {shape}x{K}")


def test_in_place_residual(mx):
    # c is the residual (out = sum + bias + c, written over c) on the copied-in path.
    M, N, K = 2048, 7168, 1024
    assert large_kernel_tile_n(M, N, K) == 224
    w = synth.gemm_inputs("acts", "fp4", M, N, K, seed=501, with_bias=True)
    a, a_s, kind, A, B, bias = operands(w)
    args = (dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s))
    res_bits = synth.bf16_normal(synth.rng_for(502), (M, N))
    bias_t = dev_bf16(w.bias)
    note(f"gemm {kind} residual in place {M}x{N}x{K}")
    out = run_residual(mx, kind, args, dev_bf16(res_bits), bias_t, (M, N))
    c = dev_bf16(res_bits)
    getattr(mx, f"mx_gemm_{kind}_bias_residual")(*args, c, c, bias=bias_t)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(c), out)
