"""Out-of-bounds writes: every output of every kind of kernel sits between two 4 KB canary regions.

Each output buffer is carved out of a larger allocation filled with the byte 0xA5, 4 KB from its
start (which keeps the 16-byte alignment the operands need), with 4 KB of canary after it; the
inputs are ordinary tensors.  After the call the canaries must be untouched and the output
must have been written (no byte pattern of the fill left in a region the call writes whole).
The shapes have ragged M, N and K tails and take every kernel: the producers (E4M3, MXFP4,
E5M2 round-to-nearest and stochastic, both quantize-transposes), the GEMMs on 64x64, 128x128,
256x256 and 256x224 tiles, the skinny MXFP4 kernels (register loads and LDS staging), the
quantized-output epilogues, and split-K.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth

from gpu_util import dev_bf16, dev_u8, note

pytestmark = pytest.mark.gpu

PAD = 4096
FILL = 0xA5


class Guarded:
    """A device tensor of `shape` and `dtype` with FILL canaries of PAD bytes on both sides."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((PAD + n + PAD,), FILL, dtype=torch.uint8, device="cuda")
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        raw = self.raw.cpu().numpy()
        head, tail = raw[:PAD], raw[PAD + self.n:]
        bad_head = np.flatnonzero(head != FILL)
        bad_tail = np.flatnonzero(tail != FILL)
        assert bad_head.size == 0 and bad_tail.size == 0, (
            f"{what}: canary overwritten ({bad_head.size} bytes before the output, "
            f"{bad_tail.size} after; first after-offsets {bad_tail[:8].tolist()})")
        body = raw[PAD:PAD + self.n]
        assert not np.all(body == FILL), f"{what}: output never written"


def _acts(x_bits):
    return dev_bf16(x_bits)


@pytest.mark.parametrize("M,K", [(129, 160), (1, 32), (300, 2080)])
def test_producers(mx, M, K):
    x = synth.bf16_normal(synth.rng_for(M + K), (M, K), outlier_frac=0.01)
    xd = _acts(x)
    for name, qcols in (("mx_act_quant", K), ("mx_act_quant_fp4", K // 2)):
        q, s = Guarded((M, qcols), torch.uint8), Guarded((M, K // 32), torch.uint8)
        note(f"canaries {name} {M}x{K}")
        getattr(mx, name)(xd, q.t, s.t)
        q.check(f"{name} codes {M}x{K}")
        s.check(f"{name} scales {M}x{K}")
    for seed in (None, 7):
        q, s = Guarded((M, K), torch.uint8), Guarded((M, K // 32), torch.uint8)
        mx.mx_quant_e5m2(xd, q.t, s.t, seed=seed)
        q.check(f"e5m2 seed={seed}")
        s.check(f"e5m2 scales seed={seed}")


@pytest.mark.parametrize("R,C", [(256, 520), (96, 1000)])
def test_quant_transposes(mx, R, C):
    x = synth.bf16_normal(synth.rng_for(R * C), (R, C))
    xd = _acts(x)
    for name, kw in (("mx_quant_transpose_e4m3", {}), ("mx_quant_transpose_e5m2", {"seed": 3})):
        q, s = Guarded((C, R), torch.uint8), Guarded((C, R // 32), torch.uint8)
        note(f"canaries {name} {R}x{C}")
        getattr(mx, name)(xd, q.t, s.t, **kw)
        q.check(f"{name} codes")
        s.check(f"{name} scales")


# (kind, M, N, K): each takes a different kernel or tile
GEMMS = [("fp8_fp4", 129, 257, 160),      # 64x64 tiles
         ("fp8_fp8", 600, 1000, 512),     # 128x128 tiles
         ("fp8_fp8", 4100, 3600, 1024),   # 256x256 tiles, M and N tails
         ("fp8_fp4", 2000, 7000, 512),    # 256x224 tiles, N tail
         ("fp8_fp4", 2000, 7168, 512),    # 256x224 tiles, quantized output
         ("fp4_fp4", 41, 4607, 1536),     # skinny MXFP4, LDS-staged
         ("fp4_fp4", 33, 65, 2080),       # skinny MXFP4, register loads
         ("fp4_fp4", 300, 544, 1024)]     # FP4 A on the tiled kernels


@pytest.mark.parametrize("kind,M,N,K", GEMMS)
def test_gemm_outputs(mx, kind, M, N, K):
    a_kind, b_kind = kind.split("_")
    w = synth.gemm_inputs("acts" if a_kind == "fp8" else a_kind, b_kind, M, N, K,
                          seed=M + N + K, with_bias=True)
    if a_kind == "fp8":
        xd = _acts(w.x)
        a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        a_s = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
        mx.mx_act_quant(xd, a, a_s)
    else:
        a, a_s = dev_u8(w.a), dev_u8(w.a_s)
    b, b_s, bias = dev_u8(w.b), dev_u8(w.b_s), dev_bf16(w.bias)
    c = Guarded((M, N), torch.bfloat16)
    note(f"canaries gemm {kind} {M}x{N}x{K}")
    getattr(mx, f"mx_gemm_{kind}")(a, a_s, b, b_s, c.t, bias=bias)
    c.check(f"gemm {kind} {M}x{N}x{K}")
    c = Guarded((M, N), torch.bfloat16)
    getattr(mx, f"mx_gemm_{kind}_bias_gelu")(a, a_s, b, b_s, c.t, bias=bias)
    c.check(f"gemm {kind} gelu {M}x{N}x{K}")
    if N % 32 == 0:
        qcols = N // 2 if kind == "fp4_fp4" else N
        q, qs = Guarded((M, qcols), torch.uint8), Guarded((M, N // 32), torch.uint8)
        getattr(mx, f"mx_gemm_{kind}_quant")(a, a_s, b, b_s, q.t, qs.t, bias=bias)
        q.check(f"gemm {kind} quant codes {M}x{N}x{K}")
        qs.check(f"gemm {kind} quant scales {M}x{N}x{K}")


def test_batched_gemm_output(mx):
    w = synth.gemm_inputs("fp4", "fp4", 41, 200, 1536, seed=5, batch=3, with_bias=True)
    c = Guarded((3, 41, 200), torch.bfloat16)
    note("canaries batched fp4_fp4")
    mx.mx_gemm_fp4_fp4(dev_u8(w.a), dev_u8(w.a_s), dev_u8(w.b), dev_u8(w.b_s), c.t,
                       bias=dev_bf16(w.bias))
    c.check("batched fp4_fp4")


def test_split_k_output_and_workspace(mx):
    M, N, K = 2000, 4000, 5152
    w = synth.gemm_inputs("fp8", "fp4", M, N, K, seed=11, with_bias=True)
    size = mx.mx_gemm_splitk_workspace_size(M, N, K)
    assert size > 0
    ws = Guarded((size,), torch.uint8)
    ws.raw[PAD:PAD + size].zero_()            # the counters start at zero
    c = Guarded((M, N), torch.bfloat16)
    note(f"canaries split-K {M}x{N}x{K}")
    mx.mx_gemm_fp8_fp4_splitk(dev_u8(w.a), dev_u8(w.a_s), dev_u8(w.b), dev_u8(w.b_s), c.t, ws.t,
                              bias=dev_bf16(w.bias))
    c.check("split-K output")
    ws.check("split-K workspace")
