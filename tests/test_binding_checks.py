"""The Python binding's argument checks, which run before any library call.

The library sees raw pointers only, so a host tensor, a wrong element type, rows that are not
contiguous or a buffer smaller than the sizes imply would make a kernel read or write out of
bounds; the binding refuses them.  Host tensors are refused without a GPU (CPU tests); the other
checks need tensors on the GPU.
"""
import pytest
import torch

import block_scaled_precision_act_amd as mx


def _cpu_u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def _cpu_bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_host_tensors_are_refused_before_any_library_call():
    x, q, s = _cpu_bf16(4, 64), _cpu_u8(4, 64), _cpu_u8(4, 2)
    for fn, args in [
        (mx.mx_act_quant, (x, q, s)),
        (mx.mx_act_quant_fp4, (x, _cpu_u8(4, 32), s)),
        (mx.mx_quant_e5m2, (x, q, s)),
        (mx.mx_quant_transpose_e4m3, (_cpu_bf16(64, 32), _cpu_u8(32, 64), _cpu_u8(32, 2))),
        (mx.mx_gemm_fp8_fp4, (_cpu_u8(4, 64), _cpu_u8(4, 2), _cpu_u8(32, 32), _cpu_u8(32, 2),
                              _cpu_bf16(4, 32))),
        (mx.mx_gemm_fp8_fp8_quant, (_cpu_u8(4, 64), _cpu_u8(4, 2), _cpu_u8(32, 64),
                                    _cpu_u8(1, 2), _cpu_u8(4, 32), _cpu_u8(4, 1))),
        (mx.mx_gemm_fp4_fp4_bias_gelu, (_cpu_u8(4, 32), _cpu_u8(4, 2), _cpu_u8(32, 32),
                                        _cpu_u8(32, 2), _cpu_bf16(4, 32))),
        (mx.mx_gemm_e5m2_e4m3, (_cpu_u8(4, 64), _cpu_u8(4, 2), _cpu_u8(32, 64), _cpu_u8(32, 2),
                                _cpu_bf16(4, 32))),
    ]:
        with pytest.raises(mx.MxError) as e:
            fn(*args)
        assert e.value.status == mx.MX_ERR_DEVICE, fn.__name__


@pytest.mark.gpu
class TestOnGpu:
    def test_non_tensors_are_refused(self, mx):
        x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
        s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
        with pytest.raises(TypeError):
            mx.mx_act_quant(x, [0] * 256, s)

    def test_wrong_dtype(self, mx):
        x = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
        q = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
        s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
        with pytest.raises(TypeError):
            mx.mx_act_quant(x, q, s)

    def test_undersized_outputs(self, mx):
        x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
        for q, s in [(torch.zeros((4, 32), dtype=torch.uint8, device="cuda"),
                      torch.zeros((4, 2), dtype=torch.uint8, device="cuda")),
                     (torch.zeros((4, 64), dtype=torch.uint8, device="cuda"),
                      torch.zeros((4, 1), dtype=torch.uint8, device="cuda")),
                     (torch.zeros((3, 64), dtype=torch.uint8, device="cuda"),
                      torch.zeros((3, 2), dtype=torch.uint8, device="cuda"))]:
            with pytest.raises(mx.MxError) as e:
                mx.mx_act_quant(x, q, s)
            assert e.value.status == mx.MX_ERR_SHAPE

    def test_gemm_operand_shapes_must_agree(self, mx):
        M, N, K = 16, 64, 128
        a = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
        a_s = torch.zeros((M, K // 32), dtype=torch.uint8, device="cuda")
        b = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
        b_s = torch.zeros((N, K // 32), dtype=torch.uint8, device="cuda")
        c = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        mx.mx_gemm_fp8_fp4(a, a_s, b, b_s, c)                 # consistent: runs
        torch.cuda.synchronize()
        for bad in [dict(b=torch.zeros((N, K), dtype=torch.uint8, device="cuda")),      # FP8 B
                    dict(b_s=torch.zeros((N // 32, K // 32), dtype=torch.uint8, device="cuda")),
                    dict(a_s=torch.zeros((M, K // 64), dtype=torch.uint8, device="cuda")),
                    dict(c=torch.zeros((M, N + 1), dtype=torch.bfloat16, device="cuda")[:, :N])]:
            args = dict(a=a, a_s=a_s, b=b, b_s=b_s, c=c)
            args.update(bad)
            with pytest.raises(mx.MxError) as e:
                mx.mx_gemm_fp8_fp4(args["a"], args["a_s"], args["b"], args["b_s"], args["c"])
            assert e.value.status in (mx.MX_ERR_SHAPE, mx.MX_ERR_STRIDE)
        with pytest.raises(mx.MxError) as e:                  # bias of the wrong length
            mx.mx_gemm_fp8_fp4(a, a_s, b, b_s, c,
                               bias=torch.zeros(N - 1, dtype=torch.bfloat16, device="cuda"))
        assert e.value.status == mx.MX_ERR_SHAPE

    def test_transposed_views_are_refused(self, mx):
        x = torch.zeros((64, 4), dtype=torch.bfloat16, device="cuda").t()     # [4, 64] view
        q = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
        s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
        with pytest.raises(mx.MxError) as e:
            mx.mx_act_quant(x, q, s)
        assert e.value.status == mx.MX_ERR_STRIDE

    def test_batched_output_must_be_batched(self, mx):
        M, N, K = 8, 32, 64
        a = torch.zeros((2, M, K), dtype=torch.uint8, device="cuda")
        a_s = torch.zeros((2, M, K // 32), dtype=torch.uint8, device="cuda")
        b = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
        b_s = torch.zeros((1, K // 32), dtype=torch.uint8, device="cuda")
        c = torch.zeros((3, M, N), dtype=torch.bfloat16, device="cuda")     # 3 != 2
        with pytest.raises(mx.MxError) as e:
            mx.mx_gemm_fp8_fp8(a, a_s, b, b_s, c)
        assert e.value.status == mx.MX_ERR_SHAPE
        c = torch.zeros((2, M, N), dtype=torch.bfloat16, device="cuda")
        mx.mx_gemm_fp8_fp8(a, a_s, b, b_s, c)                 # broadcast B: runs
        torch.cuda.synchronize()

    def test_default_stream_is_torchs_current_stream(self, mx):
        assert mx._stream(None) == torch.cuda.current_stream().cuda_stream
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            assert mx._stream(None) == s.cuda_stream
            assert mx._stream(None) == torch.cuda.current_stream().cuda_stream
        assert mx._stream(s) == s.cuda_stream
