"""Why the library's FP8 GEMMs do not run on the scaled FP8 matrix instruction.

A test-only GEMM (tests/fp8_mfma_probe/fp8_mfma_gemm.hip) contracts the same bytes as the
library on gfx950's v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 activations (quantized by the oracle)
against E4M3 weights with 32x32 block scales (the 1024^3 + bias configuration) and against MXFP4
weights (the 4096x7168x2048 + bias configuration).  Every output is compared with the float64
reference of the oracle.

What the test records (printed with each case, and kept under profiles/):
* how many outputs the instruction leaves outside the GEMM bound
  |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k|: it must be more than zero, which is the
  reason for the bf16 design;
* that the probe is a correct GEMM all the same: every output lies within a bound 256 times
  looser in its sum term (2^-12 sum|a b|), so the misses are rounding inside the instruction,
  not a wrong operand layout or scale;
* that the library's own GEMM on the very same bytes meets the bound on every output.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note, poison_bf16

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_mfma_probe",
                   "libfp8_mfma_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python tests/fp8_mfma_probe/build.py)")
    lib = ctypes.CDLL(LIB)
    f = lib.fp8_mfma_probe_gemm
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    return f


def _case(w):
    a, a_s = O.act_quant(w.x)
    A = O.decode_e4m3_rows(a, a_s)
    B = O.decode_fp4_rows(w.b, w.b_s) if w.b_kind == "fp4" else O.decode_fp8_block(w.b, w.b_s)
    ref, S = O.gemm_ref(A, B, O.bf16_to_f64(w.bias))
    return a, a_s, ref, S


@pytest.mark.parametrize("name", ["fp8xfp8_1024cubed_bias", "fp8xmxfp4_4096x7168x2048_bias"])
def test_scaled_fp8_mfma_misses_the_bound(mx, probe, name):
    w = getattr(synth, name)()
    a, a_s, ref, S = _case(w)
    da, das, db, dbs, dbias = dev_u8(a), dev_u8(a_s), dev_u8(w.b), dev_u8(w.b_s), dev_bf16(w.bias)
    c = poison_bf16((w.M, w.N))
    cf = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    b_fmt = 4 if w.b_kind == "fp4" else 0
    note(f"fp8 mfma probe {name}")
    st = probe(b_fmt, da.data_ptr(), das.data_ptr(), db.data_ptr(), dbs.data_ptr(),
               dbias.data_ptr(), c.data_ptr(), cf.data_ptr(), w.M, w.N, w.K,
               torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    bias = O.bf16_to_f64(w.bias)
    ok = O.within_tolerance(out, ref, S)
    misses = int(np.count_nonzero(~ok))
    sum_err = np.abs(cf.cpu().numpy().astype(np.float64) - (ref - bias[None, :]))
    worst = float(np.max(sum_err / np.maximum(S, 1e-300)))
    loose = np.abs(O.bf16_to_f64(out) - ref) <= np.ldexp(np.abs(ref), -7) + np.ldexp(S, -12)
    note(f"fp8 mfma probe {name}: {misses} of {ok.size} outputs outside the bound; "
         f"largest |fp32 sum - exact| / sum|a*b| = {worst:.3e} (2^{np.log2(worst):.2f})")
    print(f"[fp8-mfma-bound] {name}: misses={misses} outputs={ok.size} "
          f"worst_err_over_S={worst:.6e}", flush=True)
    assert loose.all(), "probe GEMM is wrong beyond rounding: operand layout or scales"
    assert misses > 0
    # the library's GEMM on the same bytes meets the bound everywhere
    kind = "fp8_fp4" if w.b_kind == "fp4" else "fp8_fp8"
    c2 = poison_bf16((w.M, w.N))
    getattr(mx, f"mx_gemm_{kind}")(da, das, db, dbs, c2, bias=dbias)
    torch.cuda.synchronize()
    assert O.within_tolerance(host_bf16_bits(c2), ref, S).all()
