"""The MXFP4 activation producer on the GPU against the oracle, byte for byte (packed E2M1 codes
and E8M0 scale bytes), and the producer feeding the FP4 x FP4 GEMM against the oracle's own
pipeline."""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, host_u8, note, poison_bf16

pytestmark = pytest.mark.gpu


def run_fp4(mx, x_bits: np.ndarray):
    M, K = x_bits.shape
    x = dev_bf16(x_bits)
    q = torch.full((M, K // 2), 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full((M, K // 32), 0xAA, dtype=torch.uint8, device="cuda")
    mx.mx_act_quant_fp4(x, q, s)
    torch.cuda.synchronize()
    return host_u8(q), host_u8(s)


def assert_same(x, q, s):
    rq, rs = O.act_quant_fp4(x)
    bad_s = np.argwhere(s != rs)
    assert bad_s.size == 0, [(tuple(i), int(s[tuple(i)]), int(rs[tuple(i)])) for i in bad_s[:8]]
    bad = np.argwhere(q != rq)
    assert bad.size == 0, [(tuple(i), hex(x[i[0], 2 * i[1]]), hex(x[i[0], 2 * i[1] + 1]),
                            hex(q[tuple(i)]), hex(rq[tuple(i)])) for i in bad[:8]]


def _finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def _exhaustive_blocks() -> np.ndarray:
    """Every finite bf16 value under every scale it can meet.  E8M0 exponents run from -15 (the
    1e-4 floor) to 126 (the largest bf16): for each E a block's first element is 6 * 2^E, which
    makes that block's scale exactly 2^E (the largest bf16 stands in at E = 126, where 6 * 2^E
    overflows), and the other 31 run through every finite bf16 x with |x| <= 6 * 2^E."""
    b = _finite_bf16()
    mag = O.bf16_to_f64(b & 0x7FFF)
    blocks = []
    for E in range(-15, 127):
        if E == 126:
            head, lim = np.array([0x7F7F], np.uint16), np.inf
        else:
            lim = 6.0 * 2.0 ** E
            head = (np.array([lim], np.float32).view(np.uint32) >> 16).astype(np.uint16)
        vals = b[mag <= lim]
        n = -(-len(vals) // 31)
        body = np.zeros(n * 31, np.uint16)
        body[:len(vals)] = vals
        blocks.append(np.concatenate([np.repeat(head, n)[:, None], body.reshape(n, 31)], axis=1))
    allb = np.concatenate(blocks, axis=0)
    pad = (-len(allb)) % 32
    allb = np.concatenate([allb, np.zeros((pad, 32), np.uint16)], axis=0)
    return allb.reshape(-1, 1024)


def test_exhaustive_bf16_times_scales(mx):
    x = _exhaustive_blocks()
    note(f"act_quant_fp4 exhaustive {x.shape}")
    q, s = run_fp4(mx, x)
    assert_same(x, q, s)


def test_every_bf16_amax_sets_the_scale(mx):
    # One block per finite bf16 value v, all 32 elements v (and -v in the odd ones): the scale
    # byte follows from amax = |v| alone, over every amax that exists, floor included.
    b = _finite_bf16()
    x = np.repeat(b[:, None], 32, axis=1)
    x[:, 1::2] ^= 0x8000
    pad = (-len(x)) % 8
    x = np.concatenate([x, np.zeros((pad, 32), np.uint16)]).reshape(-1, 256)
    note(f"act_quant_fp4 every amax {x.shape}")
    q, s = run_fp4(mx, x)
    assert_same(x, q, s)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (5, 160), (7, 1056), (33, 4128), (1, 8192),
                                 (129, 288), (1000, 1024), (41, 1536), (41, 6144)])
def test_ragged_shapes(mx, M, K):
    rng = np.random.default_rng(M * 7919 + K)
    x = synth.bf16_normal(rng, (M, K), outlier_frac=0.02)
    note(f"act_quant_fp4 M={M} K={K}")
    q, s = run_fp4(mx, x)
    assert_same(x, q, s)


def test_edge_values(mx):
    rng = np.random.default_rng(11)
    x = synth.bf16_normal(rng, (16, 256))
    x[0, :32] = 0                                       # zero block: the floor, all codes 0
    x[1, :32] = 0x8000                                  # negative zeros: code 8
    x[2, :32] = rng.integers(1, 128, 32)                # subnormal bf16
    x[3, :32] = rng.integers(0x8001, 0x8080, 32)        # negative subnormals
    x[4, :32] = 0x7F7F                                  # the largest bf16
    x[5, :32] = 0xFF7F
    x[6, 32:64] = 0x40C0                                # 6.0: scale 2^0, code 7
    x[7, :16] = 0x40C0
    x[7, 16:32] = np.array([0x3E80, 0x3F40, 0x3FA0, 0x3FE0, 0x4020, 0x4060, 0x40A0,    # ties
                            0xBE80, 0xBF40, 0xBFA0, 0xBFE0, 0xC020, 0xC060, 0xC0A0,
                            0x3E7F, 0x3E81], np.uint16)
    x[8, :] = x[8, :] | 0x8000
    x[9, :32] = 0x38D1                                  # 1e-4 in bf16, just under the floor
    x[10, :32] = 0x40C1                                 # just over 6: scale 2^1
    note("act_quant_fp4 edges")
    q, s = run_fp4(mx, x)
    assert_same(x, q, s)
    assert s[6, 1] == 127 and np.all(q[6, 16:32] == 0x77)
    assert np.all(q[1, :16] == 0x88) and np.all(q[0, :16] == 0) and s[0, 0] == 127 - 15


def test_headline_activations_16384x7168_sampled_rows(mx):
    x = synth.act_quant_standalone_16384x7168()
    note("act_quant_fp4 16384x7168")
    q, s = run_fp4(mx, x)
    rows = np.unique(np.concatenate([[0, 1, 16383], np.random.default_rng(2).integers(0, 16384, 300)]))
    assert_same(x[rows], q[rows], s[rows])


def test_strided_batched_with_gaps(mx):
    B, M, K = 3, 40, 96
    x = synth.bf16_normal(np.random.default_rng(19), (B, M, K), outlier_frac=0.05)
    sx, sq, ss = M * K + 1024, M * K // 2 + 4096, M * K // 32 + 160
    xd = torch.zeros(B * sx, dtype=torch.int16, device="cuda")
    for i in range(B):
        xd[i * sx:i * sx + M * K] = torch.from_numpy(x[i].reshape(-1).view(np.int16)).cuda()
    xv = xd.view(torch.bfloat16).as_strided((B, M, K), (sx, K, 1))
    qd = torch.full((B * sq,), 0x5A, dtype=torch.uint8, device="cuda")
    sd = torch.full((B * ss,), 0x5A, dtype=torch.uint8, device="cuda")
    qv = qd.as_strided((B, M, K // 2), (sq, K // 2, 1))
    sv = sd.as_strided((B, M, K // 32), (ss, K // 32, 1))
    note("act_quant_fp4 strided batched")
    mx.mx_act_quant_fp4_strided_batched(xv, qv, sv)
    torch.cuda.synchronize()
    qh, sh = host_u8(qd), host_u8(sd)
    for i in range(B):
        rq, rs = O.act_quant_fp4(x[i])
        n = M * K // 2
        assert np.array_equal(qh[i * sq:i * sq + n].reshape(M, K // 2), rq)
        assert np.array_equal(sh[i * ss:i * ss + M * K // 32].reshape(M, K // 32), rs)
        assert np.all(qh[i * sq + n:(i + 1) * sq] == 0x5A)
        assert np.all(sh[i * ss + M * K // 32:(i + 1) * ss] == 0x5A)


def test_broadcast_input_and_repeat_deterministic(mx):
    B, M, K = 4, 17, 512
    x = synth.bf16_normal(synth.rng_for(23), (M, K))
    xv = dev_bf16(x).unsqueeze(0).expand(B, M, K)            # batch stride 0
    q = torch.empty((B, M, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((B, M, K // 32), dtype=torch.uint8, device="cuda")
    note("act_quant_fp4 broadcast batch")
    mx.mx_act_quant_fp4_strided_batched(xv, q, s)
    torch.cuda.synchronize()
    rq, rs = O.act_quant_fp4(x)
    for i in range(B):
        assert np.array_equal(host_u8(q[i]), rq) and np.array_equal(host_u8(s[i]), rs)
    first = run_fp4(mx, x)
    for _ in range(3):
        again = run_fp4(mx, x)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    mx.mx_act_quant_fp4(e, torch.empty((0, 32), dtype=torch.uint8, device="cuda"),
                        torch.empty((0, 2), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("M,N,K", [(41, 4608, 1536), (41, 1536, 6144), (300, 1024, 2048),
                                   (4096, 7168, 2048)])
def test_pipeline_act_quant_fp4_then_fp4_gemm(mx, M, N, K):
    # bf16 activations -> MXFP4 on the GPU -> FP4 x FP4 GEMM with bias, on one stream, against
    # the oracle's pipeline (oracle producer, exact decode, float64 GEMM).
    rng = synth.rng_for(M * 31 + N * 7 + K)
    x = synth.bf16_normal(rng, (M, K), outlier_frac=0.01)
    wb = synth.fp4_packed_uniform(rng, N, K)
    wbs = synth.e8m0_uniform(rng, (N, K // 32))
    bias = synth.bf16_normal(rng, (N,))
    xd = dev_bf16(x)
    q = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    c = poison_bf16((M, N))
    note(f"pipeline act_quant_fp4 -> gemm fp4_fp4 {M}x{N}x{K}")
    mx.mx_act_quant_fp4(xd, q, s)
    mx.mx_gemm_fp4_fp4(q, s, dev_u8(wb), dev_u8(wbs), c, bias=dev_bf16(bias))
    torch.cuda.synchronize()
    out = host_bf16_bits(c)
    a, a_s = O.act_quant_fp4(x)
    if M * N > 4_000_000:
        rows = np.random.default_rng(3).integers(0, M, 4000)
        cols = np.random.default_rng(4).integers(0, N, 4000)
        ur, ri = np.unique(rows, return_inverse=True)
        uc, ci = np.unique(cols, return_inverse=True)
        A = O.decode_fp4_rows(a[ur], a_s[ur])
        B = O.decode_fp4_rows(wb[uc], wbs[uc])
        ref, S = O.gemm_ref_at(A, B, ri, ci, O.bf16_to_f64(bias)[uc])
        ok = O.within_tolerance(out[rows, cols], ref, S)
        assert np.isfinite(O.bf16_to_f64(out)).all()
    else:
        ref, S = O.gemm_ref(O.decode_fp4_rows(a, a_s), O.decode_fp4_rows(wb, wbs),
                            O.bf16_to_f64(bias))
        ok = O.within_tolerance(out, ref, S)
    assert ok.all(), f"{np.count_nonzero(~ok)} of {ok.size} outputs outside the bound"
