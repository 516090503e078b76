"""The hot path captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

The library's entry points launch on the stream they are given and allocate, free and
synchronize nothing, so a producer -> GEMM pipeline can be captured once and replayed.  Each
replay must give exactly the bytes of the same calls made eagerly (the kernels are
deterministic), with the program's own eager work and synchronizations between replays, and the
eager result itself is checked against the oracle.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import dev_bf16, dev_u8, host_bf16_bits, note

pytestmark = pytest.mark.gpu


def _pipelines(mx):
    rng = synth.rng_for(4242)
    # E4M3 producer -> FP8 x MXFP4 GEMM + bias
    M1, N1, K1 = 300, 520, 512
    x1 = synth.bf16_normal(rng, (M1, K1), outlier_frac=0.01)
    w1, ws1 = synth.fp4_packed_uniform(rng, N1, K1), synth.e8m0_uniform(rng, (N1, K1 // 32))
    b1 = synth.bf16_normal(rng, (N1,), std=0.1)
    # MXFP4 producer -> FP4 x FP4 GEMM + bias + GELU (a skinny A4W4 shape)
    M2, N2, K2 = 41, 1536, 1536
    x2 = synth.bf16_normal(rng, (M2, K2))
    w2, ws2 = synth.fp4_packed_uniform(rng, N2, K2), synth.e8m0_uniform(rng, (N2, K2 // 32))
    b2 = synth.bf16_normal(rng, (N2,), std=0.1)
    host = dict(x1=x1, w1=w1, ws1=ws1, b1=b1, x2=x2, w2=w2, ws2=ws2, b2=b2)
    d = dict(x1=dev_bf16(x1), w1=dev_u8(w1), ws1=dev_u8(ws1), b1=dev_bf16(b1),
             q1=torch.empty((M1, K1), dtype=torch.uint8, device="cuda"),
             s1=torch.empty((M1, K1 // 32), dtype=torch.uint8, device="cuda"),
             c1=torch.empty((M1, N1), dtype=torch.bfloat16, device="cuda"),
             x2=dev_bf16(x2), w2=dev_u8(w2), ws2=dev_u8(ws2), b2=dev_bf16(b2),
             q2=torch.empty((M2, K2 // 2), dtype=torch.uint8, device="cuda"),
             s2=torch.empty((M2, K2 // 32), dtype=torch.uint8, device="cuda"),
             c2=torch.empty((M2, N2), dtype=torch.bfloat16, device="cuda"))

    def calls(stream=None):
        mx.mx_act_quant(d["x1"], d["q1"], d["s1"], stream=stream)
        mx.mx_gemm_fp8_fp4(d["q1"], d["s1"], d["w1"], d["ws1"], d["c1"], bias=d["b1"],
                           stream=stream)
        mx.mx_act_quant_fp4(d["x2"], d["q2"], d["s2"], stream=stream)
        mx.mx_gemm_fp4_fp4_bias_gelu(d["q2"], d["s2"], d["w2"], d["ws2"], d["c2"], bias=d["b2"],
                                     stream=stream)

    return host, d, calls


def _snapshot(d):
    torch.cuda.synchronize()
    return {k: d[k].view(torch.uint8).cpu().numpy().copy() for k in ("q1", "s1", "c1", "q2", "s2", "c2")}


def _poison(d):
    for k in ("q1", "s1", "q2", "s2"):
        d[k].fill_(0xA5)
    for k in ("c1", "c2"):
        d[k].view(torch.int16).fill_(-1)


def test_graph_replays_match_eager_and_oracle(mx):
    host, d, calls = _pipelines(mx)
    note("graph: eager run")
    calls()
    eager = _snapshot(d)

    # the eager result against the oracle
    q1, s1 = O.act_quant(host["x1"])
    assert np.array_equal(eager["q1"], q1) and np.array_equal(eager["s1"], s1)
    ref, S = O.gemm_ref(O.decode_e4m3_rows(q1, s1), O.decode_fp4_rows(host["w1"], host["ws1"]),
                        O.bf16_to_f64(host["b1"]))
    assert O.within_tolerance(eager["c1"].view(np.uint16), ref, S).all()
    q2, s2 = O.act_quant_fp4(host["x2"])
    assert np.array_equal(eager["q2"], q2) and np.array_equal(eager["s2"], s2)
    _, pre, S2 = O.gemm_gelu_ref(O.decode_fp4_rows(q2, s2),
                                 O.decode_fp4_rows(host["w2"], host["ws2"]),
                                 O.bf16_to_f64(host["b2"]))
    assert O.gelu_within(eager["c2"].view(np.uint16), pre, S2).all()

    note("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    other = torch.empty_like(d["c1"])
    for i in range(4):
        _poison(d)
        # eager work of the program's own between replays, then a synchronization
        mx.mx_gemm_fp8_fp4(d["q1"], d["s1"], d["w1"], d["ws1"], other)
        torch.cuda.synchronize()
        note(f"graph: replay {i}")
        g.replay()
        got = _snapshot(d)
        for k in eager:
            assert np.array_equal(got[k], eager[k]), (i, k)
    # and the eager calls still give the same bytes after the graph ran
    _poison(d)
    calls()
    again = _snapshot(d)
    for k in eager:
        assert np.array_equal(again[k], eager[k]), k
    del g


def test_graph_replays_splitk_quant_epilogue_and_stochastic_quantizers(mx):
    # Split-K leaves its counters at zero after every launch, so a captured split GEMM replays
    # with the same workspace; the quantizing epilogue and the seeded stochastic quantizers are
    # deterministic too.  Each replay must give the eager bytes.
    M, N, K = 1280, 3328, 5120                          # 65 tiles: the split plan cuts K in two
    w = synth.gemm_inputs("fp8", "fp4", M, N, K, seed=91, with_bias=True)
    wsz = mx.mx_gemm_splitk_workspace_size(M, N, K)
    assert wsz > 0
    rng = synth.rng_for(92)
    g_host = synth.bf16_normal(rng, (256, 1024), std=1e-3)
    d = dict(a=dev_u8(w.a), a_s=dev_u8(w.a_s), b=dev_u8(w.b), b_s=dev_u8(w.b_s),
             bias=dev_bf16(w.bias), ws=torch.zeros(wsz, dtype=torch.uint8, device="cuda"),
             c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
             q=torch.empty((M, N), dtype=torch.uint8, device="cuda"),
             qs=torch.empty((M, N // 32), dtype=torch.uint8, device="cuda"),
             g=dev_bf16(g_host),
             gq=torch.empty((256, 1024), dtype=torch.uint8, device="cuda"),
             gs=torch.empty((256, 32), dtype=torch.uint8, device="cuda"),
             tq=torch.empty((1024, 256), dtype=torch.uint8, device="cuda"),
             ts=torch.empty((1024, 8), dtype=torch.uint8, device="cuda"))
    outs = ("c", "q", "qs", "gq", "gs", "tq", "ts")

    def calls(stream=None):
        mx.mx_gemm_fp8_fp4_splitk(d["a"], d["a_s"], d["b"], d["b_s"], d["c"], d["ws"],
                                  bias=d["bias"], stream=stream)
        mx.mx_gemm_fp8_fp4_quant(d["a"], d["a_s"], d["b"], d["b_s"], d["q"], d["qs"],
                                 bias=d["bias"], stream=stream)
        mx.mx_quant_e5m2(d["g"], d["gq"], d["gs"], seed=1234, stream=stream)
        mx.mx_quant_transpose_e5m2(d["g"], d["tq"], d["ts"], seed=1234, stream=stream)

    def snap():
        torch.cuda.synchronize()
        return {k: d[k].view(torch.uint8).cpu().numpy().copy() for k in outs}

    note("graph 2: eager run")
    calls()
    eager = snap()
    assert int(d["ws"][:65 * 8].count_nonzero()) == 0
    # the stochastic codes against the oracle's Philox draws
    oq, os_ = O.grad_quant_e5m2(g_host, seed=1234)
    assert np.array_equal(eager["gq"], oq) and np.array_equal(eager["gs"], os_)
    tq, ts = O.quant_transpose_e5m2(g_host, seed=1234)
    assert np.array_equal(eager["tq"], tq) and np.array_equal(eager["ts"], ts)

    note("graph 2: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for i in range(4):
        for k in outs:
            d[k].view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        note(f"graph 2: replay {i}")
        g.replay()
        got = snap()
        for k in outs:
            assert np.array_equal(got[k], eager[k]), (i, k)
        assert int(d["ws"][:65 * 8].count_nonzero()) == 0, i
    del g
