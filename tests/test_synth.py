"""The seeded generators are deterministic and stay inside each format's valid codes (CPU only)."""
import numpy as np

from block_scaled_precision_act_amd import synth


def test_seeded_and_deterministic():
    a = synth.gemm_inputs("acts", "fp8", 8, 40, 64, seed=5, with_bias=True)
    b = synth.gemm_inputs("acts", "fp8", 8, 40, 64, seed=5, with_bias=True)
    for k in ("x", "b", "b_s", "bias"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    c = synth.gemm_inputs("acts", "fp8", 8, 40, 64, seed=6, with_bias=True)
    assert not np.array_equal(a.x, c.x)


def test_code_ranges():
    rng = synth.rng_for(1)
    e = synth.e4m3_uniform_nonnan(rng, (200000,))
    assert not np.any((e == 0x7F) | (e == 0xFF))
    assert len(np.unique(e)) == 254
    s = synth.e8m0_uniform(rng, (100000,))
    assert s.min() == 118 and s.max() == 136
    p = synth.fp4_packed_uniform(rng, 64, 4096)
    assert p.shape == (64, 2048) and len(np.unique(p & 15)) == 16 and len(np.unique(p >> 4)) == 16


def test_shapes_of_named_workloads():
    w = synth.fp8xmxfp4_16x256x512()
    assert w.x.shape == (16, 512) and w.b.shape == (256, 256) and w.b_s.shape == (256, 16)
    w = synth.gemm_inputs("acts", "fp8", 100, 70, 96, seed=1)
    assert w.b_s.shape == (3, 3)
    w = synth.gemm_inputs("fp4", "fp4", 41, 64, 1536, seed=1)
    assert w.a.shape == (41, 768) and w.a_s.shape == (41, 48)
    x = synth.bf16_normal(synth.rng_for(2), (1000, 100), outlier_frac=0.01)
    v = (x.astype(np.uint32) << 16).view(np.float32)
    assert 0.005 < np.mean(np.abs(v) > 10) < 0.02
