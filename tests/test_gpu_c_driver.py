"""The library driven from C alone: tests/c_abi/mx_c_driver (built by __graft_entry__.build())
allocates device memory with hipMalloc and calls act_quant and the GEMMs through include/mx.h,
with no Python or torch in between.  This test writes the inputs of 3 operand kinds x 4 layouts
(plain, bias, batched with distinct operands, batched with the weight, its scales and the bias
broadcast by stride 0) x 6 shapes, runs the program once over all of them, and checks what it
wrote against the oracle: act_quant's codes and scale bytes byte for byte, every GEMM output
within |out - ref| <= 2^-7 |ref| + 2^-20 sum_k |a_k b_k| of the float64 reference from the
same bytes.
"""
import os
import subprocess

import numpy as np
import pytest

from block_scaled_precision_act_amd import synth
from oracle import mx_oracle as O

from gpu_util import note

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "c_abi", "mx_c_driver")

KINDS = {"fp8_fp4": ("acts", "fp4"), "fp8_fp8": ("acts", "fp8"), "fp4_fp4": ("fp4", "fp4")}
LAYOUTS = ["plain", "bias", "batched", "broadcast"]
SHAPES = [(1, 32, 64), (17, 33, 96), (41, 96, 1536), (129, 257, 160), (300, 520, 1024),
          (600, 1000, 512)]
BATCH = 3


def _cases():
    for kind in KINDS:
        for layout in LAYOUTS:
            for (M, N, K) in SHAPES:
                yield kind, layout, M, N, K


def _write(path, arr):
    np.ascontiguousarray(arr).tofile(path)


def _read(path, dtype, shape):
    return np.fromfile(path, dtype=dtype).reshape(shape)


def _decode_b(b_kind, b, b_s):
    return O.decode_fp4_rows(b, b_s) if b_kind == "fp4" else O.decode_fp8_block(b, b_s)


def test_c_program_over_kinds_layouts_and_shapes(tmp_path):
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built; run tests/c_abi/build.py (or __graft_entry__.build())")
    lines, work = [], []
    for i, (kind, layout, M, N, K) in enumerate(_cases()):
        a_kind, b_kind = KINDS[kind]
        batched = layout in ("batched", "broadcast")
        w = synth.gemm_inputs(a_kind, b_kind, M, N, K, seed=1000 + i,
                              batch=BATCH if batched else None, with_bias=layout != "plain")
        name = f"c{i:03d}"
        d = tmp_path / name
        d.mkdir()
        b, b_s, bias = w.b, w.b_s, w.bias
        if layout == "broadcast":                       # one weight, scales and bias for all
            b, b_s, bias = w.b[0], w.b_s[0], w.bias[0]
        if a_kind == "acts":
            _write(d / "x.bin", w.x)
        else:
            _write(d / "a.bin", w.a)
            _write(d / "a_s.bin", w.a_s)
        _write(d / "b.bin", b)
        _write(d / "b_s.bin", b_s)
        if bias is not None:
            _write(d / "bias.bin", bias)
        lines.append(f"{name} {kind} {layout} {M} {N} {K} {BATCH if batched else 1}")
        work.append((name, kind, layout, M, N, K, batched, w, b, b_s, bias))
    (tmp_path / "cases.txt").write_text("\n".join(lines) + "\n")
    note(f"c driver: {len(lines)} cases")
    r = subprocess.run([DRIVER, str(tmp_path)], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, f"mx_c_driver failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    assert f"{len(lines)} cases, 0 failed" in r.stdout

    bad = []
    for name, kind, layout, M, N, K, batched, w, b, b_s, bias in work:
        a_kind, b_kind = KINDS[kind]
        nb = BATCH if batched else 1
        lead = (nb,) if batched else ()
        d = tmp_path / name
        c = _read(d / "c.bin", np.uint16, lead + (M, N))
        if a_kind == "acts":
            q = _read(d / "q.bin", np.uint8, lead + (M, K))
            s = _read(d / "s.bin", np.uint8, lead + (M, K // 32))
        for i in range(nb):
            if a_kind == "acts":
                x = w.x[i] if batched else w.x
                rq, rs = O.act_quant(x)
                qi, si = (q[i], s[i]) if batched else (q, s)
                if not (np.array_equal(qi, rq) and np.array_equal(si, rs)):
                    bad.append(f"{name} {kind} {layout} {M}x{N}x{K}[{i}]: act_quant bytes differ")
                    continue
                A = O.decode_e4m3_rows(rq, rs)
            else:
                A = O.decode_fp4_rows(w.a[i] if batched else w.a, w.a_s[i] if batched else w.a_s)
            if layout == "broadcast":
                B, bi = _decode_b(b_kind, b, b_s), bias
            elif batched:
                B, bi = _decode_b(b_kind, b[i], b_s[i]), bias[i]
            else:
                B, bi = _decode_b(b_kind, b, b_s), bias
            ref, S = O.gemm_ref(A, B, None if bi is None else O.bf16_to_f64(bi))
            ci = c[i] if batched else c
            ok = O.within_tolerance(ci, ref, S)
            if not ok.all():
                bad.append(f"{name} {kind} {layout} {M}x{N}x{K}[{i}]: {np.count_nonzero(~ok)} of "
                           f"{ok.size} outside the bound")
    assert not bad, "\n".join(bad[:20])
