"""The committed rocprofv3 summaries name the kernels bench.py picks out of them.

bench.py finds the timed kernels in a kernel trace and in the counter runs by regular
expressions over their demangled names (template arguments included), so a change to a kernel's
template parameters must come with a change to those patterns, or the summaries silently lose
those kernels.  This checks every pattern against the names in the committed trace summary, and
the MFMA-utilisation summary's arithmetic on a synthetic counter run.
"""
import glob
import json
import os
import re

import bench

PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def _stats_kernel_names():
    names = []
    for path in glob.glob(os.path.join(PROFILES, "kernel_stats_*.txt")):
        with open(path) as fh:
            names += [ln.split(" | ")[0] for ln in fh if " | " in ln]
    return names


def test_every_kernel_pattern_names_a_profiled_kernel():
    # the kernels of a default run, in the kernel-trace summary of a default run
    names = _stats_kernel_names()
    assert names, "no kernel-trace summary under profiles/"
    for pattern in bench.KERNEL_PATTERNS:
        hits = [n for n in names if re.search(pattern, n)]
        assert len(hits) == 1, f"{pattern!r} matches {len(hits)} profiled kernels"


def test_traffic_summaries_are_complete():
    paths = glob.glob(os.path.join(PROFILES, "traffic_*.json"))
    assert paths
    for path in paths:
        with open(path) as fh:
            d = json.load(fh)
        for key in ("source_hash", "hbm_bytes_per_launch", "algorithmic_bytes_per_launch",
                    "traffic_over_algorithmic"):
            assert key in d, f"{os.path.basename(path)} lacks {key}"
        assert d["hbm_bytes_per_launch"] >= d["algorithmic_bytes_per_launch"] * 0.99, path


def _write_csv(path, header, rows):
    with open(path, "w") as fh:
        fh.write(",".join(header) + "\n")
        for r in rows:
            fh.write(",".join(f'"{v}"' if isinstance(v, str) else str(v) for v in r) + "\n")


def test_summarize_busy_arithmetic(tmp_path):
    """A synthetic counter run: 2 dispatches of the GEMM and one other kernel, counters summed over
    8 XCDs as rocprofv3 writes them.  Active cycles per XCD g = 200000 over 100 us (2 GHz);
    MFMA busy = 0.5 of g x 1024 SIMDs; busy CU cycles = 0.75 of g x 256 CUs."""
    busy = tmp_path / "busy"
    busy.mkdir()
    _write_csv(busy / "run_agent_info.csv", ["Name", "Simd_Count", "Cu_Count", "Num_Xcc"],
               [["gfx950", 1024, 256, 8]])
    gemm = ("void mx::(anonymous namespace)::gemm_mx_kernel<0, 4, true, false, 0, false, 224>"
            "(mx::(anonymous namespace)::Args)")
    _write_csv(busy / "run_kernel_trace.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                                "End_Timestamp"],
               [[1, gemm, 1000, 101000], [2, gemm, 200000, 300000], [3, "other", 0, 10]])
    g = 200000.0
    counters = {"SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * g * 1024, "SQ_BUSY_CYCLES": 1.0,
                "SQ_BUSY_CU_CYCLES": 0.75 * g * 256, "GRBM_GUI_ACTIVE": g * 8,
                "SQ_INSTS_MFMA": 0.5 * g * 1024 / 32}
    rows = [[d, gemm, name, v] for d in (1, 2) for name, v in counters.items()]
    rows += [[3, "other", "GRBM_GUI_ACTIVE", 5.0]]
    _write_csv(busy / "run_counter_collection.csv",
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    out = bench.summarize_busy(str(busy), prof_dir=str(tmp_path))
    assert out["dispatches"] == 2
    assert abs(out["clock_ghz"] - 2.0) < 1e-4
    assert abs(out["mfma_util"] - 0.5) < 1e-4
    assert abs(out["cu_busy"] - 0.75) < 1e-4
    assert abs(out["mfma_busy_over_busy_cu"] - 0.5 / 0.75) < 1e-3
    assert out["mfma_busy_cycles_per_inst"] == 32.0
    assert (tmp_path / "mfma_util_gemm_fp8_fp4_4096x7168x2048.json").exists()


def test_summarize_busy_picks_the_fp8_gemms_by_grid(tmp_path):
    """The 8192^3 and batched FP8 x FP8 GEMMs run one kernel; their profiles are told apart by the
    dispatch grid (work-items) the counter csv records.  Each gets its own file, from its own
    dispatches only: 8192^3 at MFMA util 0.25, the batched shape at 0.75."""
    busy = tmp_path / "busy"
    busy.mkdir()
    _write_csv(busy / "run_agent_info.csv", ["Name", "Simd_Count", "Cu_Count", "Num_Xcc"],
               [["gfx950", 1024, 256, 8]])
    fp8 = ("void mx::(anonymous namespace)::gemm_mx_kernel<0, 0, false, false, 0, false, 256>"
           "(mx::(anonymous namespace)::Args)")
    _write_csv(busy / "run_kernel_trace.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                                "End_Timestamp"],
               [[1, fp8, 0, 100000], [2, fp8, 200000, 300000]])
    g = 200000.0
    rows = []
    for d, grid, util in ((1, 32 * 32 * 256, 0.25), (2, 4 * 8 * 256 * 8, 0.75)):
        counters = {"SQ_VALU_MFMA_BUSY_CYCLES": util * g * 1024, "SQ_BUSY_CYCLES": 1.0,
                    "SQ_BUSY_CU_CYCLES": g * 256, "GRBM_GUI_ACTIVE": g * 8,
                    "SQ_INSTS_MFMA": util * g * 1024 / 32}
        rows += [[d, fp8, grid, name, v] for name, v in counters.items()]
    _write_csv(busy / "run_counter_collection.csv",
               ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"], rows)
    bench.summarize_busy(str(busy), prof_dir=str(tmp_path))
    for key, util in (("gemm_fp8_fp8_8192cubed", 0.25),
                      ("gemm_fp8_fp8_batched_8x1024x2048x2048", 0.75)):
        with open(tmp_path / f"mfma_util_{key}.json") as fh:
            d = json.load(fh)
        assert d["dispatches"] == 1 and abs(d["mfma_util"] - util) < 1e-4, key
    assert not (tmp_path / "mfma_util_gemm_fp8_fp4_4096x7168x2048.json").exists()
