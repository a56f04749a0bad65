"""bench.py on the CPU: the algorithmic byte counts reproduce the per-config figures worked
out for the c3 and c4 shapes (8,192 tokens, 65,536 routed rows, H = 7168, K = 8, W = 16,
E = 256), and a multi-GPU request exits with a message instead of running."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bytes(wl):
    # every pick routed, no mask, no smooth table, no copy experts: only shapes matter
    P, T = wl.T * wl.K, wl.T
    return bench.algorithmic_bytes(wl, {}, P, 0, T)


def test_c4_bytes():
    d, c = _bytes(workloads.WORKLOADS["c4_w16_int8_roundtrip"])
    # dispatch: x + ids + rows (7168 codes + 4-byte scale + 12-byte triple) + expand_idx
    #           + ep_recv_count + expert_token_nums + recv_offsets
    assert d == (2 * 7168 * 8192 + 4 * 65536 + 65536 * (7168 + 4 + 12) + 4 * 65536
                 + 4 * 4096 + 8 * 256 + 8 * 17)
    assert round(d / 1e6, 2) == 588.79
    # combine: expert rows + ids/expand_idx/weights + ep_recv_count + recv_offsets + y
    assert c == 2 * 7168 * 65536 + 12 * 65536 + 4 * 4096 + 8 * 17 + 2 * 7168 * 8192
    assert round(c / 1e6, 2) == 1057.77


def test_c3_bytes():
    d, c = _bytes(workloads.WORKLOADS["c3_w16_mxfp8_zipf"])
    # 224 MX blocks per row: 224 fp32 scales (Align2 of 224 is 224)
    assert bench.scale_bytes_per_row(workloads.WORKLOADS["c3_w16_mxfp8_zipf"]) == 896
    assert round(d / 1e6, 2) == 647.25
    assert round(c / 1e6, 2) == 1057.77


def test_fp4_rows_are_half_a_byte_per_element():
    wl = workloads.WORKLOADS["c3v_w16_mxfp4_e8m0"]
    d4, _ = _bytes(wl)
    d8, _ = _bytes(wl.replace(out_dtype=2))
    assert d8 - d4 == wl.T * wl.K * wl.H // 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ceiling_library_exports_the_probes_bench_calls():
    """bench.py --mode ceilings loads libmoe_dc_ceiling.so and calls these probes."""
    import ctypes
    from combine_quant_amd.build import CEILING_LIB
    lib = ctypes.CDLL(CEILING_LIB)
    for name in ("ceiling_scatter_copy", "ceiling_write_rows", "ceiling_gather_sum",
                 "ceiling_write_chunks", "ceiling_read_chunks"):
        assert hasattr(lib, name), name
        assert name in open(bench.__file__).read(), name


def test_roofline_names_the_timed_combine_kernel():
    w = workloads.WORKLOADS
    assert bench.combine_kernel_name(w[bench.DEFAULT_WORKLOAD]) == "combine_wave_kernel"
    assert bench.combine_kernel_name(w["c4v_w16_combine_int8"]) == "combine_int8_wide_kernel"
    assert bench.combine_kernel_name(w["c4v_w16_scatter_back_shared"]).endswith(
        "combine_wave_kernel")
