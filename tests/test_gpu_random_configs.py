"""GPU parity over seeded random configurations: each case draws a valid attribute set
(ranks, experts, special experts, batch, hidden size including ragged and element-wise
sizes, top-k, every quant mode with every output type, scales shape and scale format it
allows, both mask kinds, the three routings) and a seeded input, then compares the HIP
library with the CPU oracle -- dispatch bit for bit, combine within 1e-2 relative / 1e-3
absolute -- on both routing paths (inside the scatter launch where the batch is small, and
as kernels of their own).  The int8 block-quantized and scatter-back combines run over the
same configurations.  A further set of draws carries IEEE binary16 tokens instead of bf16."""
import numpy as np
import pytest

import harness
import workloads

pytestmark = pytest.mark.gpu

N_CASES = 100

# (out_dtype, scales_kind, scale_format) choices per quant mode
_VARIANTS = {
    0: [(0, 0, 0)],
    1: [(o, k, 0) for o in (0, 1) for k in (1, 2, 3)],
    2: [(o, k, 0) for o in (0, 1, 2, 3) for k in (0, 1, 2, 3)],
    3: [(o, k, 0) for o in (0, 2, 3) for k in (0, 1, 2, 3)],
    4: [(o, 0, f) for o in (0, 2, 3, 4) for f in (0, 1, 2)],
    5: [(o, 0, f) for o in (0, 2, 3, 4) for f in (0, 1, 2)],
}
_H = (1024, 1030, 1032, 1040, 1056, 1152, 1280, 2048, 2056)


def random_workload(i):
    rng = np.random.default_rng(1000 + i)
    W = int(rng.choice([2, 3, 4, 8]))
    E = W * int(rng.choice([1, 2, 4, 8]))
    Z, C = int(rng.choice([0, 0, 1, 2])), int(rng.choice([0, 0, 1]))
    routing = str(rng.choice(["uniform", "randint", "zipf"]))
    if routing == "zipf":
        Z = C = 0
    n_ids = E + Z + C
    kmax = min(16, E if routing == "zipf" else n_ids)
    K = int(rng.integers(1, kmax + 1))
    BS = int(rng.integers(1, 48))
    H = int(rng.choice(_H))
    mode = int(rng.integers(0, 6))
    variants = [v for v in _VARIANTS[mode] if not (v[0] == 4 and H % 2)]
    out_dtype, scales_kind, scale_format = variants[int(rng.integers(0, len(variants)))]
    mask_kind = int(rng.choice([0, 1, 2]))
    inactive = int(rng.integers(0, BS // 2 + 1)) if mask_kind else 0
    return workloads.Workload(
        f"rand{i}", W=W, E=E, BS=BS, H=H, K=K, quant_mode=mode, zero_expert_num=Z,
        copy_expert_num=C, expert_token_nums_type=int(rng.integers(0, 2)),
        mask_kind=mask_kind, scales_kind=scales_kind, out_dtype=out_dtype,
        scale_format=scale_format, routing=routing, inactive_tokens_per_rank=inactive,
        outlier_prob=float(rng.choice([0.0, 0.02])))


def test_random_configs_are_valid():
    import combine_quant_amd as cq
    for i in range(N_CASES):
        wl = random_workload(i)
        assert cq.moe_dc_validate(harness.lib_cfg(wl)) == cq.MOE_OK, (wl, cq.moe_dc_last_error())


@pytest.mark.parametrize("flags", [0, 1])     # 1: MOE_DC_FLAG_SEPARATE_ROUTE
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config_roundtrip(i, flags):
    wl = random_workload(i)
    harness.roundtrip(wl, seed=i, flags=flags)


# the other two combines over the same random configurations: the int8 block-quantized
# combine (codes and block scales bit for bit, y within tolerance) on even cases, the
# scatter-back combine (with a shared expert's output on every other one) on odd cases
@pytest.mark.parametrize("i", range(0, N_CASES, 2))
def test_random_config_int8_combine(i):
    import test_gpu_combine_quant as combine_quant_tests
    combine_quant_tests._run(random_workload(i), seed=i)


@pytest.mark.parametrize("i", range(1, N_CASES, 2))
def test_random_config_scatter_back(i):
    import test_gpu_combine_scatter as combine_scatter_tests
    combine_scatter_tests._run(random_workload(i), i, with_shared=(i % 4 == 1))


# binary16 tokens (x, expert outputs, shared output and y) over further draws of the same
# law; the routing path alternates with the case number
N_F16 = 40


@pytest.mark.parametrize("i", range(N_CASES, N_CASES + N_F16))
def test_random_config_roundtrip_f16(i):
    harness.roundtrip(random_workload(i).replace(token_dtype=1), seed=i, flags=i % 2)


@pytest.mark.parametrize("i", range(N_CASES, N_CASES + N_F16, 2))
def test_random_config_int8_combine_f16(i):
    import test_gpu_combine_quant as combine_quant_tests
    combine_quant_tests._run(random_workload(i).replace(token_dtype=1), seed=i)


@pytest.mark.parametrize("i", range(N_CASES + 1, N_CASES + N_F16, 2))
def test_random_config_scatter_back_f16(i):
    import test_gpu_combine_scatter as combine_scatter_tests
    combine_scatter_tests._run(random_workload(i).replace(token_dtype=1), i,
                               with_shared=(i % 4 == 1))


# per-expert scales in the two batch ranges of their kernels: past 16,384 picks, where the
# windowed kernel (one workgroup per window of tokens and expert) runs, and from 8,193 to 16,384
# picks, the upper half of the pick kernel's range (one workgroup per pick and expert group);
# ranks, experts, special experts, top-k, batch, row length (ragged ones included), the three
# per-expert modes with their output types, masks and the three routings (repeated ids under
# randint)
N_WINDOW = 24
N_PICK_BAND = 16
_H_WINDOW = (1024, 1032, 1056, 1160, 2048, 2056, 3080)


def _per_expert_workload(name, rng, lo, hi):
    """A per-expert-scales workload with lo < W * BS * K <= hi picks."""
    while True:
        W = int(rng.choice([2, 4, 8, 16, 32]))
        E = min(1024, W * int(rng.choice([1, 2, 4, 8, 16, 32])))
        Z, C = int(rng.choice([0, 0, 1, 2])), int(rng.choice([0, 0, 1]))
        routing = str(rng.choice(["uniform", "randint", "zipf"]))
        if routing == "zipf":
            Z = C = 0
        kmax = min(16, E if routing == "zipf" else E + Z + C)
        K = int(rng.integers(1, kmax + 1))
        bs_min = lo // (W * K) + 1                     # W * BS * K > lo
        bs_max = min(512, bs_min + 96, hi // (W * K))  # W * BS * K <= hi
        if bs_min <= bs_max:
            break
    BS = int(rng.integers(bs_min, bs_max + 1))
    H = int(rng.choice(_H_WINDOW))
    mode = int(rng.choice([1, 2, 3]))
    out_dtype = int(rng.choice({1: [0, 1], 2: [0, 1, 2, 3], 3: [0, 2, 3]}[mode]))
    mask_kind = int(rng.choice([0, 1, 2]))
    inactive = int(rng.integers(0, BS // 4 + 1)) if mask_kind else 0
    return workloads.Workload(
        name, W=W, E=E, BS=BS, H=H, K=K, quant_mode=mode, zero_expert_num=Z,
        copy_expert_num=C, expert_token_nums_type=int(rng.integers(0, 2)),
        mask_kind=mask_kind, scales_kind=3, out_dtype=out_dtype, routing=routing,
        inactive_tokens_per_rank=inactive, outlier_prob=float(rng.choice([0.0, 0.02])))


def random_window_workload(i):
    return _per_expert_workload(f"randwin{i}", np.random.default_rng(5000 + i), 16384, 1 << 30)


def random_pick_band_workload(i):
    return _per_expert_workload(f"randpick{i}", np.random.default_rng(6000 + i), 8192, 16384)


@pytest.mark.parametrize("i", range(N_WINDOW))
def test_random_window_config_roundtrip(i):
    wl = random_window_workload(i)
    assert wl.W * wl.BS * wl.K > 16384
    harness.roundtrip(wl, seed=i, flags=i % 2)


@pytest.mark.parametrize("i", range(N_PICK_BAND))
def test_random_pick_band_config_roundtrip(i):
    wl = random_pick_band_workload(i)
    assert 8192 < wl.W * wl.BS * wl.K <= 16384
    harness.roundtrip(wl, seed=i, flags=i % 2)
