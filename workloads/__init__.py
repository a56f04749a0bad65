"""Seeded synthetic inputs for MoE dispatch/combine.

This module is shared by the tests, the bench and the smoke check; it holds only input
generation (random draws, bf16 rounding of the draws, softmax of the routing logits) and none
of the dispatch/combine arithmetic, so neither the oracle nor the HIP path depends on the
other through it.

The pages measure only on random synthetic data (the sample's data generator draws random
tokens and routing); there is no public dataset to stand in for.  Workloads below follow the
shapes the pages work with: H up to 8192, BS <= 512 tokens per rank, K <= 16 and
DeepSeek-V3-style 256-expert routing.

Recipe (numpy PCG64, one spawned sub-stream per tensor, base seed 0 by default):
  x              bf16 (or binary16 for a workload with token_dtype 1) of N(0,1) fp32
                 samples (round to nearest even); optional outliers:
                 each value independently x10 with the workload's probability.  At the
                 largest sizes x is drawn on the device with torch's seeded generator
                 instead (x_torch)
  expert_ids     uniform: K distinct ids per token, in the order of a uniform random
                 permutation; zipf: K distinct ids drawn one after another without
                 replacement with probability proportional to 1/rank^s over a seeded
                 permutation of the experts (drawn with the Gumbel top-K construction,
                 which has exactly that sequential law); randint: K independent uniform ids
                 (duplicates allowed)
  scales         the quantization scales tensor: shape (1,), (H,) or (E, H) for scales
                 kinds 1, 2, 3; fp32 U(0.5, 1.5) as smooth scales (modes 2, 3), U(16, 48) as
                 static int8 coefficients (mode 1: about 127 / max|x| of an N(0,1) row, so
                 the largest elements of a row saturate)
  mask           none; per token [W][BS]; or per pick [W][BS][K] with a fixed number of
                 tokens per rank fully inactive (seeded choice)
  expert_scales  fp32 softmax of N(0,1) logits over each token's K picks
  expert_out     bf16 (or binary16) of N(0,1) fp32 samples, one row per received row
  shared_x       bf16 of N(0,1) fp32 samples [W][BS][H] (the shared expert's output, drawn
                 on the device like expert_out)
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

# sub-stream slots of SeedSequence(seed).spawn(N_STREAMS)
_X, _IDS, _SMOOTH, _MASK, _WEIGHTS, _EXPERT_OUT, _OUTLIER, _SPARE = range(8)
N_STREAMS = 8


@dataclass(frozen=True)
class Workload:
    name: str
    W: int                      # logical EP ranks
    E: int                      # routed experts
    BS: int                     # tokens per rank
    H: int                      # hidden size
    K: int                      # picks per token
    quant_mode: int             # 0..5
    zero_expert_num: int = 0
    copy_expert_num: int = 0
    expert_token_nums_type: int = 1
    mask_kind: int = 0          # 0 none, 1 per token, 2 per pick
    scales_kind: int = 0        # 0 none, 1 scalar, 2 shared row (H,), 3 per expert (E, H)
    out_dtype: int = 0          # 0 the mode's default, 1 int8, 2 E4M3, 3 E5M2
    scale_format: int = 0       # MX modes: 0 fp32 2^se, 1 E8M0 bytes, 2 fp32 2^-se
    combine_quant: int = 0      # 0 bf16 expert rows, 1 int8 blocks of 8 on the return path
    combine_path: str = "gather"  # gather (expand_idx addressing) | scatter (assist_info
                                  # triples, with a shared expert's output added)
    routing: str = "uniform"    # uniform | zipf | randint
    zipf_s: float = 1.2
    outlier_prob: float = 0.0
    inactive_tokens_per_rank: int = 0
    token_dtype: int = 0        # token elements: 0 bf16, 1 IEEE binary16
    description: str = ""

    @property
    def L(self) -> int:
        return self.E // self.W

    @property
    def T(self) -> int:
        return self.W * self.BS

    @property
    def n_ids(self) -> int:
        return self.E + self.zero_expert_num + self.copy_expert_num

    @property
    def cap(self) -> int:
        """Rows that always suffice for the packed expand_x (every pick routed)."""
        return self.W * self.BS * self.K

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


C1_MODE0 = Workload(
    "c1_tiny_mode0", W=2, E=8, BS=16, H=1024, K=2, quant_mode=0,
    description="tiny: W=2, E=8 (L=4), BS=16, H=1024, K=2, bf16 N(0,1), uniform distinct "
                "top-2, no quantization, softmax weights")
C1_MODE2 = C1_MODE0.replace(
    name="c1_tiny_mode2", quant_mode=2,
    description="tiny: W=2, E=8 (L=4), BS=16, H=1024, K=2, int8 per-token quant without "
                "smooth scales")
C2 = Workload(
    "c2_w8_smooth", W=8, E=256, BS=128, H=7168, K=8, quant_mode=2, scales_kind=3,
    outlier_prob=0.01, expert_token_nums_type=0,
    description="W=8, E=256 (L=32), BS=128, H=7168, K=8, bf16 N(0,1) with 1% of values x10, "
                "int8 per-token quant with per-expert smooth scales U(0.5,1.5), uniform "
                "distinct top-8")
C3 = Workload(
    "c3_w16_mxfp8_zipf", W=16, E=256, BS=512, H=7168, K=8, quant_mode=4, routing="zipf",
    description="W=16, E=256 (L=16), BS=512, H=7168, K=8, bf16 N(0,1), MX E4M3 32-element "
                "blocks, Zipf(1.2) routing over a seeded expert permutation")
C4 = Workload(
    "c4_w16_int8_roundtrip", W=16, E=256, BS=512, H=7168, K=8, quant_mode=2,
    description="W=16, E=256 (L=16), BS=512, H=7168, K=8, bf16 N(0,1), int8 per-token quant "
                "(no smooth), uniform distinct top-8; combine reads bf16 N(0,1) expert "
                "outputs per received row")
C5 = Workload(
    "c5_w32_mxclip_special", W=32, E=512, BS=512, H=8192, K=16, quant_mode=5,
    zero_expert_num=2, copy_expert_num=2, mask_kind=2, inactive_tokens_per_rank=51,
    description="W=32, E=512 (L=16) + 2 zero + 2 copy experts, BS=512, H=8192, K=16, bf16 "
                "N(0,1), MX clip E4M3, per-pick mask with 51 of 512 tokens per rank fully "
                "inactive, uniform distinct top-16 over all 516 ids")

# the further quantization variants at the C3/C4 shape (measurement of those variants)
C3_E5M2_E8M0 = C3.replace(
    name="c3v_w16_mx_e5m2_e8m0", out_dtype=3, scale_format=1,
    description="C3 with MX E5M2 elements and E8M0 scale bytes (the SMP article's stored "
                "format)")
C3_MXFP4 = C3.replace(
    name="c3v_w16_mxfp4_e8m0", out_dtype=4, scale_format=1,
    description="C3 with MX E2M1 (fp4) elements, two per byte, and E8M0 scale bytes")
C4_STATIC = C4.replace(
    name="c4v_w16_static_int8_shared", quant_mode=1, scales_kind=2,
    description="C4 with static int8 quantization, one shared [H] coefficient row "
                "U(16, 48)")
C4_TOKEN_E4M3 = C4.replace(
    name="c4v_w16_token_e4m3", out_dtype=2,
    description="C4 with per-token dynamic E4M3 codes")
C4_GROUP = C4.replace(
    name="c4v_w16_group_e4m3", quant_mode=3,
    description="C4 with per-128-group dynamic E4M3 codes (56 scales per row)")
C2_GROUP_SMOOTH = C2.replace(
    name="c2v_w8_group_e4m3_smooth", quant_mode=3,
    description="C2 with per-128-group dynamic E4M3 codes and per-expert smooth scales")

C4_SMOOTH = C4.replace(
    name="c4v_w16_smooth", scales_kind=3,
    description="C4 with per-expert smooth scales U(0.5, 1.5) [256][7168] (per-pick int8 "
                "quantization)")
C4_COMBINE_INT8 = C4.replace(
    name="c4v_w16_combine_int8", combine_quant=1,
    description="C4 with the combine-side int8 block quantization: the expert outputs are "
                "coded as int8 with one fp32 scale per 8 elements, then combined")

C4_SCATTER_SHARED = C4.replace(
    name="c4v_w16_scatter_back_shared", combine_path="scatter",
    description="C4 with the scatter-back combine (rows return by their source triples) "
                "and a shared expert's bf16 N(0,1) output added to every token")

# the shapes of the sample article's performance table (性能数据): 8 ranks with 4 experts each,
# H=7168, K=8, BS 8 or 256; non-quantized, or MXFP8 (E5M2 codes, E8M0 scales) dispatch with the
# int8 block-quantized combine.  Here all 8 ranks run on one GPU.
SAMPLE_BS8 = Workload(
    "sample_w8_bs8_bf16", W=8, E=32, BS=8, H=7168, K=8, quant_mode=0,
    description="the sample table's low-latency shape: 8 ranks x 4 experts, BS=8, H=7168, "
                "K=8, no quantization")
SAMPLE_BS8_Q = SAMPLE_BS8.replace(
    name="sample_w8_bs8_mxfp8_cint8", quant_mode=4, out_dtype=3, scale_format=1,
    combine_quant=1,
    description="the sample table's low-latency shape with MXFP8 (E5M2 + E8M0) dispatch and "
                "the int8 block-quantized combine")
SAMPLE_BS256 = SAMPLE_BS8.replace(
    name="sample_w8_bs256_bf16", BS=256,
    description="the sample table's throughput shape: 8 ranks x 4 experts, BS=256, H=7168, "
                "K=8, no quantization")
SAMPLE_BS256_Q = SAMPLE_BS8_Q.replace(
    name="sample_w8_bs256_mxfp8_cint8", BS=256,
    description="the sample table's throughput shape with MXFP8 (E5M2 + E8M0) dispatch and "
                "the int8 block-quantized combine")

C4_F16 = C4.replace(
    name="c4v_w16_f16_tokens", token_dtype=1,
    description="C4 with IEEE binary16 tokens (x, expert outputs and y in fp16)")

# the widest count matrix the library accepts (768 ranks x 768 experts: 589,824 (expert,
# source) counts, which the receive-side scan takes in chunks) with small rows, to time the
# routing and scan steps at that width
W768_SCAN = Workload(
    "w768_e768_scan", W=768, E=768, BS=16, H=1024, K=4, quant_mode=2,
    description="W=768 ranks, E=768 experts (one per rank), BS=16, H=1024, K=4, int8 per "
                "token: the largest count matrix, for the routing and chunked scan steps")

WORKLOADS = {w.name: w for w in (C1_MODE0, C1_MODE2, C2, C3, C4, C5, C3_E5M2_E8M0, C4_STATIC,
                                 C4_TOKEN_E4M3, C4_GROUP, C2_GROUP_SMOOTH, C4_COMBINE_INT8,
                                 C4_SCATTER_SHARED, C4_SMOOTH, SAMPLE_BS8, SAMPLE_BS8_Q,
                                 SAMPLE_BS256, SAMPLE_BS256_Q, C3_MXFP4, C4_F16, W768_SCAN)}


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(N_STREAMS)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 bit patterns (nearest, ties to even); inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 samples to binary16 bit patterns (numpy's cast: nearest, ties to even)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def tok_bits_to_f32(b: np.ndarray, token_dtype: int) -> np.ndarray:
    """Token bit patterns (bf16, or binary16 when token_dtype is 1) widened to fp32."""
    return f16_bits_to_f32(b) if token_dtype == 1 else bf16_bits_to_f32(b)


def f32_to_tok_bits(a: np.ndarray, token_dtype: int) -> np.ndarray:
    return f32_to_f16_bits(a) if token_dtype == 1 else f32_to_bf16_bits(a)


def _normal_tok(rng, shape, token_dtype, chunk=1 << 24) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        out[lo:hi] = f32_to_tok_bits(rng.standard_normal(hi - lo, dtype=np.float32), token_dtype)
    return out.reshape(shape)


def _normal_bf16(rng, shape, chunk=1 << 24) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))
    return out.reshape(shape)


def _topk_keys(keys: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest keys per row, largest first."""
    part = np.argpartition(-keys, K - 1, axis=1)[:, :K]
    order = np.argsort(-np.take_along_axis(keys, part, axis=1), axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


def gen_expert_ids(wl: Workload, rng) -> np.ndarray:
    T, K, n = wl.T, wl.K, wl.n_ids
    if wl.routing == "randint":
        ids = rng.integers(0, n, size=(T, K), dtype=np.int64)
    elif wl.routing == "uniform":
        ids = np.empty((T, K), np.int64)
        step = max(1, (1 << 22) // n)
        for lo in range(0, T, step):
            hi = min(T, lo + step)
            ids[lo:hi] = _topk_keys(rng.random((hi - lo, n)), K)
    elif wl.routing == "zipf":
        if wl.zero_expert_num or wl.copy_expert_num:
            raise ValueError("zipf routing is defined over routed experts only")
        perm = rng.permutation(wl.E)                 # perm[rank-1] = expert id
        logw = np.empty(wl.E)
        logw[perm] = -wl.zipf_s * np.log(np.arange(1, wl.E + 1, dtype=np.float64))
        ids = np.empty((T, K), np.int64)
        step = max(1, (1 << 22) // wl.E)
        for lo in range(0, T, step):
            hi = min(T, lo + step)
            g = rng.gumbel(size=(hi - lo, wl.E))
            ids[lo:hi] = _topk_keys(logw[None, :] + g, K)
    else:
        raise ValueError(f"unknown routing {wl.routing!r}")
    return ids.astype(np.int32).reshape(wl.W, wl.BS, K)


def gen_mask(wl: Workload, rng):
    if wl.mask_kind == 0:
        return None
    if wl.mask_kind == 1:
        # per token, trues before falses within each rank
        m = np.ones((wl.W, wl.BS), np.uint8)
        n_off = wl.inactive_tokens_per_rank
        if n_off:
            m[:, wl.BS - n_off:] = 0
        return m
    m = np.ones((wl.W, wl.BS, wl.K), np.uint8)
    for s in range(wl.W):
        off = rng.choice(wl.BS, size=wl.inactive_tokens_per_rank, replace=False)
        m[s, off, :] = 0
    return m


def gen_expert_scales(wl: Workload, rng) -> np.ndarray:
    logits = rng.standard_normal((wl.T, wl.K), dtype=np.float32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return w.reshape(wl.W, wl.BS, wl.K)


def gen_scales(wl: Workload, rng):
    if wl.scales_kind == 0:
        return None
    shape = {1: (1,), 2: (wl.H,), 3: (wl.E, wl.H)}[wl.scales_kind]
    lo, hi = (16.0, 48.0) if wl.quant_mode == 1 else (0.5, 1.5)
    return rng.uniform(lo, hi, shape).astype(np.float32)


def generate(wl: Workload, seed: int = 0, expert_out_rows: int | None = None) -> dict:
    """All host inputs of one dispatch+combine round trip.

    expert_out is generated only when expert_out_rows is given (it can be large)."""
    st = _streams(seed)
    x = _normal_tok(st[_X], (wl.W, wl.BS, wl.H), wl.token_dtype)
    if wl.outlier_prob > 0:
        hit = st[_OUTLIER].random((wl.W, wl.BS, wl.H)) < wl.outlier_prob
        xf = tok_bits_to_f32(x, wl.token_dtype)
        xf[hit] *= np.float32(10.0)
        x = f32_to_tok_bits(xf, wl.token_dtype)
    out = dict(x=x, **generate_routing(wl, seed))
    if expert_out_rows is not None:
        out["expert_out"] = _normal_tok(st[_EXPERT_OUT], (expert_out_rows, wl.H), wl.token_dtype)
    return out


def generate_routing(wl: Workload, seed: int = 0) -> dict:
    """Every host input of generate() except x (each tensor has its own sub-stream, so the
    values are the same as generate()'s)."""
    st = _streams(seed)
    return dict(
        expert_ids=gen_expert_ids(wl, st[_IDS]),
        mask=gen_mask(wl, st[_MASK]),
        expert_scales=gen_expert_scales(wl, st[_WEIGHTS]),
        scales=gen_scales(wl, st[_SMOOTH]),
    )


def _torch_token_dtype(wl: Workload):
    import torch
    return torch.float16 if wl.token_dtype == 1 else torch.bfloat16


def x_torch(wl: Workload, seed: int = 0, device="cuda"):
    """bf16 N(0,1) tokens [W][BS][H] drawn on the device with torch's seeded generator, for
    sizes where the numpy draw would take minutes (no outliers).  The oracle reads the host
    copy of the same bytes."""
    import torch
    if wl.outlier_prob > 0:
        raise ValueError("x_torch draws no outliers")
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(seed).spawn(N_STREAMS)[_X].generate_state(1)[0]))
    x = torch.empty((wl.W, wl.BS, wl.H), dtype=_torch_token_dtype(wl), device=device)
    for s in range(wl.W):            # one rank at a time: a small fp32 temporary
        x[s] = torch.randn((wl.BS, wl.H), generator=g, device=device,
                           dtype=torch.float32).to(_torch_token_dtype(wl))
    return x


def expert_out_torch(wl: Workload, rows: int, seed: int = 0, device="cuda"):
    """bf16 N(0,1) expert outputs drawn on the device with torch's seeded generator.

    Used where the numpy draw of a multi-GB buffer would dominate a run; the values are
    still a pure function of (seed, rows, H), and the host copy of the same bytes is what
    the oracle reads."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(seed).spawn(N_STREAMS)[_EXPERT_OUT]
                      .generate_state(1)[0]))
    return torch.randn((rows, wl.H), generator=g, device=device,
                       dtype=torch.float32).to(_torch_token_dtype(wl))
