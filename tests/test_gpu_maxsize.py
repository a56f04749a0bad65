"""GPU parity at the largest configuration the library accepts: W = 768 ranks, E = 768
experts (one per rank), BS = 512 tokens per rank, K = 16 distinct picks, H = 8192.  That is
393,216 source tokens and 6,291,456 routed rows, so packed-row element offsets reach 5.2e10
(far past 2^32) and unquantized rows fill 103 GB of HBM.

In the library's normal launch configuration:
  * routing outputs (expand_idx, ep_recv_count, expert_token_nums, recv_offsets) in full
    against the oracle;
  * the packed layout whole, as a property that holds at any size: read in row order,
    assist_info visits every routed pick exactly once, in strictly increasing (expert,
    source rank, token, pick) order -- the stable sort that defines the packed order;
  * payload rows of sampled tokens (including the picks that land in the first and the last
    row) against the oracle, one row at a time: unquantized copies, int8 per-token codes,
    int8 codes with per-expert smooth scales [768][8192] (one workgroup per window of tokens
    and expert) and MXFP4 clip codes with E8M0 scales;
  * combine over the unquantized packed rows (an identity expert): sampled tokens against
    the oracle, and every token against the k-ordered fp32 weighted sum of its own row
    within the combine tolerance.
x is drawn on the device with torch's seeded generator; the oracle reads the host copies of
the sampled rows.
"""
import os

import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

MAX = workloads.Workload("max_w768_e768_bs512_k16_h8192", W=768, E=768, BS=512, H=8192,
                         K=16, quant_mode=0)
N_SAMPLE = 40
# x + unquantized packed rows + y, with room for the check's temporaries
NEED_BYTES = 130 * 10**9


@pytest.fixture(scope="module")
def max_case():
    import torch
    torch.cuda.empty_cache()                      # blocks cached by earlier tests
    free, _ = torch.cuda.mem_get_info()
    if free < NEED_BYTES:
        pytest.skip(f"needs {NEED_BYTES / 1e9:.0f} GB of free device memory, "
                    f"{free / 1e9:.0f} GB free")
    wl = MAX
    r = workloads.generate_routing(wl, seed=0)
    ids = r["expert_ids"]
    ocfg = harness.oracle_cfg(wl)
    cnt, eidx = oracle.route(ocfg, ids)
    erc, etn, off = oracle.recv_counts(ocfg, cnt)
    # sampled tokens, plus the tokens whose picks land in the first and the last packed row
    # (the smallest and the largest (expert, rank, token, pick) key)
    rng = np.random.default_rng(77)
    flat = set(int(f) for f in rng.choice(wl.T, size=N_SAMPLE, replace=False))
    first = np.argwhere(ids.reshape(wl.T, wl.K) == 0)[0]
    last = np.argwhere(ids.reshape(wl.T, wl.K) == wl.E - 1)[-1]
    flat |= {int(first[0]), int(last[0])}
    tokens = [(f // wl.BS, f % wl.BS) for f in sorted(flat)]
    case = dict(
        wl=wl, ids=ids, w=r["expert_scales"], ocfg=ocfg, eidx=eidx, erc=erc, etn=etn,
        off=off, tokens=tokens,
        x=workloads.x_torch(wl, seed=0),
        ids_dev=harness.to_dev(ids), w_dev=harness.to_dev(r["expert_scales"]))
    tok_t = torch.tensor([s * wl.BS + i for s, i in tokens], dtype=torch.long, device="cuda")
    case["x_rows"] = harness.host(case["x"].view(wl.T, wl.H).index_select(0, tok_t))
    case["tok_t"] = tok_t
    yield case
    case.clear()
    torch.cuda.empty_cache()


def _picks(c):
    """(sample index, s, i, k, e, oracle row) of every pick of the sampled tokens."""
    out = []
    for n, (s, i) in enumerate(c["tokens"]):
        for k in range(c["wl"].K):
            e = int(c["ids"][s, i, k])
            row = int(oracle.dest_row(c["ocfg"], c["erc"], c["off"], s, e,
                                      int(c["eidx"][s, i, k])))
            out.append((n, s, i, k, e, row))
    return out


def _dispatch_and_check_routing(c, wl, scales=None):
    import torch
    import combine_quant_amd as cq
    cfg = harness.lib_cfg(wl)
    out = cq.dispatch(cfg, c["x"], c["ids_dev"], scales)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(harness.host(out["expand_idx"]), c["eidx"])
    np.testing.assert_array_equal(harness.host(out["ep_recv_count"]), c["erc"])
    np.testing.assert_array_equal(harness.host(out["expert_token_nums"]), c["etn"])
    np.testing.assert_array_equal(harness.host(out["recv_offsets"]), c["off"])
    return cfg, out


def test_max_dispatch_layout_and_unquantized_rows(max_case, tmp_path):
    import torch
    import combine_quant_amd as cq
    c = max_case
    wl = c["wl"]
    cfg, out = _dispatch_and_check_routing(c, wl)
    P = int(c["off"][-1])
    assert P == wl.cap                              # distinct ids, no mask: every pick routed

    # the whole packed layout through assist_info
    ai = harness.host(out["assist_info"]).astype(np.int64)
    s_, i_, k_ = ai[:, 0], ai[:, 1], ai[:, 2]
    assert ((s_ >= 0) & (s_ < wl.W) & (i_ >= 0) & (i_ < wl.BS) & (k_ >= 0)
            & (k_ < wl.K)).all()
    e_ = c["ids"][s_, i_, k_].astype(np.int64)
    key = ((e_ * wl.W + s_) * wl.BS + i_) * wl.K + k_
    assert (np.diff(key) > 0).all()
    del ai, s_, i_, k_, e_, key

    # payload rows of the sampled tokens: copies of their token rows, at the oracle's rows
    picks = _picks(c)
    assert max(p[5] for p in picks) == P - 1 and min(p[5] for p in picks) == 0
    rows_t = torch.tensor([p[5] for p in picks], dtype=torch.long, device="cuda")
    ex = harness.host(out["expand_x"].index_select(0, rows_t))
    for m, (n, s, i, k, e, row) in enumerate(picks):
        assert (ex[m] == c["x_rows"][n]).all(), (s, i, k, row)     # mode 0: bit copy

    # combine with the packed rows themselves as the expert outputs
    y = cq.combine(cfg, out["expand_x"], c["ids_dev"], out["expand_idx"], c["w_dev"],
                   out["ep_recv_count"], out["recv_offsets"])
    torch.cuda.synchronize()
    # the oracle reads only the sampled tokens' rows: a sparse file-backed buffer holding
    # exactly those rows (a 103 GB host array is not needed)
    eo_host = np.memmap(os.path.join(tmp_path, "expert_out.bin"), dtype=np.uint16, mode="w+",
                        shape=(wl.cap, wl.H))
    for m, p in enumerate(picks):
        eo_host[p[5]] = ex[m]
    y_s = harness.host(y.view(wl.T, wl.H).index_select(0, c["tok_t"]))
    for n, (s, i) in enumerate(c["tokens"]):
        want = oracle.combine_token(c["ocfg"], eo_host, c["ids"], c["eidx"], c["w"], c["erc"],
                                    c["off"], s, i)
        assert harness.check_combine_tolerance(y_s[n], want) == 0, (s, i)
    del eo_host

    # every token: y against the k-ordered fp32 sum of w_k * x (its rows are copies of x)
    xv, yv = c["x"].view(wl.T, wl.H), y.view(wl.T, wl.H)
    wv = c["w_dev"].view(wl.T, wl.K)
    chunk = 16384
    for lo in range(0, wl.T, chunk):
        xf = xv[lo:lo + chunk].float()
        acc = torch.zeros_like(xf)
        for k in range(wl.K):
            acc = acc + wv[lo:lo + chunk, k:k + 1] * xf
        ref = acc.to(torch.bfloat16).float()
        err = (yv[lo:lo + chunk].float() - ref).abs()
        assert bool((err <= 1e-3 + 1e-2 * ref.abs()).all()), lo


@pytest.mark.parametrize("variant", ["int8_per_token", "mxfp4_clip_e8m0",
                                     "int8_per_expert_scales"])
def test_max_dispatch_quantized_rows(max_case, variant):
    import torch
    c = max_case
    wl = {"int8_per_token": c["wl"].replace(quant_mode=2),
          "mxfp4_clip_e8m0": c["wl"].replace(quant_mode=5, out_dtype=4,
                                             scale_format=1),
          # per-expert smooth scales [768][8192]: 1,536 windows of 256 tokens, one workgroup
          # per (window, expert)
          "int8_per_expert_scales": c["wl"].replace(quant_mode=2, scales_kind=3)}[variant]
    sm = None
    if wl.scales_kind == 3:
        r = workloads.generate_routing(wl, seed=0)
        assert (r["expert_ids"] == c["ids"]).all()
        sm = r["scales"]
    cfg, out = _dispatch_and_check_routing(c, wl, harness.to_dev(sm))
    picks = _picks(c)
    rows_t = torch.tensor([p[5] for p in picks], dtype=torch.long, device="cuda")
    ex = harness.host(out["expand_x"].index_select(0, rows_t))
    ds = harness.host(out["dynamic_scales"].index_select(0, rows_t))
    ai = harness.host(out["assist_info"].index_select(0, rows_t))
    nb = (wl.H + 31) // 32
    for m, (n, s, i, k, e, row) in enumerate(picks):
        assert tuple(ai[m]) == (s, i, k)
        q, sc = oracle.quant_row(wl.quant_mode, c["x_rows"][n], None if sm is None else sm[e],
                                 wl.out_dtype)
        assert (ex[m].view(np.uint8) == q.view(np.uint8)).all(), (s, i, k, row)
        if wl.scale_format == 1:
            want = [oracle.e8m0_from_scale(v) for v in sc[:nb]] + [0] * (len(sc) - nb)
            assert ds[m].tolist() == want, (s, i, k, row)
        else:
            assert (np.atleast_1d(ds[m]).view(np.uint32)
                    == np.atleast_1d(sc).view(np.uint32)).all(), (s, i, k, row)
