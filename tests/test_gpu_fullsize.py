"""GPU parity at the full workload sizes, in the library's normal launch configuration.

Routing outputs (expand_idx, ep_recv_count, expert_token_nums, recv_offsets) are compared in
full; payload rows and combine outputs on a seeded sample of source tokens, each recomputed
one by one by the oracle; the packed layout is checked whole through assist_info.
"""
import numpy as np
import pytest

import harness
import oracle
import workloads

pytestmark = pytest.mark.gpu

N_SAMPLE = 192


def _sample_tokens(wl, seed=123):
    rng = np.random.default_rng(seed)
    flat = rng.choice(wl.T, size=min(N_SAMPLE, wl.T), replace=False)
    return [(int(f) // wl.BS, int(f) % wl.BS) for f in np.sort(flat)]


def _rows_for(ocfg, wl, inp, eidx, erc, off, tokens):
    out = []
    for s, i in tokens:
        for k in range(wl.K):
            o = int(eidx[s, i, k])
            if o >= 0:
                e = int(inp["expert_ids"][s, i, k])
                out.append((s, i, k, e, int(oracle.dest_row(ocfg, erc, off, s, e, o))))
    return out


@pytest.mark.parametrize("name", ["c3_w16_mxfp8_zipf", "c4_w16_int8_roundtrip",
                                  "c5_w32_mxclip_special"])
def test_fullsize_dispatch_and_combine(name):
    import torch
    import combine_quant_amd as cq
    wl = workloads.WORKLOADS[name]
    inp = workloads.generate(wl, seed=0)
    ocfg = harness.oracle_cfg(wl)
    cnt, eidx = oracle.route(ocfg, inp["expert_ids"], inp.get("mask"))
    erc, etn, off = oracle.recv_counts(ocfg, cnt)
    P = int(off[-1])

    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(harness.host(out["expand_idx"]), eidx)
    np.testing.assert_array_equal(harness.host(out["ep_recv_count"]), erc)
    np.testing.assert_array_equal(harness.host(out["expert_token_nums"]), etn)
    np.testing.assert_array_equal(harness.host(out["recv_offsets"]), off)

    # the whole packed layout: every row holds the triple of the pick whose row it is
    ai = harness.host(out["assist_info"][:P])
    seen = np.zeros(P, bool)
    ids = inp["expert_ids"]
    for s in range(wl.W):
        for i in range(wl.BS):
            for k in range(wl.K):
                o = int(eidx[s, i, k])
                if o < 0:
                    continue
                row = int(oracle.dest_row(ocfg, erc, off, s, int(ids[s, i, k]), o))
                assert tuple(ai[row]) == (s, i, k)
                seen[row] = True
    assert seen.all()

    # payload rows of sampled tokens, recomputed by the oracle row by row
    tokens = _sample_tokens(wl)
    picks = _rows_for(ocfg, wl, inp, eidx, erc, off, tokens)
    rows_t = torch.tensor([p[4] for p in picks], dtype=torch.long, device="cuda")
    ex = harness.host(out["expand_x"].index_select(0, rows_t))
    sc = harness.host(out["dynamic_scales"].index_select(0, rows_t))
    for n, (s, i, k, e, row) in enumerate(picks):
        xr = inp["x"][s, i]
        if wl.quant_mode == 2:
            q, scale = oracle.quant_int8_row(xr, None if inp["scales"] is None
                                             else inp["scales"][e])
            assert (ex[n] == q).all(), (s, i, k)
            assert np.float32(sc[n]).view(np.uint32) == np.float32(scale).view(np.uint32)
        else:
            c, scales = oracle.quant_mx_row(xr, wl.quant_mode == 5)
            assert (ex[n] == c).all(), (s, i, k)
            assert (sc[n].view(np.uint32) == scales.view(np.uint32)).all(), (s, i, k)

    # combine on bf16 N(0,1) expert outputs drawn on the device, one per packed row
    eo = workloads.expert_out_torch(wl, wl.cap, seed=0)
    w_dev = harness.to_dev(inp["expert_scales"])
    y = cq.combine(cfg, eo, dev_in["ids"], out["expand_idx"], w_dev, out["ep_recv_count"],
                   out["recv_offsets"], dev_in["mask"], dev_in["x"])
    torch.cuda.synchronize()
    # the oracle reads only the rows of the sampled tokens: a lazily zeroed host buffer
    # filled with exactly those rows
    eo_host = np.zeros((wl.cap, wl.H), np.uint16)
    eo_host[rows_t.cpu().numpy()] = harness.host(eo.index_select(0, rows_t))
    tok_t = torch.tensor([s * wl.BS + i for s, i in tokens], dtype=torch.long, device="cuda")
    y_s = harness.host(y.view(wl.T, wl.H).index_select(0, tok_t))
    ndiff = 0
    for n, (s, i) in enumerate(tokens):
        y_ref = oracle.combine_token(ocfg, eo_host, ids, eidx, inp["expert_scales"], erc, off,
                                     s, i, mask=inp.get("mask"), ori_x=inp["x"])
        ndiff += harness.check_combine_tolerance(y_s[n], y_ref)
    assert ndiff == 0


def test_c4_identity_dequant_roundtrip_fullsize():
    """Full dispatch (int8) -> identity-dequant expert (bf16(q*scale)) -> combine, at full
    size: sampled tokens against the oracle's own round trip, and every token against the
    fp32 weighted sum of x within the int8 quantization bound."""
    import torch
    import combine_quant_amd as cq
    wl = workloads.C4
    inp = workloads.generate(wl, seed=0)
    ocfg = harness.oracle_cfg(wl)
    cfg, dev_in, out = harness.gpu_dispatch(wl, inp)
    eo = (out["expand_x"].float() * out["dynamic_scales"][:, None]).to(torch.bfloat16)
    w_dev = harness.to_dev(inp["expert_scales"])
    y = cq.combine(cfg, eo, dev_in["ids"], out["expand_idx"], w_dev, out["ep_recv_count"],
                   out["recv_offsets"])
    # property at any size: y ~ sum_k w_k x within half an int8 step + bf16 roundings
    xf = dev_in["x"].float()
    wsum = w_dev.sum(dim=2, keepdim=True)
    amax = xf.abs().amax(dim=2, keepdim=True)
    err = (y.float() - wsum * xf).abs()
    bound = 0.5 * amax / 127 + xf.abs() * 2.0 ** -7 + amax * 2.0 ** -8
    assert bool((err <= bound).all())
    torch.cuda.synchronize()
    # sampled tokens against the oracle's own round trip
    cnt, eidx = oracle.route(ocfg, inp["expert_ids"])
    erc, etn, off = oracle.recv_counts(ocfg, cnt)
    tokens = _sample_tokens(wl, seed=7)
    eo_host = np.zeros((wl.cap, wl.H), np.uint16)
    for (s, i, k, e, row) in _rows_for(ocfg, wl, inp, eidx, erc, off, tokens):
        q, scale = oracle.quant_int8_row(inp["x"][s, i])
        eo_host[row] = workloads.f32_to_bf16_bits(q.astype(np.float32) * np.float32(scale))
    tok_t = torch.tensor([s * wl.BS + i for s, i in tokens], dtype=torch.long, device="cuda")
    y_s = harness.host(y.view(wl.T, wl.H).index_select(0, tok_t))
    for n, (s, i) in enumerate(tokens):
        y_ref = oracle.combine_token(ocfg, eo_host, inp["expert_ids"], eidx,
                                     inp["expert_scales"], erc, off, s, i)
        assert harness.check_combine_tolerance(y_s[n], y_ref) == 0
