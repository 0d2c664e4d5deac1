"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every output element; they span several key tiles and
chunks, ragged tails, and the degenerate cases (empty history, chunks beyond
a request's end, one-token history). Full-size cases run the verification
workloads in the launch configuration the benchmark times and compare sampled
(request, KV head) slices, which the oracle computes one at a time.

Tolerances (max-abs on O and on lse): 2e-3 for bf16 inputs, 1e-5 for fp32.
Masks compare bit for bit.
"""

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_speculative_amd import rounds
from long_context_speculative_amd import ssverify as ss
from long_context_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}
C = wl.CONFIGS

SMALL = {
    "c1": C["c1_tiny_f32"],
    "c2_small": C["c2_qwen3_8b"].with_(batch=2, hist_len=4500, chunk_len=1024),
    "c3_small": C["c3_internlm25_7b_ragged"].with_(batch=6, hist_len=3000, ragged_lo=1, chunk_len=512),
    "c3_small_token": C["c3_internlm25_7b_ragged"].with_(batch=6, hist_len=3000, ragged_lo=1, chunk_len=512,
                                                         packing="token"),
    "c4_small": C["c4_tree_72b"].with_(batch=2, hist_len=1500, chunk_len=512),
    "c5_small": C["c5_streamed"].with_(batch=2, hist_len=2048, chunk_len=512),
    "f32_g8_tree": C["c4_tree_72b"].with_(batch=1, hist_len=700, chunk_len=128, dtype="f32", n_queries=20),
    "bf16_d64": C["c2_qwen3_8b"].with_(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, hist_len=333,
                                       chunk_len=100),
    "bf16_small_rows": C["c2_qwen3_8b"].with_(batch=3, n_queries=2, hist_len=1000, chunk_len=256),
    # small-row VALU kernel: 4, 12 and 15 rows, ragged
    "valu_r4": C["c2_qwen3_8b"].with_(batch=2, n_queries=1, hist_len=777, chunk_len=200),
    "valu_r12_ragged": C["c3_internlm25_7b_ragged"].with_(batch=4, n_queries=3, hist_len=1500, ragged_lo=1,
                                                          chunk_len=300),
    "valu_r15": C["c2_qwen3_8b"].with_(batch=2, n_q_heads=15, n_kv_heads=5, n_queries=5, hist_len=1000,
                                       chunk_len=512),
    "bf16_rows16": C["c2_qwen3_8b"].with_(batch=3, n_queries=4, hist_len=2100, chunk_len=700),
    "bf16_rows32_g8": C["c4_tree_72b"].with_(batch=2, n_queries=4, hist_len=1337, chunk_len=512),
    # wide-row MFMA kernel: one wave (64 rows), two waves, four with one idle,
    # two row groups with the second mostly idle
    "wide_r64": C["c2_qwen3_8b"].with_(batch=2, n_queries=16, hist_len=1500, chunk_len=512),
    "wide_r96_ragged": C["c3_internlm25_7b_ragged"].with_(batch=5, n_queries=24, hist_len=2000, ragged_lo=1,
                                                           chunk_len=300),
    "wide_r192_tree": C["c4_tree_72b"].with_(batch=2, n_queries=24, hist_len=999, chunk_len=256),
    "wide_r320_tree": C["c4_tree_72b"].with_(batch=1, n_queries=40, hist_len=1200, chunk_len=1000),
    # other GQA group sizes: one query head per KV head (plain multi-head
    # attention), two, and sixteen (96 rows: the wide-row kernel)
    "mha_g1": C["c2_qwen3_8b"].with_(batch=2, n_q_heads=8, n_kv_heads=8, hist_len=1234, chunk_len=512),
    "mha_g1_tree_wide": C["c4_tree_72b"].with_(batch=1, n_q_heads=4, n_kv_heads=4, n_queries=40, hist_len=700,
                                               chunk_len=256),
    "gqa_g2_ragged": C["c3_internlm25_7b_ragged"].with_(batch=3, n_q_heads=8, n_kv_heads=4, hist_len=1500,
                                                        ragged_lo=1, chunk_len=512),
    "gqa_g16_wide": C["c2_qwen3_8b"].with_(batch=2, n_q_heads=32, n_kv_heads=2, hist_len=900, chunk_len=256),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cand_visibility(inp):
    cfg = inp.cfg
    if cfg.mask == "tree":
        return np.stack([oracle.tree_mask(inp.parents[b]) for b in range(cfg.batch)])
    return np.stack([oracle.chain_mask(cfg.n_queries)] * cfg.batch)


def oracle_round(inp, requests=None, kv_heads=None):
    return oracle.attention_reference(inp.q.float().numpy(), inp.hist_per_request("k"), inp.hist_per_request("v"),
                                      inp.hist_len, inp.k_cand.float().numpy(), inp.v_cand.float().numpy(),
                                      cand_visibility(inp), inp.cfg.scale, requests=requests, kv_heads=kv_heads)


def rows_of(cfg, b, g):
    """Index arrays selecting the O/lse entries of (request b, KV head g)."""
    hs = np.arange(g * cfg.group, (g + 1) * cfg.group)
    return b, slice(None), hs


def compare(cfg, o_gpu, lse_gpu, o_ref, lse_ref, sel=None):
    tol = TOL[cfg.dtype]
    if sel is None:
        eo = np.abs(o_gpu - o_ref).max()
        el = np.abs(lse_gpu - lse_ref).max()
    else:
        b, _, hs = sel
        eo = np.abs(o_gpu[b][:, hs] - o_ref[b][:, hs]).max()
        el = np.abs(lse_gpu[b][:, hs] - lse_ref[b][:, hs]).max()
    log(f"  {cfg.name}: max|dO| = {eo:.3e}, max|dlse| = {el:.3e} (tol {tol})")
    assert eo <= tol and el <= tol, (eo, el)


def check_mask(rnd, inp):
    want = np.stack([oracle.mask_to_bits(v) for v in cand_visibility(inp)]).astype(np.uint64)
    got = rnd.mask_out.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", list(SMALL))
def test_round_small(name):
    cfg = SMALL[name]
    log(f"[round_small] {name}: {cfg}")
    inp = wl.make_inputs(cfg)
    if cfg.streamed:
        rnd = rounds.StreamedRound(inp, n_buf=2)
    else:
        rnd = rounds.ResidentRound(inp)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    if not cfg.streamed:
        check_mask(rnd, inp)


@pytest.mark.parametrize("name", ["c1", "c2_small", "c3_small", "c3_small_token", "c4_small", "bf16_d64",
                                  "valu_r12_ragged", "wide_r96_ragged"])
@pytest.mark.parametrize("split", ["chunks", "balanced"])
def test_interleaved_kv_layout(name, split):
    """One history tensor with each token's K and V rows adjacent (the
    layout the benchmark uses): the views step over both rows."""
    cfg = SMALL[name]
    log(f"[interleaved] {name} {split}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, split=split, kv_layout="interleaved",
                               fuse_candidates="auto" if split == "balanced" else False)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


@pytest.mark.parametrize("name", ["valu_r4", "bf16_small_rows", "valu_r12_ragged", "valu_r15", "c2_small"])
def test_forced_valu_engine(name):
    """The VALU engine (SS_ENGINE_VALU) on bf16 shapes: the small-row kernel
    below 16 rows, the general VALU kernel above."""
    cfg = SMALL[name]
    log(f"[valu engine] {name}: rows={cfg.rows}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, engine="valu")
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("width", [2, 4, 6, 8])
def test_verification_widths(width):
    """Verification widths q in {2, 4, 6, 8} under 4-way GQA (8 to 32 rows per
    KV head) on the default engine."""
    cfg = C["c2_qwen3_8b"].with_(batch=3, n_queries=width, hist_len=2500, chunk_len=1024)
    log(f"[width] q={width} rows={cfg.rows}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("chunk_len,cps", [(64, 1), (100, 3), (512, 2), (4096, 1)])
def test_chunk_slot_states(chunk_len, cps):
    """Per-slot states of ss_verify_chunk against the oracle's local states
    (Eq. 7 over each slot's chunks), including slots past a request's end."""
    cfg = SMALL["c3_small"]
    log(f"[slot_states] chunk {chunk_len} cps {cps}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, chunk_len=chunk_len, chunks_per_slot=cps)
    rnd.chunks()
    torch.cuda.synchronize()
    m, l, acc = oracle.chunk_slot_states(inp.q.float().numpy(), inp.hist_per_request("k"),
                                         inp.hist_per_request("v"), inp.hist_len, chunk_len, 0, rnd.n_chunks, cps,
                                         cfg.scale)
    hs = slice(1, 1 + rnd.n_hist_slots)          # slot 0 holds the candidate region
    gm = rnd.state.m[hs].cpu().numpy()
    gl = rnd.state.l[hs].cpu().numpy()
    gacc = rnd.state.acc[hs].cpu().numpy()
    empty = np.isneginf(m)
    assert np.array_equal(np.isneginf(gm), empty)
    assert (gl[empty] == 0).all() and (gacc[empty] == 0).all()
    full = ~empty
    tol = TOL[cfg.dtype]
    # A slot state is an intermediate. The wide-row kernel rounds each weight
    # e^(s - m) of a long history to bf16 (relative error <= u = 2^-8, bf16
    # keeping 8 significant bits) and uses the same rounded weights in acc
    # and l, so the slot's normalised output acc / l moves by at most
    # u / (1 - u) * max_t |V_t - O| <= 2 u / (1 - u) * max|V|. The other
    # kernels keep each weight's rounding remainder too (or compute in fp32)
    # and take the plain bound. The final O and lse are held to 2e-3 always.
    vmax = float(inp.v_hist.float().abs().max())
    u = 2.0 ** -8
    wide_long = cfg.dtype == "bf16" and cfg.rows > 32 and int(np.max(inp.hist_len)) >= 2048
    tol_norm = max(tol, 2 * u / (1 - u) * vmax) if wide_long else tol
    e_m = np.abs(gm[full] - m[full]).max()
    e_l = np.abs(gl[full] / l[full] - 1).max()
    e_a = np.abs(gacc[full] / gl[full][:, None] - acc[full] / l[full][:, None]).max()
    log(f"  slot states: max|dm| {e_m:.2e}, max|dl/l| {e_l:.2e}, max|d(acc/l)| {e_a:.2e} (tol {tol_norm:.2e})")
    assert e_m <= tol and e_l <= tol and e_a <= tol_norm


def test_chunk_size_and_split_invariance():
    cfg = SMALL["c2_small"]
    inp = wl.make_inputs(cfg)
    o_ref, lse_ref = oracle_round(inp)
    outs = []
    for c, cps in ((64, 1), (512, 4), (2048, 1), (4500, 1), (1000, 2)):
        log(f"[invariance] chunk {c} cps {cps}")
        rnd = rounds.ResidentRound(inp, chunk_len=c, chunks_per_slot=cps)
        rnd.run()
        torch.cuda.synchronize()
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
        outs.append(rnd.o.cpu().numpy())
    # reversed slot order in the merge: fold the same slots in reverse
    rnd = rounds.ResidentRound(inp, chunk_len=512)
    rnd.chunks()
    rnd.candidates()
    for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
        t.copy_(t.flip(0))
    rnd.merge()
    torch.cuda.synchronize()
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


def test_empty_history_and_zero_lengths():
    cfg = SMALL["c3_small"].with_(batch=4)
    inp = wl.make_inputs(cfg)
    # request 1 has no history at all, request 2 a single token
    inp.hist_len = inp.hist_len.copy()
    inp.hist_len[1] = 0
    inp.hist_len[2] = 1
    rnd = rounds.ResidentRound(inp)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    # uniform empty history: every chunk call is a no-op, candidates alone
    cfg0 = SMALL["c2_small"].with_(hist_len=0)
    inp0 = wl.make_inputs(cfg0)
    rnd0 = rounds.ResidentRound(inp0)
    assert rnd0.n_chunks == 0
    rnd0.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp0)
    compare(cfg0, rnd0.o.cpu().numpy(), rnd0.lse.cpu().numpy(), o_ref, lse_ref)


def test_merge_all_empty_and_slots_per_req():
    cfg = SMALL["c2_small"]
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, chunk_len=1024)
    rnd.chunks()
    rnd.candidates()
    torch.cuda.synchronize()
    # request 0 folds only its first two slots (candidates + chunk 0),
    # request 1 none at all
    spr = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    ss.ss_merge_states(rnd.problem, rnd.state, spr, rnd.o, rnd.lse)
    torch.cuda.synchronize()
    o = rnd.o.cpu().numpy()
    lse = rnd.lse.cpu().numpy()
    assert (o[1] == 0).all() and np.isneginf(lse[1]).all()
    q = inp.q.float().numpy()
    m, l, acc = oracle.chunk_slot_states(q, inp.hist_per_request("k"), inp.hist_per_request("v"), inp.hist_len,
                                         1024, 0, 1, 1, cfg.scale)
    cm, cl, cacc = oracle.candidate_state(q, inp.k_cand.float().numpy(), inp.v_cand.float().numpy(),
                                          cand_visibility(inp), cfg.scale)
    o_ref, lse_ref = oracle.merge_slots(np.concatenate([cm[None], m]), np.concatenate([cl[None], l]),
                                        np.concatenate([cacc[None], acc]))
    assert np.abs(o[0] - o_ref[0]).max() <= 2e-3 and np.abs(lse[0] - lse_ref[0]).max() <= 2e-3


def test_closed_forms_on_gpu():
    """Q = 0 gives the mean of the visible values and lse = ln(#visible); a
    planted needle key dominates its rows."""
    cfg = SMALL["c2_small"]
    inp = wl.make_inputs(cfg)
    inp.q.zero_()
    rnd = rounds.ResidentRound(inp)
    rnd.run()
    torch.cuda.synchronize()
    lse = rnd.lse.cpu().numpy()
    n = cfg.hist_len
    want = np.log(n + np.arange(cfg.n_queries) + 1.0)
    assert np.abs(lse - want[None, :, None]).max() <= 1e-4
    o = rnd.o.cpu().numpy()
    vh = inp.v_hist.float().numpy()
    vc = inp.v_cand.float().numpy()
    for b in range(cfg.batch):
        for i in range(cfg.n_queries):
            for h in range(0, cfg.n_q_heads, 5):
                g = h // cfg.group
                ref = (vh[b, g].sum(0) + vc[b, g, :i + 1].sum(0)) / (n + i + 1)
                assert np.abs(o[b, i, h] - ref).max() <= 1e-4
    # needle: one key in chunk 3 scores +30 for every row of KV head 1 of request 0
    inp = wl.make_inputs(cfg)
    u = torch.randn(cfg.head_dim, generator=torch.Generator().manual_seed(9))
    u = u / u.norm()
    inp.q[0, :, cfg.group:2 * cfg.group, :] = u.to(inp.q.dtype)
    qrow = inp.q[0, 0, cfg.group].float()
    t = 3 * cfg.chunk_len + 77
    inp.k_hist[0, 1, t] = (30.0 / cfg.scale * qrow / qrow.dot(qrow)).to(inp.k_hist.dtype)
    rnd = rounds.ResidentRound(inp)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp, requests=[0], kv_heads=[1])
    sel = rows_of(cfg, 0, 1)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref, sel)
    assert np.abs(rnd.o.cpu().numpy()[0][:, sel[2]] - inp.v_hist[0, 1, t].float().numpy()).max() < 5e-3


@pytest.mark.parametrize("n_buf,per_copy", [(1, 1), (2, 1), (3, 1), (2, 3), (1, 2)])
def test_streamed_matches_resident_and_oracle(n_buf, per_copy):
    cfg = SMALL["c5_small"].with_(hist_len=8 * 256, chunk_len=256)
    log(f"[streamed] n_buf {n_buf}, chunks per copy {per_copy}")
    inp = wl.make_inputs(cfg)
    srd = rounds.StreamedRound(inp, n_buf=n_buf, chunks_per_copy=per_copy)
    srd.run(record_timings=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, srd.o.cpu().numpy(), srd.lse.cpu().numpy(), o_ref, lse_ref)
    rrd = rounds.ResidentRound(inp, chunk_len=256)
    rrd.run()
    torch.cuda.synchronize()
    assert np.abs(srd.o.cpu().numpy() - rrd.o.cpu().numpy()).max() <= 1e-5
    c0, c1, k0, k1 = ss.ss_stream_timings(srd.n_chunks)
    for j in range(srd.n_chunks):
        assert c0[j] <= c1[j] <= k0[j] + 1e-3 and k0[j] <= k1[j]     # compute starts after its chunk landed
        if j % per_copy:                                              # one copy per group of chunks
            assert c0[j] == c0[j - 1] and c1[j] == c1[j - 1]
    assert rounds.exposed_wait((c0, c1, k0, k1)) >= 0


@pytest.mark.parametrize("n_buf,per_copy", [(1, 1), (2, 1), (2, 2), (3, 2)])
@pytest.mark.parametrize("checks", ["poison", "delay", "poison+delay"])
def test_streamed_ordering_checks(n_buf, per_copy, checks):
    """Ordering of the streaming pipeline (SpecStream section 4.2: a staging
    buffer takes the next chunk only after every query of the group has
    attended the chunk it holds). SS_STREAM_POISON overwrites each buffer
    with NaN right after its wait for the last reader and before its copy,
    so a kernel still reading it, or reading it before the copy landed,
    would see NaN; SS_STREAM_DELAY holds the copy stream ~2 ms before every
    copy, so compute that did not wait for its chunk would read the previous
    contents. The result must match the oracle, with no NaN."""
    cfg = SMALL["c5_small"].with_(hist_len=8 * 256, chunk_len=256)
    flag = {"poison": ss.SS_STREAM_POISON, "delay": ss.SS_STREAM_DELAY,
            "poison+delay": ss.SS_STREAM_POISON | ss.SS_STREAM_DELAY}[checks]
    log(f"[stream checks] {checks}, n_buf {n_buf}, chunks per copy {per_copy}")
    inp = wl.make_inputs(cfg)
    o_ref, lse_ref = oracle_round(inp)
    srd = rounds.StreamedRound(inp, n_buf=n_buf, chunks_per_copy=per_copy)
    for rep in range(2):
        srd.o.fill_(float("nan"))
        srd.run(record_timings=True, checks=flag)
        torch.cuda.synchronize()
        o, lse = srd.o.cpu().numpy(), srd.lse.cpu().numpy()
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        compare(cfg, o, lse, o_ref, lse_ref)
        c0, c1, k0, k1 = ss.ss_stream_timings(srd.n_chunks)
        assert all(c1[j] <= k0[j] + 1e-3 for j in range(srd.n_chunks))
        if flag & ss.SS_STREAM_DELAY:
            # every copy group waited ~2 ms on the host before its copy
            starts = sorted(set(c0))
            assert all(b - a >= 1.5 for a, b in zip(starts, starts[1:])), starts
    # after the round the buffers hold the last copied chunks, not the poison
    last = srd.staging[(srd.n_chunks // per_copy - 1) % n_buf].view(per_copy, -1)[-1]
    assert torch.equal(last.cpu(), srd.host_kv[srd.n_chunks - 1])


def test_streamed_calls_overlap_on_two_stream_pairs():
    """Two streaming calls on one device, each with its own copy and compute
    streams and staging buffers, enqueued back to back with nothing ordering
    them (the first held back by SS_STREAM_DELAY, the second poisoning its
    buffers): both give the results of the same calls run one after the
    other, bit for bit. The calls share the device's event objects; every
    wait refers to a mark its own call recorded."""
    cfgs = [SMALL["c5_small"].with_(hist_len=8 * 256, chunk_len=256),
            SMALL["c5_small"].with_(batch=3, n_queries=4, hist_len=6 * 256, chunk_len=256, seed=77)]
    rnds = [rounds.StreamedRound(wl.make_inputs(c), n_buf=2) for c in cfgs]
    refs = []
    for r in rnds:
        r.run()
        torch.cuda.synchronize()
        refs.append((r.o.clone(), r.lse.clone()))
    streams = [(torch.cuda.Stream(), torch.cuda.Stream()) for _ in rnds]
    for rep in range(2):
        torch.cuda.synchronize()
        for r in rnds:
            r.o.fill_(float("nan"))
            r.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        for i, (r, (cp, cs)) in enumerate(zip(rnds, streams)):
            ss.ss_stream_history(r.problem, r.q, r.host_kv, r.chunk_len, r.n_chunks, r.staging, r.n_buf, r.state, 0,
                                 cp, cs, checks=ss.SS_STREAM_DELAY if i == 0 else ss.SS_STREAM_POISON)
            ss.ss_verify_candidates(r.problem, r.q, r.cand_view, r.parents, None, r.state, r.n_chunks, cs)
            ss.ss_merge_states(r.problem, r.state, None, r.o, r.lse, cs)
        torch.cuda.synchronize()
        for i, (r, (o_ref, lse_ref)) in enumerate(zip(rnds, refs)):
            assert torch.equal(r.o, o_ref), (rep, i)
            assert torch.equal(r.lse, lse_ref), (rep, i)
        log(f"  overlapping calls, repetition {rep}: both identical to the sequential runs")


@pytest.mark.parametrize("n_buf,per_copy", [(1, 1), (2, 1), (2, 2), (3, 1)])
def test_layered_stream_with_prefetch(n_buf, per_copy):
    """Three layers, each with its own host-resident history, the staging
    ring continued across layers (cross-layer prefetch) or restarted per
    layer: every layer's result matches the oracle, and chunks are attended
    only after they landed."""
    base = SMALL["c5_small"].with_(hist_len=6 * 256, chunk_len=256)
    inputs = [wl.make_inputs(base.with_(seed=base.seed + 10 * i)) for i in range(3)]
    lr = rounds.LayeredStreamedRound(inputs, n_buf=n_buf, chunks_per_copy=per_copy, rest_dim=512, rest_reps=2)
    refs = [oracle_round(inp) for inp in inputs]
    for prefetch in (True, False, True):
        log(f"[layered] n_buf {n_buf}, chunks per copy {per_copy}, prefetch {prefetch}")
        for lay in lr.layers:
            lay.o.fill_(float("nan"))
        lr.run(prefetch=prefetch, record_timings=True)
        torch.cuda.synchronize()
        for lay, (o_ref, lse_ref) in zip(lr.layers, refs):
            compare(base, lay.o.cpu().numpy(), lay.lse.cpu().numpy(), o_ref, lse_ref)
        for i, lay in enumerate(lr.layers):
            c0, c1, k0, k1 = ss.ss_stream_timings(lay.n_chunks, back=len(lr.layers) - 1 - i)
            assert all(c1[j] <= k0[j] + 1e-3 for j in range(lay.n_chunks))
        log(f"  exposed waits (ms): {[round(w, 3) for w in lr.layer_waits()]}")


BALANCED = {
    "c3_small_s2": ("c3_small", 2),
    "c3_small_s6": ("c3_small", 6),
    "c3_small_token_s3": ("c3_small_token", 3),
    "c2_small_s3": ("c2_small", 3),
    "rows16_s4": ("bf16_rows16", 4),
    "rows4_mfma_s2": ("valu_r4", 2),
    "rows32_g8_s5": ("bf16_rows32_g8", 5),
    # cuts by fixed chunks: fp32 (VALU), wide rows, one slot
    "c1_fallback_s3": ("c1", 3),
    "wide_fallback_s3": ("wide_r96_ragged", 3),
    "c2_one_slot": ("c2_small", 1),
    # GQA group sizes 1, 2 and 16
    "mha_g1_s3": ("mha_g1", 3),
    "gqa_g2_ragged_s4": ("gqa_g2_ragged", 4),
    "gqa_g16_wide_s3": ("gqa_g16_wide", 3),
}


def _history_only(inp):
    """The oracle's state of each request's whole history (one slot)."""
    cfg = inp.cfg
    n = max(int(inp.hist_len.max()), 1)
    return oracle.chunk_slot_states(inp.q.float().numpy(), inp.hist_per_request("k"), inp.hist_per_request("v"),
                                    inp.hist_len, n, 0, 1, 1, cfg.scale)


def _check_history_slots(rnd, inp):
    """Folding the history slots (1 ..) alone gives the history-only result:
    every slot was written (the state was pre-filled with NaN) and together
    they cover each request's history exactly once."""
    cfg = inp.cfg
    m, l, acc = _history_only(inp)
    o_ref, lse_ref = oracle.merge_slots(m, l, acc)
    hs = slice(1, 1 + rnd.n_hist_slots)
    gm = rnd.state.m[hs].double().cpu().numpy()
    gl = rnd.state.l[hs].double().cpu().numpy()
    gacc = rnd.state.acc[hs].double().cpu().numpy()
    assert not np.isnan(gm).any() and not np.isnan(gl).any() and not np.isnan(gacc).any()
    o, lse = oracle.merge_slots(gm, gl, gacc)
    # requests without history: lse = -inf and O = 0 on both sides
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty)
    assert (o[empty] == 0).all()
    tol = TOL[cfg.dtype]
    eo = np.abs(o - o_ref).max()
    el = np.abs(lse[~empty] - lse_ref[~empty]).max() if (~empty).any() else 0.0
    log(f"  history slots: max|dO| = {eo:.3e}, max|dlse| = {el:.3e} (tol {tol})")
    assert eo <= tol and el <= tol, (eo, el)


@pytest.mark.parametrize("name", list(BALANCED))
def test_history_balanced(name):
    base, n_slots = BALANCED[name]
    cfg = SMALL[base]
    log(f"[history] {name}: rows={cfg.rows} slots={n_slots}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, split="balanced", history_slots=n_slots)
    for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
        t.fill_(float("nan"))
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)
    _check_history_slots(rnd, inp)


@pytest.mark.parametrize("name", list(BALANCED))
def test_history_fused_candidates(name):
    """ss_verify_history with the candidate region: folded into each stream's
    first piece on the MFMA kernels, in a slot of its own on the VALU ones."""
    base, n_slots = BALANCED[name]
    cfg = SMALL[base]
    if n_slots < 2 and not rounds.mfma_fuses_candidates(cfg):
        pytest.skip("candidates need a slot of their own outside the narrow kernel")
    log(f"[fused] {name}: rows={cfg.rows} slots={n_slots}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, split="balanced", history_slots=n_slots, fuse_candidates=True)
    for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
        t.fill_(float("nan"))
    rnd.mask_out.fill_(-1)
    rnd.run()
    torch.cuda.synchronize()
    assert not torch.isnan(rnd.state.m).any() and not torch.isnan(rnd.state.acc).any()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


@pytest.mark.parametrize("group", [2, 8])
def test_wide_fused_candidates_forest(group):
    """The wide-row kernel with the candidate region folded in: 64 candidates
    forming two trees (node 32 is a second root and nodes 33.. hang below
    it), two requests without history. With 128 rows (32-key tiles) the rows
    of the second tree see nothing in the first candidate tile and nothing
    before it, so they stay empty through that tile; with 512 rows (64-key
    tiles) the candidates are one tile. Rows without history average at
    most 64 candidate values, so the weights' bf16 rounding remainders must
    be carried for them to stay within 2e-3."""
    cfg = C["c3_internlm25_7b_ragged"].with_(batch=4, n_q_heads=2 * group, n_kv_heads=2, n_queries=64,
                                              hist_len=700, ragged_lo=1, chunk_len=256, mask="tree")
    log(f"[wide fused forest] rows={cfg.rows}")
    inp = wl.make_inputs(cfg)
    inp.hist_len = inp.hist_len.copy()
    inp.hist_len[[0, 2]] = 0
    inp.parents = inp.parents.copy()
    inp.parents[:, 32] = -1
    inp.parents[:, 33:] = np.arange(32, 63)
    rnd = rounds.ResidentRound(inp, split="balanced", history_slots=3, fuse_candidates=True)
    for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
        t.fill_(float("nan"))
    rnd.mask_out.fill_(-1)
    rnd.run()
    torch.cuda.synchronize()
    assert not torch.isnan(rnd.state.m).any() and not torch.isnan(rnd.state.acc).any()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


# Short histories: a row then averages over a handful of keys, where a weight
# rounded to bf16 without its remainder would move O by up to ~4e-3.
SHORT_KERNELS = {
    "narrow_mfma": dict(n_q_heads=32, n_kv_heads=8, n_queries=6, mask="causal", engine="auto"),
    "wide_mfma_r128": dict(n_q_heads=16, n_kv_heads=2, n_queries=16, mask="tree", engine="auto"),
    "wide_mfma_r512": dict(n_q_heads=64, n_kv_heads=8, n_queries=64, mask="tree", engine="auto"),
    "wide_mfma_r128_d64": dict(n_q_heads=16, n_kv_heads=2, n_queries=16, mask="tree", engine="auto", head_dim=64),
    "wide_mfma_r512_d64": dict(n_q_heads=64, n_kv_heads=8, n_queries=64, mask="tree", engine="auto", head_dim=64),
    "valu_small_r8": dict(n_q_heads=32, n_kv_heads=8, n_queries=2, mask="causal", engine="valu"),
}


# A uniform view needs at least one token; zero-token requests go through
# the ragged layout (and test_empty_history_and_zero_lengths).
SHORT_LENGTHS = [(layout, hist) for layout in ("uniform", "ragged") for hist in (0, 1, 3, 8, 31, 64)
                 if layout == "ragged" or hist > 0]


@pytest.mark.parametrize("layout,hist", SHORT_LENGTHS)
@pytest.mark.parametrize("kernel", list(SHORT_KERNELS))
@pytest.mark.parametrize("path", ["chunks", "balanced"])
def test_short_histories(kernel, hist, layout, path):
    """Requests whose whole committed history is 0-64 tokens (the GPU region
    after the history is then much of what a query sees), against the oracle
    at 2e-3 on O and lse. Uniform lengths (no length array) and ragged ones
    (the requests at hist, hist // 2 and hist tokens); the fixed-chunk round
    (candidates in a slot of their own) and the balanced history call (the
    candidate region folded in where an MFMA kernel serves the shape)."""
    kw = dict(SHORT_KERNELS[kernel])
    engine = kw.pop("engine")
    if layout == "uniform":
        cfg = C["c2_qwen3_8b"].with_(batch=3, hist_len=hist, chunk_len=128, **kw)
    else:
        cfg = C["c3_internlm25_7b_ragged"].with_(batch=3, hist_len=64, ragged_lo=64, chunk_len=128, **kw)
    log(f"[short] {kernel} hist={hist} {layout} {path} rows={cfg.rows}")
    inp = wl.make_inputs(cfg)
    if layout == "ragged":
        inp.hist_len = np.array([hist, hist // 2, hist], dtype=np.int32)
    if path == "chunks":
        rnd = rounds.ResidentRound(inp, engine=engine)
    else:
        rnd = rounds.ResidentRound(inp, engine=engine, split="balanced", history_slots=3,
                                   fuse_candidates=rounds.mfma_fuses_candidates(cfg, engine))
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


def test_history_balanced_many_requests_and_empties():
    """More requests than a wavefront has lanes (the start search spans
    several blocks), empty requests between and at the end, lengths off the
    128-token alignment, drawn from [1, 2000] apart from the planted ones."""
    cfg = SMALL["c3_small"].with_(batch=70, hist_len=2000, ragged_lo=1, chunk_len=256)
    inp = wl.make_inputs(cfg)
    inp.hist_len = inp.hist_len.copy()
    inp.hist_len[[0, 5, 6, 40, 68, 69]] = 0
    inp.hist_len[7] = 1
    inp.hist_len[8] = 128
    inp.hist_len[9] = 129
    o_ref, lse_ref = oracle_round(inp)
    for n_slots in (2, 3, 9):
        for fuse in (False, True):
            log(f"[history] 70 requests, slots={n_slots}, candidates fused={fuse}")
            rnd = rounds.ResidentRound(inp, split="balanced", history_slots=n_slots, fuse_candidates=fuse)
            for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
                t.fill_(float("nan"))
            rnd.run()
            torch.cuda.synchronize()
            compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
            check_mask(rnd, inp)
            if not fuse:
                _check_history_slots(rnd, inp)
            else:
                assert not torch.isnan(rnd.state.m).any() and not torch.isnan(rnd.state.acc).any()
    # no history at all: every history slot is empty, the result is the
    # candidate region alone
    inp.hist_len[:] = 0
    o_ref, lse_ref = oracle_round(inp)
    for fuse in (False, True):
        rnd = rounds.ResidentRound(inp, split="balanced", history_slots=3, fuse_candidates=fuse)
        for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
            t.fill_(float("nan"))
        rnd.run()
        torch.cuda.synchronize()
        assert np.isneginf(rnd.state.m[1:].cpu().numpy()).all()
        assert (rnd.state.l[1:] == 0).all() and (rnd.state.acc[1:] == 0).all()
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
        check_mask(rnd, inp)


ROUND_CASES = {
    "narrow_uniform": C["c2_qwen3_8b"].with_(batch=3, hist_len=3000, chunk_len=1024),
    "narrow_ragged": C["c3_internlm25_7b_ragged"].with_(batch=7, hist_len=2500, ragged_lo=1, chunk_len=512),
    # 256 streams of at most 2000 tokens: the library's choice is one piece per stream
    "narrow_ragged_short_many": C["c3_internlm25_7b_ragged"].with_(batch=32, hist_len=2000, ragged_lo=1,
                                                                   chunk_len=512),
    "wide_tree": C["c4_tree_72b"].with_(batch=2, hist_len=2600, chunk_len=1024),
    "wide_r96_ragged": C["c3_internlm25_7b_ragged"].with_(batch=3, n_queries=24, hist_len=2200, ragged_lo=1,
                                                          chunk_len=300),
    "valu_f32": C["c1_tiny_f32"],
    "valu_small_rows": C["c2_qwen3_8b"].with_(batch=2, n_queries=2, hist_len=1500, chunk_len=512),
}


@pytest.mark.parametrize("name", list(ROUND_CASES))
@pytest.mark.parametrize("n_slots", [0, 3])
def test_verify_round(name, n_slots):
    """ss_verify_round (history and candidates into a workspace, then the
    merge, in one call) against the oracle; the library's slot choice
    (n_slots = 0) and a given one; the workspace starts as NaN."""
    cfg = ROUND_CASES[name]
    log(f"[round call] {name}: rows={cfg.rows} n_slots={n_slots}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp)
    work = ss.StateBuffers(rnd.problem, 12, "cuda")
    for t in (work.acc, work.m, work.l):
        t.fill_(float("nan"))
    rnd.mask_out.fill_(-1)
    ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, n_slots, work,
                       rnd.o, rnd.lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


ONE_SLOT_CASES = {
    "ragged_empties": C["c3_internlm25_7b_ragged"].with_(batch=70, hist_len=2000, ragged_lo=1, chunk_len=256),
    "ragged_no_history": C["c3_internlm25_7b_ragged"].with_(batch=4, hist_len=300, ragged_lo=1, chunk_len=128),
    "ragged_tree_32_rows": C["c3_internlm25_7b_ragged"].with_(batch=5, n_queries=8, mask="tree", hist_len=3000,
                                                              ragged_lo=1, chunk_len=512),
    "uniform": C["c2_qwen3_8b"].with_(batch=3, hist_len=3000, chunk_len=1024),
    "uniform_4_rows": C["c2_qwen3_8b"].with_(batch=2, n_queries=1, hist_len=1500, chunk_len=512),
    # wide-row kernel: 8-wave groups (512 rows per KV head, a tree) and 4-wave groups (96 rows)
    "wide_tree": C["c4_tree_72b"].with_(batch=2, hist_len=2600, chunk_len=1024),
    "wide_tree_short_histories": C["c4_tree_72b"].with_(batch=3, hist_len=70, ragged_lo=1, chunk_len=64),
    "wide_96_rows_ragged": C["c3_internlm25_7b_ragged"].with_(batch=3, n_queries=24, hist_len=2200, ragged_lo=1,
                                                              chunk_len=300),
}


@pytest.mark.parametrize("name", list(ONE_SLOT_CASES))
def test_round_one_slot_writes_the_result(name):
    """ss_verify_round with one slot per stream on the MFMA engines (narrow
    and wide-row) writes O and lse from the history launch (no merge
    launch): the same
    values as ss_verify_history into one slot followed by ss_merge_states,
    with the outputs poisoned before each call; the workspace is left
    untouched; the result matches the oracle. Ragged cases include empty
    requests, with and without any history."""
    cfg = ONE_SLOT_CASES[name]
    inp = wl.make_inputs(cfg)
    if cfg.ragged:
        inp.hist_len = inp.hist_len.copy()
        if name == "ragged_empties":
            inp.hist_len[[0, 5, 6, 40, 68, 69]] = 0
            inp.hist_len[7], inp.hist_len[8], inp.hist_len[9] = 1, 128, 129
        elif name == "ragged_no_history":
            inp.hist_len[:] = 0
    log(f"[one-slot round] {name}: rows={cfg.rows}")
    rnd = rounds.ResidentRound(inp, split="balanced", history_slots=1, fuse_candidates=True)
    assert rnd.n_call_slots == 1
    # the launch path: one slot, then the merge
    rnd.o.fill_(float("nan"))
    rnd.lse.fill_(float("nan"))
    rnd.run()
    torch.cuda.synchronize()
    o_m, lse_m, mask_m = rnd.o.clone(), rnd.lse.clone(), rnd.mask_out.clone()
    work = ss.StateBuffers(rnd.problem, 4, "cuda")
    for t in (work.acc, work.m, work.l):
        t.fill_(float("nan"))
    for rep in range(2):
        rnd.o.fill_(float("nan"))
        rnd.lse.fill_(float("nan"))
        rnd.mask_out.fill_(-1)
        ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, 1, work,
                           rnd.o, rnd.lse)
        torch.cuda.synchronize()
        assert torch.equal(rnd.o, o_m) and torch.equal(rnd.lse, lse_m), (name, rep)
        assert torch.equal(rnd.mask_out, mask_m), (name, rep)
    assert torch.isnan(work.m).all() and torch.isnan(work.acc).all()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


@pytest.mark.parametrize("hist_len", [2000, 3500])
def test_round_slot_choice_short_ragged(hist_len):
    """ss_verify_round with n_slots = 0 on short ragged histories with at
    least one stream per compute unit takes one piece per stream (its result
    is the n_slots = 1 call's, bit for bit): up to 4096 tokens for the
    whole-round call, up to 2048 for the Python helper's history + merge
    count; both match the oracle."""
    cfg = ROUND_CASES["narrow_ragged_short_many"].with_(hist_len=hist_len)
    cus = rounds.device_cus()
    streams = cfg.batch * cfg.n_kv_heads
    inp = wl.make_inputs(cfg)
    mx = int(inp.hist_len.max())
    expect_one = (mx <= 4096 and streams >= cus) or (mx <= 2048 and 4 * streams >= 3 * cus)
    log(f"[round slots] {streams} streams, longest history {mx}, {cus} CUs: one piece per stream expected: "
        f"{expect_one}")
    assert (rounds.auto_history_slots(cfg, inp.hist_len, cus) == 1) == rounds.one_piece_per_stream(mx, streams, cus)
    rnd = rounds.ResidentRound(inp)
    work = ss.StateBuffers(rnd.problem, 12, "cuda")
    outs = {}
    for n_slots in (0, 1):
        o, lse = torch.full_like(rnd.o, float("nan")), torch.full_like(rnd.lse, float("nan"))
        ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, n_slots,
                           work, o, lse)
        torch.cuda.synchronize()
        outs[n_slots] = (o, lse)
    if expect_one:
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    o_ref, lse_ref = oracle_round(inp)
    for n_slots in (0, 1):
        compare(cfg, outs[n_slots][0].cpu().numpy(), outs[n_slots][1].cpu().numpy(), o_ref, lse_ref)


def test_invalid_call_enqueues_nothing():
    cfg = SMALL["c2_small"]
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp)
    rnd.state.m.fill_(7.0)
    with pytest.raises(ss.SSError) as e:
        ss.ss_verify_chunk(rnd.problem, rnd.q, rnd.hist_view, cfg.chunk_len, 0, rnd.n_chunks + 10, 1, rnd.state, 0)
    assert e.value.code == ss.SS_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (rnd.state.m == 7.0).all()


# ---------------------------------------------------------------------------
# full-size workloads, sampled slices
# ---------------------------------------------------------------------------

FULL = ["c1_tiny_f32", "c2_qwen3_8b", "c3_internlm25_7b_ragged", "c4_tree_72b", "c5_streamed"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = C[name]
    log(f"[full] {name}: generating inputs")
    inp = wl.make_inputs(cfg)
    log(f"[full] {name}: running")
    # the launch configuration the benchmark times
    rnd = rounds.StreamedRound(inp, n_buf=2) if cfg.streamed else rounds.ResidentRound(inp, **rounds.BENCH_RESIDENT)
    rnd.run()
    torch.cuda.synchronize()
    o = rnd.o.cpu().numpy()
    lse = rnd.lse.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    if not cfg.streamed:
        check_mask(rnd, inp)
    rng = np.random.default_rng(cfg.seed)
    picks = [(0, 0), (cfg.batch - 1, cfg.n_kv_heads - 1)]
    picks.append((int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_kv_heads))))
    if cfg.ragged:
        picks.append((int(np.argmax(inp.hist_len)), 2))
        picks.append((int(np.argmin(inp.hist_len)), 5))
    for b, g in picks:
        log(f"[full] {name}: oracle slice b={b} g={g}")
        o_ref, lse_ref = oracle_round(inp, requests=[b], kv_heads=[g])
        compare(cfg, o, lse, o_ref, lse_ref, rows_of(cfg, b, g))


D64_CASES = {
    "uniform": C["c2_qwen3_8b"].with_(batch=3, head_dim=64, hist_len=3000, chunk_len=1024),
    "ragged_empties": C["c3_internlm25_7b_ragged"].with_(batch=70, head_dim=64, hist_len=2500, ragged_lo=1,
                                                         chunk_len=256),
    "ragged_tree_32_rows": C["c3_internlm25_7b_ragged"].with_(batch=5, head_dim=64, n_queries=8, mask="tree",
                                                              hist_len=3000, ragged_lo=1, chunk_len=512),
    "rows_4": C["c2_qwen3_8b"].with_(batch=2, head_dim=64, n_queries=1, hist_len=1500, chunk_len=512),
    "short_histories": C["c3_internlm25_7b_ragged"].with_(batch=9, head_dim=64, hist_len=64, ragged_lo=1,
                                                          chunk_len=32),
}


@pytest.mark.parametrize("name", list(D64_CASES))
def test_head_dim_64_on_the_matrix_cores(name):
    """bf16 with head_dim 64 and up to 32 rows per KV head runs on the narrow
    MFMA kernels (the V staging map with one key group per lane): the
    benchmark's launch configuration (balanced cut, candidates folded in),
    the chunked split, the whole-round call with the library's slot choice
    and with one slot, and the forced VALU engine all match the oracle.
    Ragged cases include empty requests."""
    cfg = D64_CASES[name]
    assert rounds.narrow_mfma(cfg)
    inp = wl.make_inputs(cfg)
    if name == "ragged_empties":
        inp.hist_len = inp.hist_len.copy()
        inp.hist_len[[0, 5, 6, 40, 68, 69]] = 0
        inp.hist_len[7], inp.hist_len[8], inp.hist_len[9] = 1, 128, 129
    o_ref, lse_ref = oracle_round(inp)
    for label, kw in (("balanced", dict(rounds.BENCH_RESIDENT)),
                      ("balanced, 3 slots", dict(rounds.BENCH_RESIDENT, history_slots=3)),
                      ("chunks", dict(split="chunks", chunks_per_slot=2)),
                      ("valu", dict(split="chunks", chunks_per_slot=2, engine="valu"))):
        log(f"[d64] {name}: {label}")
        rnd = rounds.ResidentRound(inp, **kw)
        rnd.run()
        torch.cuda.synchronize()
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
        check_mask(rnd, inp)
    rnd = rounds.ResidentRound(inp)
    work = ss.StateBuffers(rnd.problem, 12, "cuda")
    for n_slots in (0, 1):
        log(f"[d64] {name}: round call, n_slots={n_slots}")
        rnd.o.fill_(float("nan"))
        rnd.lse.fill_(float("nan"))
        ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, n_slots,
                           work, rnd.o, rnd.lse)
        torch.cuda.synchronize()
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


D64_WIDE_CASES = {
    "tree_512_rows": C["c4_tree_72b"].with_(batch=2, head_dim=64, hist_len=5000, chunk_len=1024),
    "tree_128_rows_ragged_empties": C["c3_internlm25_7b_ragged"].with_(
        batch=12, n_q_heads=16, n_kv_heads=2, n_queries=16, mask="tree", head_dim=64, hist_len=4000, ragged_lo=1,
        chunk_len=512),
    "rows_40": C["c2_qwen3_8b"].with_(batch=3, n_q_heads=16, n_kv_heads=4, n_queries=10, head_dim=64,
                                      hist_len=3000, chunk_len=512),
}


@pytest.mark.parametrize("name", list(D64_WIDE_CASES))
def test_head_dim_64_wide_rows(name):
    """bf16 with head_dim 64 and more than 32 rows per KV head runs on the
    wide-row MFMA kernel (eight-wave groups of 256 rows, or four-wave groups
    of 128): the benchmark's launch configuration (balanced cut, candidates
    folded in), the chunked split, the whole-round call with the library's
    slot choice and with one slot (O and lse written by the history launch),
    and the forced VALU engine all match the oracle. The ragged case has
    empty requests and requests below the short-history threshold."""
    cfg = D64_WIDE_CASES[name]
    assert cfg.rows > 32 and rounds.mfma_fuses_candidates(cfg) and not rounds.narrow_mfma(cfg)
    inp = wl.make_inputs(cfg)
    if name == "tree_128_rows_ragged_empties":
        inp.hist_len = inp.hist_len.copy()
        inp.hist_len[[0, 5, 11]] = 0
        inp.hist_len[6], inp.hist_len[7], inp.hist_len[8] = 1, 2047, 2048
    o_ref, lse_ref = oracle_round(inp)
    for label, kw in (("balanced", dict(rounds.BENCH_RESIDENT)),
                      ("chunks", dict(split="chunks", chunks_per_slot=2)),
                      ("valu", dict(split="chunks", chunks_per_slot=2, engine="valu"))):
        log(f"[d64 wide] {name}: {label}")
        rnd = rounds.ResidentRound(inp, **kw)
        rnd.run()
        torch.cuda.synchronize()
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
        check_mask(rnd, inp)
    rnd = rounds.ResidentRound(inp)
    work = ss.StateBuffers(rnd.problem, 64, "cuda")
    for n_slots in (0, 1):
        log(f"[d64 wide] {name}: round call, n_slots={n_slots}")
        rnd.o.fill_(float("nan"))
        rnd.lse.fill_(float("nan"))
        ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, n_slots,
                           work, rnd.o, rnd.lse)
        torch.cuda.synchronize()
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


F32_CASES = {
    "tiny_d64": C["c1_tiny_f32"],
    "uniform_d128": C["c2_qwen3_8b"].with_(batch=3, dtype="f32", hist_len=3000, chunk_len=1024),
    "ragged_empties_d128": C["c3_internlm25_7b_ragged"].with_(batch=20, dtype="f32", hist_len=2500, ragged_lo=1,
                                                              chunk_len=256),
    "tree_32_rows_d64": C["c3_internlm25_7b_ragged"].with_(batch=5, dtype="f32", head_dim=64, n_queries=8,
                                                           mask="tree", hist_len=3000, ragged_lo=1, chunk_len=512),
    "rows_4_d128": C["c2_qwen3_8b"].with_(batch=2, dtype="f32", n_queries=1, hist_len=1500, chunk_len=512),
    "short_histories_d128": C["c3_internlm25_7b_ragged"].with_(batch=9, dtype="f32", hist_len=40, ragged_lo=1,
                                                               chunk_len=16),
    # beyond 32 rows: one work-group per row group of 32 rows
    "tree_512_rows_d128": C["c4_tree_72b"].with_(batch=2, dtype="f32", hist_len=2000, chunk_len=512),
    "tree_96_rows_d128_ragged": C["c3_internlm25_7b_ragged"].with_(batch=7, dtype="f32", n_queries=12, n_q_heads=64,
                                                                   mask="tree", hist_len=3000, ragged_lo=1,
                                                                   chunk_len=512),
    "rows_40_d64": C["c2_qwen3_8b"].with_(batch=3, dtype="f32", head_dim=64, n_queries=10, n_q_heads=16,
                                          n_kv_heads=4, hist_len=2500, chunk_len=256),
}


@pytest.mark.parametrize("name", list(F32_CASES))
def test_fp32_on_both_engines(name):
    """fp32 inputs run on the fp32 MFMA kernel (AUTO; beyond 32 rows per KV
    head one work-group per row group of 32), and on the VALU kernel when
    forced: both, under the chunked split and ss_verify_history, and the
    whole-round call, match the oracle within 1e-5. Ragged cases include
    empty requests."""
    cfg = F32_CASES[name]
    assert rounds.f32_mfma(cfg)
    inp = wl.make_inputs(cfg)
    if name == "tree_96_rows_d128_ragged":
        inp.hist_len = inp.hist_len.copy()
        inp.hist_len[[1, 6]] = 0
        inp.hist_len[2] = 1
    if name == "ragged_empties_d128":
        inp.hist_len = inp.hist_len.copy()
        inp.hist_len[[0, 5, 19]] = 0
        inp.hist_len[7] = 1
    o_ref, lse_ref = oracle_round(inp)
    for engine in ("auto", "valu"):
        for label, kw in (("chunks", dict(split="chunks", chunks_per_slot=2)),
                          ("history cut", dict(split="balanced", history_slots=3))):
            log(f"[fp32] {name}: {engine}, {label}")
            rnd = rounds.ResidentRound(inp, engine=engine, **kw)
            rnd.run()
            torch.cuda.synchronize()
            compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
            check_mask(rnd, inp)
    rnd = rounds.ResidentRound(inp)
    work = ss.StateBuffers(rnd.problem, 12, "cuda")
    rnd.o.fill_(float("nan"))
    ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, 0, work, rnd.o,
                       rnd.lse)
    torch.cuda.synchronize()
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


F32_CUT_CASES = {
    # 16 streams over the whole device: every stream is cut into as many
    # pieces as it has slots, and with few slots the ranges grow
    "few_long_streams": C["c3_internlm25_7b_ragged"].with_(batch=2, dtype="f32", hist_len=20000, ragged_lo=5000,
                                                           chunk_len=1024),
    # 320 streams of odd lengths (none a multiple of 128), empties included
    "many_odd_streams": C["c3_internlm25_7b_ragged"].with_(batch=40, dtype="f32", hist_len=3001, ragged_lo=1,
                                                           chunk_len=256),
    "tree_d64": C["c3_internlm25_7b_ragged"].with_(batch=6, dtype="f32", head_dim=64, n_queries=8, mask="tree",
                                                   hist_len=9000, ragged_lo=1, chunk_len=512),
}


@pytest.mark.parametrize("slots", [2, 5, 8])
@pytest.mark.parametrize("name", list(F32_CUT_CASES))
def test_fp32_balanced_cut(name, slots):
    """Ragged fp32 histories on the balanced cut (the fp32 MFMA kernel's
    history launch, one work-group per CU walking its range) with 2, 5 and
    8 history slots match the oracle within 1e-5."""
    cfg = F32_CUT_CASES[name]
    assert rounds.f32_mfma(cfg) and cfg.ragged
    inp = wl.make_inputs(cfg)
    if name == "many_odd_streams":
        inp.hist_len = inp.hist_len.copy()
        inp.hist_len[[3, 17]] = 0
        # 128k + 1 tokens (never longer than generated): a one-token tail tile
        n = inp.hist_len[[4, 21]]
        assert (n >= 1).all()
        inp.hist_len[[4, 21]] = n - (n - 1) % 128
    o_ref, lse_ref = oracle_round(inp)
    log(f"[fp32 cut] {name}: {slots} slots")
    rnd = rounds.ResidentRound(inp, split="balanced", history_slots=slots)
    rnd.run()
    torch.cuda.synchronize()
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


FULL_VARIANTS = {
    "d64": C["c3_internlm25_7b_ragged"].with_(head_dim=64),
    "f32": C["c3_internlm25_7b_ragged"].with_(dtype="f32"),
    "tree_d64": C["c4_tree_72b"].with_(head_dim=64),
}


@pytest.mark.parametrize("variant", list(FULL_VARIANTS))
def test_full_size_sampled_variants(variant):
    """The InternLM2.5-like ragged layer at full size (32 requests up to
    65,536 tokens) with head_dim 64, and in fp32 (the fp32 MFMA kernel on the
    balanced cut), and the 72B-like tree round at full size (4 requests of
    131,072 tokens, 512 rows per KV head) with head_dim 64 (the wide-row
    kernel), in the benchmark's launch configuration, on sampled (request,
    KV head) slices against the oracle."""
    cfg = FULL_VARIANTS[variant]
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, **rounds.BENCH_RESIDENT)
    rnd.run()
    torch.cuda.synchronize()
    o, lse = rnd.o.cpu().numpy(), rnd.lse.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    check_mask(rnd, inp)
    for b, g in ((0, 0), (cfg.batch - 1, cfg.n_kv_heads - 1), (int(np.argmax(inp.hist_len)), 3)):
        log(f"[{variant} full] oracle slice b={b} g={g}")
        o_ref, lse_ref = oracle_round(inp, requests=[b], kv_heads=[g])
        compare(cfg, o, lse, o_ref, lse_ref, rows_of(cfg, b, g))


# ---------------------------------------------------------------------------
# size extremes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["one_request_1m_tokens", "many_short_requests", "max_candidates_tree",
                                  "history_above_2g_elements", "wide_history_above_2g_elements"])
def test_size_extremes(name):
    """One request with a million committed tokens (the balanced cut splits
    its streams over the whole device), 1024 requests with short ragged
    histories, the largest candidate region (64 tree nodes under 8-way GQA:
    512 rows), and histories whose K and V tensors hold more than 2^31
    elements each (2.15M tokens x 8 KV heads x 128; every offset past 2^31
    must be 64-bit: the narrow kernel, and the wide-row kernel with 40 rows),
    each in the benchmark's launch configuration; sampled (request, KV head)
    slices against the oracle (the last KV head lies past 2^31 elements)."""
    if name == "one_request_1m_tokens":
        cfg = C["c2_qwen3_8b"].with_(batch=1, hist_len=1 << 20, chunk_len=4096)
        picks = [(0, 0), (0, 5)]
    elif name == "history_above_2g_elements":
        cfg = C["c2_qwen3_8b"].with_(batch=1, hist_len=2_150_000, chunk_len=4096)
        assert cfg.n_kv_heads * cfg.hist_len * cfg.head_dim > 1 << 31
        picks = [(0, 0), (0, 7)]
    elif name == "wide_history_above_2g_elements":
        cfg = C["c4_tree_72b"].with_(batch=1, n_q_heads=8, n_kv_heads=8, n_queries=40, hist_len=2_150_000,
                                     chunk_len=4096)
        assert cfg.rows > 32 and cfg.n_kv_heads * cfg.hist_len * cfg.head_dim > 1 << 31
        picks = [(0, 7)]
    elif name == "many_short_requests":
        cfg = C["c3_internlm25_7b_ragged"].with_(batch=1024, hist_len=600, ragged_lo=300, chunk_len=256)
        picks = [(0, 0), (511, 3), (1023, 7)]
    else:
        cfg = C["c4_tree_72b"].with_(batch=2, hist_len=3000, chunk_len=1024)
        picks = [(0, 0), (1, 7)]
    log(f"[extremes] {name}: generating")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, **rounds.BENCH_RESIDENT)
    log(f"[extremes] {name}: {rnd.n_hist_slots} history slots, running")
    rnd.run()
    torch.cuda.synchronize()
    o = rnd.o.cpu().numpy()
    lse = rnd.lse.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    check_mask(rnd, inp)
    for b, g in picks:
        log(f"[extremes] {name}: oracle slice b={b} g={g}")
        o_ref, lse_ref = oracle_round(inp, requests=[b], kv_heads=[g])
        compare(cfg, o, lse, o_ref, lse_ref, rows_of(cfg, b, g))


def _random_case(seed):
    """A seeded random shape within the library's limits: dtype, head_dim,
    GQA group, queries and mask, lengths (uniform or ragged, head- or
    token-packed), chunk length, score scale, history cut, K/V layout,
    chunks per slot."""
    r = np.random.default_rng(7000 + seed)
    dtype = "f32" if r.random() < 0.15 else "bf16"
    head_dim = 64 if r.random() < 0.2 else 128
    n_kv = int(r.choice([1, 2, 3, 4]))
    group = int(r.choice([1, 2, 3, 4, 5, 8, 16]))
    mask = "tree" if r.random() < 0.4 else "causal"
    n_q = int(r.integers(2, 65)) if mask == "tree" else int(r.integers(1, 13))
    hist = int(r.integers(0, 3001))
    ragged_lo = int(r.integers(1, hist + 1)) if hist > 0 and r.random() < 0.5 else 0
    hist = max(hist, 1)  # a uniform view needs a token (empty histories: the ragged tests)
    cfg = C["c2_qwen3_8b"].with_(
        name=f"random{seed}", batch=int(r.integers(1, 7)), n_q_heads=n_kv * group, n_kv_heads=n_kv,
        head_dim=head_dim, dtype=dtype, hist_len=hist, chunk_len=int(r.choice([64, 100, 256, 320, 512, 1024])),
        n_queries=n_q, mask=mask, seed=100 + seed, ragged_lo=ragged_lo,
        packing="token" if ragged_lo and r.random() < 0.3 else "head")
    # a third of the bf16 cases use another score scale: small (flat weights)
    # or large (scores spread over tens of log2 units: the running maximum
    # moves by more than the kernels' rescale threshold and a few keys
    # dominate). fp32 cases keep 1/sqrt(d): at |lse| near 30 the 1e-5 bound is
    # a few fp32 ulps, which plain fp32 arithmetic itself does not meet.
    scale = float(r.choice([0.0, 0.0, 0.02, 0.3, 0.6])) if r.random() < 0.5 else 0.0
    cfg = cfg.with_(score_scale=scale if dtype == "bf16" else 0.0)
    kw = dict(split="balanced" if r.random() < 0.6 else "chunks",
              kv_layout="interleaved" if r.random() < 0.5 else "separate",
              chunks_per_slot=int(r.choice([1, 2, 3])), fuse_candidates=r.random() < 0.5)
    return cfg, kw


# SS_RANDOM_SEEDS=a:b widens the sweep (default 0:64)
RANDOM_SEEDS = range(*(int(x) for x in os.environ.get("SS_RANDOM_SEEDS", "0:64").split(":")))


@pytest.mark.parametrize("seed", RANDOM_SEEDS)
def test_random_shapes(seed):
    """Seeded random combinations of shape, mask, lengths, cut and layout
    against the fp64 oracle (O and lse at the tolerance, the mask bit for
    bit)."""
    cfg, kw = _random_case(seed)
    log(f"[random {seed}] {cfg} {kw}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp, **kw)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)


# SS_RANDOM_STREAMED_SEEDS=a:b widens the sweep (default 0:16)
RANDOM_STREAMED_SEEDS = range(*(int(x) for x in os.environ.get("SS_RANDOM_STREAMED_SEEDS", "0:16").split(":")))


@pytest.mark.parametrize("seed", RANDOM_STREAMED_SEEDS)
def test_random_streamed(seed):
    """The streamed round on seeded random shapes (heads, group, queries and
    mask, chunk length and count) and staging rings (buffers, chunks per
    copy), against the fp64 oracle."""
    r = np.random.default_rng(9000 + seed)
    n_kv = int(r.choice([1, 2, 4]))
    group = int(r.choice([1, 2, 4, 8]))
    mask = "tree" if r.random() < 0.4 else "causal"
    chunk = int(r.choice([128, 256, 500, 1024]))
    cfg = C["c5_streamed"].with_(
        name=f"streamed_random{seed}", batch=int(r.integers(1, 5)), n_q_heads=n_kv * group, n_kv_heads=n_kv,
        n_queries=int(r.integers(2, 33)) if mask == "tree" else int(r.integers(1, 9)), mask=mask,
        chunk_len=chunk, hist_len=chunk * int(r.integers(1, 9)), seed=200 + seed,
        score_scale=float(r.choice([0.0, 0.0, 0.3, 0.6])))
    n_buf, per_copy = int(r.integers(1, 4)), int(r.integers(1, 4))
    log(f"[streamed random {seed}] {cfg} n_buf={n_buf} chunks_per_copy={per_copy}")
    inp = wl.make_inputs(cfg)
    srd = rounds.StreamedRound(inp, n_buf=n_buf, chunks_per_copy=per_copy)
    srd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, srd.o.cpu().numpy(), srd.lse.cpu().numpy(), o_ref, lse_ref)


PEAKED = {
    # (config, engine): histories past the 2048-key short-history path
    "wide_r512_tree": (C["c4_tree_72b"].with_(batch=1, hist_len=6000, chunk_len=1024), "auto"),
    "wide_r96": (C["c2_qwen3_8b"].with_(batch=2, n_q_heads=32, n_kv_heads=2, n_queries=6, hist_len=5000,
                                        chunk_len=1024), "auto"),
    "narrow_r24": (C["c2_qwen3_8b"].with_(batch=2, hist_len=5000, chunk_len=1024), "auto"),
    "valu_small_r8": (C["c2_qwen3_8b"].with_(batch=2, n_queries=2, hist_len=5000, chunk_len=1024), "valu"),
    "bf16_d64": (C["c2_qwen3_8b"].with_(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, hist_len=3000,
                                        chunk_len=512), "auto"),
    "wide_r512_tree_d64": (C["c4_tree_72b"].with_(batch=1, head_dim=64, hist_len=6000, chunk_len=1024), "auto"),
    "wide_r96_d64": (C["c2_qwen3_8b"].with_(batch=2, n_q_heads=32, n_kv_heads=2, n_queries=6, head_dim=64,
                                            hist_len=5000, chunk_len=1024), "auto"),
}


@pytest.mark.parametrize("scale", [0.35, 0.7])
@pytest.mark.parametrize("name", list(PEAKED))
def test_peaked_scores(name, scale):
    """Score scales several times 1/sqrt(d) spread the scores over tens of
    log2 units, so a few keys dominate each row and the bf16 rounding of the
    weights no longer averages out over a long history: every kernel must
    still hold 2e-3 against the oracle (the wide-row kernel attends such
    pieces again with the weights' rounding remainders)."""
    cfg, engine = PEAKED[name]
    cfg = cfg.with_(score_scale=scale)
    log(f"[peaked] {name} scale={scale} rows={cfg.rows} history={cfg.hist_len}")
    inp = wl.make_inputs(cfg)
    for kw in (dict(split="chunks", chunks_per_slot=2), dict(rounds.BENCH_RESIDENT)):
        rnd = rounds.ResidentRound(inp, engine=engine, **kw)
        rnd.run()
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle_round(inp)
        compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("name", ["wide_r512_tree", "narrow_r24"])
def test_late_dominant_key(name):
    """Two keys, planted near the end of a long history, score far above all
    others for the rows of their KV head (their K rows are multiples of the
    group's mean query, of nearly equal length: two comparable dominant
    weights, whose rounding errors do not cancel): the rows are dominated
    only at the end of their last piece, at the default score scale."""
    cfg, engine = PEAKED[name]
    inp = wl.make_inputs(cfg)
    g = cfg.n_kv_heads - 1
    heads = slice(g * cfg.group, (g + 1) * cfg.group)
    qmean = inp.q[0, :, heads, :].float().mean(dim=(0, 1))
    t = cfg.hist_len - 37
    for dt, length in ((0, 60.0), (7, 58.0)):
        inp.k_hist[0, g, t + dt] = (qmean / qmean.norm() * length).to(inp.k_hist.dtype)
    log(f"[late keys] {name}: request 0, KV head {g}, tokens {t}, {t + 7}")
    rnd = rounds.ResidentRound(inp, engine=engine, **rounds.BENCH_RESIDENT)
    rnd.run()
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_round(inp)
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)


WIDE_RAGGED = {
    "tree_512_rows": C["c4_tree_72b"].with_(batch=6, hist_len=6000, ragged_lo=1, chunk_len=1024),
    "tree_128_rows": C["c4_tree_72b"].with_(batch=9, n_queries=16, hist_len=5000, ragged_lo=1, chunk_len=1024),
}


@pytest.mark.parametrize("slots", [2, 3, 8])
@pytest.mark.parametrize("name", list(WIDE_RAGGED))
def test_wide_ragged_balanced_cut(name, slots):
    """Ragged histories on the wide-row kernel (fixed chunks per slot, the
    candidate region with each stream's first chunk): with empty requests,
    requests below the short-history threshold and few or many slots, O, lse
    and the mask match the oracle, and so does the whole-round call."""
    cfg = WIDE_RAGGED[name]
    inp = wl.make_inputs(cfg)
    inp.hist_len = inp.hist_len.copy()
    inp.hist_len[[0, 4]] = 0
    inp.hist_len[1], inp.hist_len[2] = 1, 2047
    o_ref, lse_ref = oracle_round(inp)
    log(f"[wide ragged] {name}: {slots} slots, rows={cfg.rows}")
    rnd = rounds.ResidentRound(inp, **dict(rounds.BENCH_RESIDENT, history_slots=slots))
    for t in (rnd.state.acc, rnd.state.m, rnd.state.l):
        t.fill_(float("nan"))
    rnd.run()
    torch.cuda.synchronize()
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
    check_mask(rnd, inp)
    work = ss.StateBuffers(rnd.problem, 8, "cuda")
    rnd.o.fill_(float("nan"))
    ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, 0, work, rnd.o,
                       rnd.lse)
    torch.cuda.synchronize()
    compare(cfg, rnd.o.cpu().numpy(), rnd.lse.cpu().numpy(), o_ref, lse_ref)
