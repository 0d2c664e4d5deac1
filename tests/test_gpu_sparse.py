"""GPU parity of block statistics and block-sparse verification.

Importance of every history block (max over a KV head's rows of the block's
softmax mass in the full round) against the fp64 oracle within a bound
derived from the bf16 weights of the MFMA path; the selection bit for bit
against the oracle's selection run on the same fp32 importances; the sparse
result against the oracle's attention over the selected blocks and the
candidates.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import sparse
from long_context_speculative_amd import rounds
from long_context_speculative_amd import ssverify as ss
from long_context_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu
C = wl.CONFIGS
TOL = {"f32": 1e-5, "bf16": 2e-3}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cand_vis(inp):
    cfg = inp.cfg
    if cfg.mask == "tree":
        return np.stack([oracle.tree_mask(inp.parents[b]) for b in range(cfg.batch)])
    return np.stack([oracle.chain_mask(cfg.n_queries)] * cfg.batch)


CASES = {
    "c2_like": (C["c2_qwen3_8b"].with_(batch=2, hist_len=3000), 256, 4),
    "ragged": (C["c3_internlm25_7b_ragged"].with_(batch=4, hist_len=2500, ragged_lo=300), 128, 6),
    "tree_g8": (C["c4_tree_72b"].with_(batch=2, n_queries=4, hist_len=1100), 128, 3),
    "k_covers_all": (C["c2_qwen3_8b"].with_(batch=2, hist_len=900), 256, 8),
    "f32_valu": (C["c1_tiny_f32"].with_(hist_len=700), 64, 5),
    "wide_rows": (C["c4_tree_72b"].with_(batch=1, n_queries=12, hist_len=1300), 256, 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_importance_selection_and_sparse_round(name):
    cfg, block_len, k = CASES[name]
    log(f"[sparse] {name}: rows={cfg.rows}, block {block_len}, k {k}")
    inp = wl.make_inputs(cfg)
    sr = rounds.SparseRound(inp, block_len, k)
    sr.full()
    sr.select()
    sr.sparse()
    torch.cuda.synchronize()
    q = inp.q.float().numpy()
    kh, vh = inp.hist_per_request("k"), inp.hist_per_request("v")
    kc, vc = inp.k_cand.float().numpy(), inp.v_cand.float().numpy()
    vis = cand_vis(inp)
    # importance
    imp_ref = sparse.block_importance(q, kh, vh, inp.hist_len, kc, vis, cfg.scale, block_len, sr.n_blocks)
    imp = sr.importance.cpu().numpy().astype(np.float64)
    # bf16 weights move a block's l by at most 2^-8 relative (same weights in
    # l and in the row's normaliser); fp32 inputs leave float rounding only
    rel = 2 ** -8 if cfg.dtype == "bf16" else 1e-5
    err = np.abs(imp - imp_ref) - rel * imp_ref
    log(f"  importance: max|d| {np.abs(imp - imp_ref).max():.2e}, max mass {imp_ref.max():.3f}")
    assert err.max() <= 1e-6
    # selection on the same fp32 values: bit for bit
    sel = sr.selected.cpu().numpy()
    want = sparse.select_blocks(imp, inp.hist_len, block_len, k)
    assert np.array_equal(sel, want)
    # sparse verification
    o_ref, lse_ref = sparse.gathered_attention(q, kh, vh, inp.hist_len, block_len, sel, kc, vc, vis, cfg.scale)
    eo = np.abs(sr.o.cpu().numpy() - o_ref).max()
    el = np.abs(sr.lse.cpu().numpy() - lse_ref).max()
    log(f"  sparse: max|dO| {eo:.2e}, max|dlse| {el:.2e}")
    assert eo <= TOL[cfg.dtype] and el <= TOL[cfg.dtype]
    if name == "k_covers_all":
        # every block kept: the sparse round is the full round
        assert np.abs(sr.o.cpu().numpy() - sr.full_round.o.cpu().numpy()).max() <= 1e-5


def test_gathered_chunks_invalid_entries():
    """Entries < 0 or past a request's end give empty slots; a repeated entry
    attends its block twice (the caller's choice), others are exact."""
    cfg = C["c3_internlm25_7b_ragged"].with_(batch=3, hist_len=1000, ragged_lo=200)
    inp = wl.make_inputs(cfg)
    rr = rounds.ResidentRound(inp)
    pat = torch.tensor([[0, -1, 99], [3, 1, -5]], dtype=torch.int32).repeat(cfg.n_kv_heads // 2, 1)
    idx = pat.unsqueeze(0).repeat(cfg.batch, 1, 1).contiguous()       # [B][Hkv][3]
    idx_d = idx.cuda()
    st = ss.StateBuffers(rr.problem, 3, "cuda")
    for t in (st.acc, st.m, st.l):
        t.fill_(float("nan"))
    ss.ss_verify_chunk_gathered(rr.problem, rr.q, rr.hist_view, 128, idx_d, st, 0)
    torch.cuda.synchronize()
    m = st.m.cpu().numpy()
    l = st.l.cpu().numpy()
    ref_m, ref_l, _ = oracle.chunk_slot_states(inp.q.float().numpy(), inp.hist_per_request("k"),
                                               inp.hist_per_request("v"), inp.hist_len, 128, 0, 8, 1, cfg.scale)
    for b in range(cfg.batch):
        nblk = -(-int(inp.hist_len[b]) // 128)
        for g in range(cfg.n_kv_heads):
            hs = slice(g * cfg.group, (g + 1) * cfg.group)
            for s in range(3):
                j = int(idx[b, g, s])
                if j < 0 or j >= nblk:
                    assert np.isneginf(m[s, b][:, hs]).all() and (l[s, b][:, hs] == 0).all()
                else:
                    assert np.abs(m[s, b][:, hs] - ref_m[j, b][:, hs]).max() <= 2e-3


STATS_CASES = {
    # uniform lengths: ss_verify_history's equal-chunk cut, chunks rounded to blocks
    "c2_like_256": (C["c2_qwen3_8b"].with_(batch=2, hist_len=3000), 256, 4),
    "c2_like_128": (C["c2_qwen3_8b"].with_(batch=2, hist_len=2900), 128, 5),
    # ragged lengths: the balanced line cut, aligned to blocks
    "ragged_128": (C["c3_internlm25_7b_ragged"].with_(batch=4, hist_len=2500, ragged_lo=300), 128, 6),
    "ragged_512": (C["c3_internlm25_7b_ragged"].with_(batch=3, hist_len=9000, ragged_lo=700), 512, 4),
    "tree_g8": (C["c4_tree_72b"].with_(batch=2, n_queries=4, hist_len=1100), 128, 3),
}


@pytest.mark.parametrize("name", list(STATS_CASES))
def test_block_statistics_of_the_full_round(name):
    """Importance from the statistics the full round records as it goes:
    against the fp64 oracle within the bf16-weight bound, against the
    importance read from per-block state slots, and the full round's O and
    lse unchanged by the recording (bit for bit where the cut is the same)."""
    cfg, block_len, k = STATS_CASES[name]
    log(f"[stats] {name}: rows={cfg.rows}, block {block_len}, k {k}")
    inp = wl.make_inputs(cfg)
    sr = rounds.SparseRound(inp, block_len, k, stats=True)
    sr.full()
    sr.select()
    slots = rounds.SparseRound(inp, block_len, k)
    slots.full()
    slots.select()
    plain = rounds.ResidentRound(inp, **rounds.BENCH_RESIDENT)
    plain.run()
    torch.cuda.synchronize()
    q = inp.q.float().numpy()
    kh, vh = inp.hist_per_request("k"), inp.hist_per_request("v")
    kc = inp.k_cand.float().numpy()
    vis = cand_vis(inp)
    imp_ref = sparse.block_importance(q, kh, vh, inp.hist_len, kc, vis, cfg.scale, block_len, sr.n_blocks)
    imp = sr.importance.cpu().numpy().astype(np.float64)
    d = np.abs(imp - imp_ref)
    log(f"  stats importance: max|d| {d.max():.2e}, max mass {imp_ref.max():.3f}")
    assert (d - 2 ** -8 * imp_ref).max() <= 1e-6
    imp_slots = slots.importance.cpu().numpy().astype(np.float64)
    assert (np.abs(imp - imp_slots) - 2 ** -7 * imp_slots).max() <= 2e-6
    sel = sr.selected.cpu().numpy()
    assert np.array_equal(sel, sparse.select_blocks(imp, inp.hist_len, block_len, k))
    # the verification result is the round's, recording or not
    o_ref, lse_ref = oracle.attention_reference(q, kh, vh, inp.hist_len, kc, inp.v_cand.float().numpy(), vis,
                                                cfg.scale)
    o, lse = sr.full_round.o.cpu().numpy(), sr.full_round.lse.cpu().numpy()
    assert np.abs(o - o_ref).max() <= TOL[cfg.dtype] and np.abs(lse - lse_ref).max() <= TOL[cfg.dtype]
    if block_len == 128:
        assert torch.equal(sr.full_round.o, plain.o) and torch.equal(sr.full_round.lse, plain.lse)


def test_block_statistics_fewer_blocks_than_history():
    """Blocks past the buffer's n_blocks are not recorded; the recorded ones
    match those of a buffer that covers the whole history. The buffer needs
    no initialisation (it starts as NaN here): the importance reads only the
    entries the lengths say exist, and blocks past a request's end get 0."""
    cfg = C["c3_internlm25_7b_ragged"].with_(batch=3, hist_len=4000, ragged_lo=1500)
    inp = wl.make_inputs(cfg)
    rr = rounds.ResidentRound(inp, **rounds.BENCH_RESIDENT)
    full_blocks = -(-rr.max_len // 256) + 2
    imps = []
    for nb in (full_blocks, 5):
        rr.stats = ss.BlockStatsBuffer(rr.problem, 256, nb)
        rr.stats.buf.fill_(float("nan"))
        rr.run()
        imp = torch.full((cfg.batch, cfg.n_kv_heads, nb), -1.0, device="cuda")
        ss.ss_block_importance_stats(rr.problem, rr.stats, rr.hist_len, rr.max_len, rr.lse, imp)
        torch.cuda.synchronize()
        imps.append(imp.cpu())
    assert torch.equal(imps[1], imps[0][..., :5])
    assert torch.isfinite(imps[0]).all() and (imps[0] >= 0).all() and (imps[0][..., :5] > 0).any()
    for b, n in enumerate(inp.hist_len):
        nb = -(-int(n) // 256)
        assert (imps[0][b, :, :nb] > 0).all() and (imps[0][b, :, nb:] == 0).all()


GATHER_CASES = {
    # name: (config, block_len, k, chunks per slot)
    "c2_like_4": (C["c2_qwen3_8b"].with_(batch=2, hist_len=3000), 256, 6, 4),
    "ragged_3": (C["c3_internlm25_7b_ragged"].with_(batch=4, hist_len=2500, ragged_lo=300), 128, 7, 3),
    "tree_g8_all": (C["c4_tree_72b"].with_(batch=2, n_queries=4, hist_len=1100), 128, 5, 5),
}


@pytest.mark.parametrize("name", list(GATHER_CASES))
def test_gathered_chunks_merged_per_slot(name):
    """Several selected blocks merged into one slot (one work-group runs
    them one after the other): against the oracle's attention over the
    selected blocks, and against one block per slot."""
    cfg, block_len, k, per = GATHER_CASES[name]
    log(f"[gather] {name}: rows={cfg.rows}, block {block_len}, k {k}, {per} per slot")
    inp = wl.make_inputs(cfg)
    many = rounds.SparseRound(inp, block_len, k, gather_per_slot=per)
    one = rounds.SparseRound(inp, block_len, k, gather_per_slot=1)
    for sr in (many, one):
        sr.full()
        sr.select()
    # plant entries without keys: -1 and past the request's end
    sel = many.selected.clone()
    sel[:, :, 1] = -1
    sel[0, 0, 2] = 10_000
    for sr in (many, one):
        sr.selected.copy_(sel)
        for t in (sr.state.acc, sr.state.m, sr.state.l):
            t.fill_(float("nan"))
        sr.sparse()
    torch.cuda.synchronize()
    assert many.n_sparse_slots == -(-k // per)
    q = inp.q.float().numpy()
    kh, vh = inp.hist_per_request("k"), inp.hist_per_request("v")
    kc, vc = inp.k_cand.float().numpy(), inp.v_cand.float().numpy()
    o_ref, lse_ref = sparse.gathered_attention(q, kh, vh, inp.hist_len, block_len, sel.cpu().numpy(), kc, vc,
                                               cand_vis(inp), cfg.scale)
    eo = np.abs(many.o.cpu().numpy() - o_ref).max()
    el = np.abs(many.lse.cpu().numpy() - lse_ref).max()
    log(f"  merged slots: max|dO| {eo:.2e}, max|dlse| {el:.2e}")
    assert eo <= TOL[cfg.dtype] and el <= TOL[cfg.dtype]
    assert (many.o - one.o).abs().max().item() <= TOL[cfg.dtype]
    assert not torch.isnan(many.state.m).any() and not torch.isnan(many.state.acc).any()
