"""ss_verify_round_noalloc: the whole round with its state slots in the
library's static device array, for callers that cannot allocate. Checked
against ss_verify_round on a caller-allocated workspace (the same kernels
and the same cut, so the results are bit for bit the same) and against the
fp64 oracle at the parity tolerance, over consecutive calls whose later
inputs are smaller than the first (the array keeps the earlier call's
contents); and captured in a HIP graph and replayed, against the eager
call."""

import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_speculative_amd import rounds
from long_context_speculative_amd import ssverify as ss
from long_context_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu

C = wl.CONFIGS
TOL = {"f32": 1e-5, "bf16": 2e-3}

# Consecutive calls, each smaller than the one before it.
SEQUENCE = [
    ("narrow_ragged_large", C["c3_internlm25_7b_ragged"].with_(batch=24, hist_len=9000, ragged_lo=1,
                                                                chunk_len=1024)),
    ("wide_tree", C["c4_tree_72b"].with_(batch=2, hist_len=3000, chunk_len=1024)),
    # 256 streams of at most 2000 tokens: one slot per stream, O and lse from the history launch
    ("narrow_ragged_one_slot", C["c3_internlm25_7b_ragged"].with_(batch=32, hist_len=2000, ragged_lo=1,
                                                                  chunk_len=512)),
    ("narrow_uniform_small", C["c2_qwen3_8b"].with_(batch=2, hist_len=1500, chunk_len=512)),
    ("valu_small_rows", C["c2_qwen3_8b"].with_(batch=2, n_queries=2, hist_len=700, chunk_len=256)),
    ("f32_tiny", C["c1_tiny_f32"]),
]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle(inp):
    cfg = inp.cfg
    if cfg.mask == "tree":
        vis = np.stack([oracle.tree_mask(inp.parents[b]) for b in range(cfg.batch)])
    else:
        vis = np.stack([oracle.chain_mask(cfg.n_queries)] * cfg.batch)
    return oracle.attention_reference(inp.q.float().numpy(), inp.hist_per_request("k"), inp.hist_per_request("v"),
                                      inp.hist_len, inp.k_cand.float().numpy(), inp.v_cand.float().numpy(), vis,
                                      cfg.scale)


def test_noalloc_round_matches_workspace_round():
    for name, cfg in SEQUENCE:
        log(f"[no-alloc] {name}: B={cfg.batch} rows={cfg.rows} history<={cfg.hist_len}")
        inp = wl.make_inputs(cfg)
        rnd = rounds.ResidentRound(inp)
        work = ss.StateBuffers(rnd.problem, 64, "cuda")
        o_ws, lse_ws = torch.empty_like(rnd.o), torch.empty_like(rnd.lse)
        mask_ws = torch.full_like(rnd.mask_out, -1)
        ss.ss_verify_round(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, mask_ws, 0, work,
                           o_ws, lse_ws)
        rnd.o.fill_(float("nan"))
        rnd.lse.fill_(float("nan"))
        rnd.mask_out.fill_(-1)
        ss.ss_verify_round_noalloc(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out,
                                   rnd.o, rnd.lse)
        torch.cuda.synchronize()
        assert torch.equal(rnd.o, o_ws), name
        assert torch.equal(rnd.lse, lse_ws), name
        assert torch.equal(rnd.mask_out, mask_ws), name
        o_ref, lse_ref = _oracle(inp)
        eo = np.abs(rnd.o.cpu().numpy() - o_ref).max()
        el = np.abs(rnd.lse.cpu().numpy() - lse_ref).max()
        log(f"  {name}: identical to the workspace call; max|dO| {eo:.3e}, max|dlse| {el:.3e}")
        assert eo <= TOL[cfg.dtype] and el <= TOL[cfg.dtype], (eo, el)
        del rnd, work


def test_noalloc_round_rejects_oversized_state():
    """A round whose state slots do not fit in the static array is refused
    before anything is enqueued."""
    cfg = C["c2_qwen3_8b"].with_(batch=64, n_q_heads=64, n_kv_heads=8, n_queries=64, hist_len=128, chunk_len=128,
                                 mask="tree")
    slot_bytes = cfg.batch * cfg.n_queries * cfg.n_q_heads * (cfg.head_dim + 2) * 4
    assert slot_bytes > 64 << 20
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp)
    rnd.o.fill_(7.0)
    with pytest.raises(ss.SSError) as e:
        ss.ss_verify_round_noalloc(rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out,
                                   rnd.o, rnd.lse)
    assert e.value.code == ss.SS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (rnd.o == 7.0).all()


GRAPH_CASES = {
    "narrow_ragged": C["c3_internlm25_7b_ragged"].with_(batch=8, hist_len=5000, ragged_lo=1, chunk_len=1024),
    "wide_tree": C["c4_tree_72b"].with_(batch=2, hist_len=2600, chunk_len=1024),
    "narrow_ragged_one_slot": C["c3_internlm25_7b_ragged"].with_(batch=32, hist_len=1800, ragged_lo=1,
                                                                 chunk_len=512),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_noalloc_round_replayed_from_a_graph(name):
    """The callers the entry point is for capture it: the round recorded in a
    HIP graph (torch.cuda.graph on the capturing stream) and replayed four
    times, with other device work and a synchronisation between replays and
    the outputs poisoned before each, gives the eager call's O, lse and mask
    bit for bit every time."""
    cfg = GRAPH_CASES[name]
    log(f"[no-alloc graph] {name}: B={cfg.batch} rows={cfg.rows} history<={cfg.hist_len}")
    inp = wl.make_inputs(cfg)
    rnd = rounds.ResidentRound(inp)
    args = (rnd.problem, rnd.q, rnd.hist_view, rnd.cand_view, rnd.parents, rnd.mask_out, rnd.o, rnd.lse)
    ss.ss_verify_round_noalloc(*args)
    torch.cuda.synchronize()
    o_ref, lse_ref, mask_ref = rnd.o.clone(), rnd.lse.clone(), rnd.mask_out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ss.ss_verify_round_noalloc(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ss.ss_verify_round_noalloc(*args)
    other = torch.empty(1 << 22, device="cuda")
    for rep in range(4):
        rnd.o.fill_(float("nan"))
        rnd.lse.fill_(float("nan"))
        rnd.mask_out.fill_(-1)
        other.normal_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(rnd.o, o_ref), (name, rep)
        assert torch.equal(rnd.lse, lse_ref), (name, rep)
        assert torch.equal(rnd.mask_out, mask_ref), (name, rep)
        log(f"  replay {rep}: identical to the eager call")
    del graph
