"""Pins for the fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: the worked mask
example printed in the Speculative Streaming post, pure-Python brute force on
tiny inputs, torch's float64 scaled-dot-product attention, closed forms, and
the exactness statement of SpecStream section 4.2, Eq. (9) (chunked online
softmax equals one materialised softmax, whatever the chunking or order).
The last block plants plausible mistakes in copies of the oracle and checks
that the pins catch each of them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from long_context_speculative_amd import workloads

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------------------
# helpers that are NOT the oracle
# ---------------------------------------------------------------------------

def load_golden_mask(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append([int(x) for x in parts[1:]])
    return np.array(rows, dtype=bool)


def brute_force(q, k_hist, v_hist, hist_len, k_cand, v_cand, vis_fn, scale):
    """Pure-Python scalar loops: for every (request, query, head) list the
    visible keys, form the scores, and evaluate softmax and lse with math.exp
    and math.fsum. vis_fn(b, i, j) says whether candidate j is visible to
    query i of request b."""
    n_b, nq, hq, d = q.shape
    hkv = k_cand.shape[1]
    grp = hq // hkv
    o = np.zeros((n_b, nq, hq, d))
    lse = np.full((n_b, nq, hq), -math.inf)
    for b in range(n_b):
        for i in range(nq):
            for h in range(hq):
                g = h // grp
                keys, vals = [], []
                for t in range(int(hist_len[b])):
                    keys.append(k_hist[b][g][t])
                    vals.append(v_hist[b][g][t])
                for j in range(k_cand.shape[2]):
                    if vis_fn(b, i, j):
                        keys.append(k_cand[b, g, j])
                        vals.append(v_cand[b, g, j])
                if not keys:
                    continue
                scores = [scale * math.fsum(float(q[b, i, h, x]) * float(kk[x]) for x in range(d)) for kk in keys]
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                den = math.fsum(w)
                for x in range(d):
                    o[b, i, h, x] = math.fsum(w[t] * float(vals[t][x]) for t in range(len(w))) / den
                lse[b, i, h] = mx + math.log(den)
    return o, lse


def sdpa_reference(q, k_hist, v_hist, hist_len, k_cand, v_cand, cand_vis, scale):
    """torch's float64 CPU scaled_dot_product_attention with an explicit
    boolean mask over [history; candidates] and KV heads repeated per group;
    lse from torch.logsumexp over the masked scores."""
    n_b, nq, hq, d = q.shape
    hkv = k_cand.shape[1]
    grp = hq // hkv
    o = np.zeros((n_b, nq, hq, d))
    lse = np.zeros((n_b, nq, hq))
    for b in range(n_b):
        n = int(hist_len[b])
        kk = torch.cat([torch.as_tensor(np.stack([k_hist[b][g][:n] for g in range(hkv)]), dtype=torch.float64),
                        torch.as_tensor(k_cand[b], dtype=torch.float64)], dim=1)     # [Hkv][T][d]
        vv = torch.cat([torch.as_tensor(np.stack([v_hist[b][g][:n] for g in range(hkv)]), dtype=torch.float64),
                        torch.as_tensor(v_cand[b], dtype=torch.float64)], dim=1)
        kk = kk.repeat_interleave(grp, dim=0)                                        # [Hq][T][d]
        vv = vv.repeat_interleave(grp, dim=0)
        qq = torch.as_tensor(q[b], dtype=torch.float64).permute(1, 0, 2)             # [Hq][nq][d]
        mask = torch.cat([torch.ones(nq, n, dtype=torch.bool), torch.as_tensor(cand_vis[b])], dim=1)
        out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
        o[b] = out.permute(1, 0, 2).numpy()
        scores = torch.matmul(qq, kk.transpose(1, 2)) * scale
        scores = scores.masked_fill(~mask, float("-inf"))
        lse[b] = torch.logsumexp(scores, dim=-1).permute(1, 0).numpy()
    return o, lse


def small_case(b_=2, hq=4, hkv=2, d=8, n=37, nq=5, tree=False, seed=0, ragged=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b_, nq, hq, d))
    hist_len = (rng.integers(0, n + 1, size=b_) if ragged else np.full(b_, n)).astype(np.int64)
    k_hist = rng.standard_normal((b_, hkv, n, d))
    v_hist = rng.standard_normal((b_, hkv, n, d))
    k_cand = rng.standard_normal((b_, hkv, nq, d))
    v_cand = rng.standard_normal((b_, hkv, nq, d))
    if tree:
        parents = np.stack([workloads.draw_tree(seed, b, nq, 3) for b in range(b_)])
        cand_vis = np.stack([oracle.tree_mask(parents[b]) for b in range(b_)])
    else:
        parents = None
        cand_vis = np.stack([oracle.chain_mask(nq)] * b_)
    return dict(q=q, k_hist=k_hist, v_hist=v_hist, hist_len=hist_len, k_cand=k_cand, v_cand=v_cand,
                cand_vis=cand_vis, parents=parents, scale=1.0 / math.sqrt(d))


def run_ref(c, fn=oracle.attention_reference):
    return fn(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], c["k_cand"], c["v_cand"], c["cand_vis"], c["scale"])


# ---------------------------------------------------------------------------
# masks and index tables
# ---------------------------------------------------------------------------

def test_golden_block_causal_mask(golden_dir):
    gold = load_golden_mask(os.path.join(golden_dir, "block_causal_mask_6x6.txt"))
    assert gold.shape == (6, 6)
    # the speculation rows are the verification visibility for history 4, candidates 2
    vis = oracle.visibility(4, oracle.chain_mask(2))
    assert np.array_equal(vis, gold[4:6])
    # the context rows are an ordinary causal mask
    assert np.array_equal(oracle.chain_mask(4), gold[:4, :4])
    # a two-node chain tree gives the same candidate block
    assert np.array_equal(oracle.tree_mask([-1, 0]), gold[4:6, 4:6])


def test_chain_tree_equivalence_and_bits():
    for n in (1, 2, 5, 6, 33, 64):
        chain = oracle.chain_mask(n)
        assert np.array_equal(oracle.tree_mask([-1] + list(range(n - 1))), chain)
        bits = oracle.mask_to_bits(chain)
        assert [int(x) for x in bits] == [(1 << (i + 1)) - 1 for i in range(n)]


def test_tree_mask_hand_example():
    #        0
    #      /   \
    #     1     2
    #    / \     \
    #   3   4     5
    parents = [-1, 0, 0, 1, 1, 2]
    expect = [0b000001, 0b000011, 0b000101, 0b001011, 0b010011, 0b100101]
    assert [int(x) for x in oracle.mask_to_bits(oracle.tree_mask(parents))] == expect
    assert list(oracle.tree_depths(parents)) == [0, 1, 1, 2, 2, 2]


@pytest.mark.parametrize("seed", [0, 1, 4, 7])
def test_tree_mask_invariants(seed):
    n, cap = 64, 8
    parents = workloads.draw_tree(seed, 0, n, cap)
    vis = oracle.tree_mask(parents)
    depth = oracle.tree_depths(parents)
    for i in range(n):
        assert vis[i, i]
        assert not vis[i, i + 1:].any()                         # ancestors precede descendants
        if parents[i] >= 0:
            expect = vis[parents[i]].copy()
            expect[i] = True
            assert np.array_equal(vis[i], expect)               # anc[i] = anc[parent] | {i}
        assert vis[i].sum() == depth[i] + 1 <= cap + 1


def test_chunk_list_tiles_history():
    assert oracle.chunk_list([10], 4) == [(0, 0, 0, 4), (0, 1, 4, 4), (0, 2, 8, 2)]
    assert oracle.chunk_list([0, 3], 4) == [(1, 0, 0, 3)]
    lens = RNG.integers(0, 5000, size=9)
    for c in (1, 7, 64, 2048):
        lst = oracle.chunk_list(lens, c)
        for b, n in enumerate(lens):
            mine = [(s, ln) for (bb, j, s, ln) in lst if bb == b]
            covered = np.zeros(int(n), dtype=np.int64)
            for s, ln in mine:
                assert 0 < ln <= c and s % c == 0
                covered[s:s + ln] += 1
            assert (covered == 1).all()
            assert sum(ln for _, ln in mine) == n


# ---------------------------------------------------------------------------
# values: brute force, library cross-check, Eq. (9), closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tree", [False, True])
def test_brute_force_tiny(tree):
    c = small_case(b_=2 if tree else 1, hq=2 if not tree else 4, hkv=1 if not tree else 2, d=4, n=7,
                   nq=3 if not tree else 6, tree=tree, seed=3)
    o, lse = run_ref(c)
    vis = c["cand_vis"]
    bo, blse = brute_force(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], c["k_cand"], c["v_cand"],
                           lambda b, i, j: bool(vis[b, i, j]), c["scale"])
    assert np.abs(o - bo).max() <= 1e-13
    assert np.abs(lse - blse).max() <= 1e-13


@pytest.mark.parametrize("tree,ragged", [(False, False), (True, False), (False, True)])
def test_sdpa_cross_check(tree, ragged):
    c = small_case(b_=3, hq=8, hkv=2, d=32, n=300, nq=10 if tree else 6, tree=tree, seed=5, ragged=ragged)
    o, lse = run_ref(c)
    so, slse = sdpa_reference(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], c["k_cand"], c["v_cand"],
                              c["cand_vis"], c["scale"])
    assert np.abs(o - so).max() <= 1e-12
    assert np.abs(lse - slse).max() <= 1e-12


@pytest.mark.parametrize("order", ["forward", "reverse", "random"])
def test_chunked_equals_materialised(order):
    n = 333
    c = small_case(b_=2, hq=8, hkv=2, d=16, n=n, nq=6, seed=11, ragged=True)
    o, lse = run_ref(c)
    for chunk in (1, 7, 64, 128, n):
        co, clse = oracle.chunked_attention(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], c["k_cand"],
                                            c["v_cand"], c["cand_vis"], c["scale"], chunk, order=order,
                                            rng=np.random.default_rng(chunk))
        assert np.abs(co - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
        assert np.abs(clse - lse).max() <= 1e-12 * max(1.0, np.abs(lse).max())


def test_slots_then_merge_equal_materialised():
    c = small_case(b_=3, hq=8, hkv=2, d=16, n=500, nq=7, tree=True, seed=13, ragged=True)
    o, lse = run_ref(c)
    for chunk, cps in ((64, 1), (64, 3), (100, 2), (512, 1)):
        n_chunks = -(-500 // chunk)
        m, l, acc = oracle.chunk_slot_states(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], chunk, 0,
                                             n_chunks, cps, c["scale"])
        cm, cl, cacc = oracle.candidate_state(c["q"], c["k_cand"], c["v_cand"], c["cand_vis"], c["scale"])
        mo, mlse = oracle.merge_slots(np.concatenate([m, cm[None]]), np.concatenate([l, cl[None]]),
                                      np.concatenate([acc, cacc[None]]))
        assert np.abs(mo - o).max() <= 1e-12
        assert np.abs(mlse - lse).max() <= 1e-12


def test_closed_form_zero_query():
    c = small_case(b_=2, hq=4, hkv=2, d=8, n=20, nq=5, seed=17, ragged=True)
    c["q"] = np.zeros_like(c["q"])
    o, lse = run_ref(c)
    for b in range(2):
        n = int(c["hist_len"][b])
        for i in range(5):
            for h in range(4):
                g = h // 2
                vals = np.concatenate([c["v_hist"][b, g, :n], c["v_cand"][b, g, :i + 1]])
                assert np.allclose(o[b, i, h], vals.mean(axis=0), rtol=0, atol=1e-14)
                assert abs(lse[b, i, h] - math.log(n + i + 1)) <= 1e-14


def test_closed_form_single_visible_key():
    c = small_case(b_=1, hq=2, hkv=1, d=8, n=0, nq=4, seed=19)
    o, lse = run_ref(c)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], c["v_cand"][0, 0, 0])
        s = c["scale"] * math.fsum(c["q"][0, 0, h] * c["k_cand"][0, 0, 0])
        assert abs(lse[0, 0, h] - s) <= 1e-14


def test_closed_form_uniform_keys():
    c = small_case(b_=1, hq=4, hkv=1, d=8, n=50, nq=3, seed=23)
    c["k_hist"][:] = c["k_hist"][0, 0, 0]
    c["k_cand"][:] = c["k_hist"][0, 0, 0]
    o, _ = run_ref(c)
    for i in range(3):
        vals = np.concatenate([c["v_hist"][0, 0], c["v_cand"][0, 0, :i + 1]])
        assert np.allclose(o[0, i], vals.mean(axis=0)[None], rtol=0, atol=1e-13)


def test_closed_form_needle():
    c = small_case(b_=1, hq=4, hkv=1, d=16, n=400, nq=3, seed=29)
    u = RNG.standard_normal(16)
    u /= np.linalg.norm(u)
    c["q"][:] = u
    big = 40.0
    t = 257
    c["k_hist"][0, 0, t] = big / c["scale"] * u
    o, lse = run_ref(c)
    assert np.abs(o - c["v_hist"][0, 0, t]).max() <= 1e-10
    assert np.abs(lse - big).max() <= 1e-10


def test_empty_visibility():
    c = small_case(b_=1, hq=2, hkv=1, d=8, n=0, nq=3, seed=31)
    c["cand_vis"] = np.zeros_like(c["cand_vis"])
    o, lse = run_ref(c)
    assert (o == 0).all() and np.isneginf(lse).all()
    m, l, acc = oracle.chunk_slot_states(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], 4, 0, 3, 1, c["scale"])
    assert np.isneginf(m).all() and (l == 0).all() and (acc == 0).all()


def test_merge_identity_and_order():
    rows, d = 6, 5
    states = []
    for k in range(4):
        states.append((RNG.standard_normal(rows) * 3, RNG.random(rows) + 0.1, RNG.standard_normal((rows, d))))
    empty = oracle.empty_state((rows,), d)
    for s in states:
        e = oracle.merge_states(empty, s)
        assert all(np.array_equal(x, y) for x, y in zip(e, s))
    a = oracle.merge_states(oracle.merge_states(states[0], states[1]), oracle.merge_states(states[2], states[3]))
    b = states[3]
    for s in (states[2], states[0], states[1]):
        b = oracle.merge_states(b, s)
    oa, la = oracle.finalize(a)
    ob, lb = oracle.finalize(b)
    assert np.abs(oa - ob).max() <= 1e-13 and np.abs(la - lb).max() <= 1e-13


def test_candidate_visibility_perturbation():
    c = small_case(b_=2, hq=6, hkv=2, d=8, n=30, nq=12, tree=True, seed=37)
    o0, l0 = run_ref(c)
    grp = 3
    for b in range(2):
        for j in (0, 3, 11):
            for g in range(2):
                c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
                c2["k_cand"][b, g, j] += 1.5
                c2["v_cand"][b, g, j] -= 2.0
                o1, l1 = run_ref(c2)
                for bb in range(2):
                    for i in range(12):
                        for h in range(6):
                            affected = bb == b and h // grp == g and c["cand_vis"][b, i, j]
                            same = np.array_equal(o0[bb, i, h], o1[bb, i, h]) and l0[bb, i, h] == l1[bb, i, h]
                            assert same != affected, (b, j, g, bb, i, h)


def test_gqa_head_permutation():
    c = small_case(b_=1, hq=8, hkv=2, d=8, n=40, nq=4, seed=41)
    o, lse = run_ref(c)
    perm = np.array([2, 0, 3, 1, 7, 5, 4, 6])        # permutes heads inside each group of 4
    c2 = dict(c)
    c2["q"] = c["q"][:, :, perm, :]
    o2, lse2 = run_ref(c2)
    assert np.abs(o2 - o[:, :, perm, :]).max() <= 1e-14
    assert np.abs(lse2 - lse[:, :, perm]).max() <= 1e-14


# ---------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# ---------------------------------------------------------------------------

def _mutant_no_diagonal(c):
    c2 = dict(c)
    c2["cand_vis"] = np.stack([np.tril(np.ones_like(v), -1) for v in c["cand_vis"]])
    return run_ref(c2)


def _mutant_wrong_gqa(c):
    # maps query head h to KV head h % Hkv instead of h // G
    q = c["q"]
    hq = q.shape[2]
    hkv = c["k_cand"].shape[1]
    grp = hq // hkv
    order = np.array([(h % hkv) * grp + h // hkv for h in range(hq)])
    inv = np.argsort(order)
    c2 = dict(c)
    c2["q"] = q[:, :, order, :]
    o, lse = run_ref(c2)
    return o[:, :, inv, :], lse[:, :, inv]


def _mutant_no_rescale(c):
    # merges chunk states without aligning them to a common maximum
    n_b, nq, hq, d = c["q"].shape
    m, l, acc = oracle.chunk_slot_states(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], 8, 0, 8, 1, c["scale"])
    cm, cl, cacc = oracle.candidate_state(c["q"], c["k_cand"], c["v_cand"], c["cand_vis"], c["scale"])
    L = l.sum(0) + cl
    A = acc.sum(0) + cacc
    return A / L[..., None], np.maximum(m.max(0), cm) + np.log(L)


def _mutant_drop_last_chunk(c):
    c2 = dict(c)
    c2["hist_len"] = np.maximum(c["hist_len"] - 8, 0)
    return run_ref(c2)


def _mutant_unscaled(c):
    c2 = dict(c)
    c2["scale"] = 1.0
    return run_ref(c2)


@pytest.mark.parametrize("mutant", [_mutant_no_diagonal, _mutant_wrong_gqa, _mutant_no_rescale,
                                    _mutant_drop_last_chunk, _mutant_unscaled])
def test_pins_catch_planted_mistakes(mutant):
    c = small_case(b_=2, hq=8, hkv=2, d=16, n=60, nq=6, seed=43)
    mo, mlse = mutant(c)
    so, slse = sdpa_reference(c["q"], c["k_hist"], c["v_hist"], c["hist_len"], c["k_cand"], c["v_cand"],
                              c["cand_vis"], c["scale"])
    err = max(np.abs(mo - so).max(), np.abs(mlse - slse).max())
    assert err > 1e-6, f"{mutant.__name__} slipped past the SDPA pin"
