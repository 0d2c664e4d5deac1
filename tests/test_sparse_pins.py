"""Pins for the block-importance and block-sparse verification oracle (CPU).

The statistics of SparseSpec-L (per-head attention mass recycled from full
verification) and the sparse verification of Dustin (attend only the
critical history) as read in oracle/sparse.py. Pinned by pure-Python brute
force of the per-row block masses, mass conservation, an independent top-k,
hand-worked ties, the full-selection special case (equals full attention),
the reduced-history special case (equals the pinned full-attention oracle on
a history made of the kept blocks), and the dropped-mass bound on the error
of the sparse result.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import sparse


def case(seed, b_=2, hq=4, hkv=2, d=8, n=(37, 20), nq=3, tree=False):
    rng = np.random.default_rng(seed)
    hist = [[rng.standard_normal((n[b], d)) for _ in range(hkv)] for b in range(b_)]
    vals = [[rng.standard_normal((n[b], d)) for _ in range(hkv)] for b in range(b_)]
    q = rng.standard_normal((b_, nq, hq, d))
    kc = rng.standard_normal((b_, hkv, nq, d))
    vc = rng.standard_normal((b_, hkv, nq, d))
    if tree:
        vis = np.stack([oracle.tree_mask(np.array([-1] + [int(rng.integers(0, i)) for i in range(1, nq)]))
                        for _ in range(b_)])
    else:
        vis = np.stack([oracle.chain_mask(nq)] * b_)
    return dict(q=q, k=hist, v=vals, n=np.array(n), kc=kc, vc=vc, vis=vis, scale=1 / math.sqrt(d))


def brute_masses(c, b, g, block_len, n_blocks):
    """Pure-Python per-row block masses of KV head g of request b."""
    q, hq, hkv = c["q"], c["q"].shape[2], c["kc"].shape[1]
    group = hq // hkv
    n = int(c["n"][b])
    out = []
    for i in range(q.shape[1]):
        for hh in range(group):
            h = g * group + hh
            sc = []
            for t in range(n):
                sc.append(c["scale"] * sum(q[b, i, h, x] * c["k"][b][g][t][x] for x in range(q.shape[3])))
            for j in range(c["kc"].shape[2]):
                if c["vis"][b][i][j]:
                    sc.append(c["scale"] * sum(q[b, i, h, x] * c["kc"][b, g, j, x] for x in range(q.shape[3])))
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            tot = math.fsum(w)
            masses = [math.fsum(w[t] for t in range(j * block_len, min((j + 1) * block_len, n))) / tot
                      for j in range(n_blocks)]
            cand = math.fsum(w[n:]) / tot
            out.append((masses, cand))
    return out


@pytest.mark.parametrize("block_len", [1, 5, 16, 64])
def test_importance_matches_brute_force_and_conserves_mass(block_len):
    c = case(1)
    n_blocks = -(-int(c["n"].max()) // block_len)
    imp = sparse.block_importance(c["q"], c["k"], c["v"], c["n"], c["kc"], c["vis"], c["scale"], block_len, n_blocks)
    for b in range(2):
        for g in range(2):
            rows = brute_masses(c, b, g, block_len, n_blocks)
            for masses, cand in rows:
                assert abs(math.fsum(masses) + cand - 1.0) < 1e-12     # every row's mass is accounted for
            want = np.max(np.array([m for m, _ in rows]), axis=0)
            assert np.abs(imp[b, g] - want).max() < 1e-12
            # blocks past the request's end carry nothing
            last = -(-int(c["n"][b]) // block_len)
            assert (imp[b, g, last:] == 0).all()


def test_select_blocks_ties_padding_and_independent_topk():
    imp = np.array([[[0.3, 0.5, 0.5, 0.1]]])
    assert sparse.select_blocks(imp, [40], 10, 2).tolist() == [[[1, 2]]]
    assert sparse.select_blocks(imp, [40], 10, 1).tolist() == [[[1]]]              # tie: lower index
    assert sparse.select_blocks(imp, [40], 10, 3).tolist() == [[[0, 1, 2]]]
    assert sparse.select_blocks(imp, [25], 10, 4).tolist() == [[[0, 1, 2, -1]]]    # 3 blocks hold the request
    assert sparse.select_blocks(imp, [0], 10, 2).tolist() == [[[-1, -1]]]
    rng = np.random.default_rng(5)
    for _ in range(200):
        nb = int(rng.integers(1, 30))
        imp = rng.integers(0, 5, size=(1, 1, nb)).astype(float)    # many ties
        n = int(rng.integers(0, nb * 8 + 1))
        k = int(rng.integers(1, nb + 3))
        got = sparse.select_blocks(imp, [n], 8, k)[0, 0]
        valid = min(nb, -(-n // 8))
        keys = np.lexsort((np.arange(valid), -imp[0, 0, :valid]))   # importance desc, then index asc
        want = np.sort(keys[:k])
        assert got[:len(want)].tolist() == want.tolist() and (got[len(want):] == -1).all()


def test_gathered_all_blocks_is_full_attention():
    c = case(2, tree=True)
    blocks = [[list(range(10)) for _ in range(2)] for _ in range(2)]
    o, lse = sparse.gathered_attention(c["q"], c["k"], c["v"], c["n"], 4, blocks, c["kc"], c["vc"], c["vis"],
                                       c["scale"])
    ro, rl = oracle.attention_reference(c["q"], c["k"], c["v"], c["n"], c["kc"], c["vc"], c["vis"], c["scale"])
    assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


def test_gathered_equals_full_attention_on_the_kept_history():
    c = case(3)
    block_len = 6
    blocks = [[[0, 3, -1], [5, 1, 2]], [[2, -1, -1], [0, 3, 1]]]
    o, lse = sparse.gathered_attention(c["q"], c["k"], c["v"], c["n"], block_len, blocks, c["kc"], c["vc"],
                                       c["vis"], c["scale"])
    # per (request, KV head) build the kept history by hand and run the
    # pinned full-attention oracle on it
    for b in range(2):
        for g in range(2):
            kept = sorted(j for j in blocks[b][g] if j >= 0)
            idx = [t for j in kept for t in range(j * block_len, min((j + 1) * block_len, int(c["n"][b])))]
            kh = [[c["k"][b][g][idx]]]
            vh = [[c["v"][b][g][idx]]]
            hs = slice(g * 2, g * 2 + 2)
            ro, rl = oracle.attention_reference(c["q"][b:b + 1, :, hs], kh, vh, np.array([len(idx)]),
                                                c["kc"][b:b + 1, g:g + 1], c["vc"][b:b + 1, g:g + 1],
                                                c["vis"][b:b + 1], c["scale"])
            assert np.abs(o[b][:, hs] - ro[0]).max() < 1e-12 and np.abs(lse[b][:, hs] - rl[0]).max() < 1e-12


def test_sparse_error_within_dropped_mass_bound():
    """|O_sparse - O_full| <= 2 * (dropped mass) * max|V| per row: the sparse
    output is the full softmax renormalised over the kept keys."""
    c = case(4, n=(200, 150), d=16)
    block_len = 16
    n_blocks = -(-200 // block_len)
    imp = sparse.block_importance(c["q"], c["k"], c["v"], c["n"], c["kc"], c["vis"], c["scale"], block_len, n_blocks)
    sel = sparse.select_blocks(imp, c["n"], block_len, 4)
    o, _ = sparse.gathered_attention(c["q"], c["k"], c["v"], c["n"], block_len, sel, c["kc"], c["vc"], c["vis"],
                                     c["scale"])
    ro, _ = oracle.attention_reference(c["q"], c["k"], c["v"], c["n"], c["kc"], c["vc"], c["vis"], c["scale"])
    vmax = max(max(np.abs(v).max() for v in c["v"][b]) for b in range(2))
    vmax = max(vmax, np.abs(c["vc"]).max())
    for b in range(2):
        for g in range(2):
            rows = brute_masses(c, b, g, block_len, n_blocks)
            kept = set(int(j) for j in sel[b, g] if j >= 0)
            for r, (masses, _) in enumerate(rows):
                i, h = r // 2, g * 2 + r % 2
                dropped = math.fsum(m for j, m in enumerate(masses) if j not in kept)
                assert np.abs(o[b, i, h] - ro[b, i, h]).max() <= 2 * dropped * vmax + 1e-12


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def test_pins_catch_planted_mistakes():
    imp = np.array([[[0.3, 0.5, 0.5, 0.1]]])
    # keeping the higher index on ties
    wrong = sorted(sorted(range(4), key=lambda j: (-imp[0, 0, j], -j))[:1])
    assert wrong != sparse.select_blocks(imp, [40], 10, 1)[0, 0].tolist()
    # importance from the history-only softmax (candidates left out) breaks
    # the brute-force match whenever candidates are visible
    c = case(6)
    n_blocks = 4
    imp_full = sparse.block_importance(c["q"], c["k"], c["v"], c["n"], c["kc"], c["vis"], c["scale"], 16, n_blocks)
    no_cand = np.zeros_like(c["vis"])
    imp_hist = sparse.block_importance(c["q"], c["k"], c["v"], c["n"], c["kc"], no_cand, c["scale"], 16, n_blocks)
    rows = brute_masses(c, 0, 0, 16, n_blocks)
    want = np.max(np.array([m for m, _ in rows]), axis=0)
    assert np.abs(imp_full[0, 0] - want).max() < 1e-12 and np.abs(imp_hist[0, 0] - want).max() > 1e-6
