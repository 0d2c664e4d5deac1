"""Plain fp64 oracle for block importance statistics and block-sparse
(index-gathered) verification.

TEST INFRASTRUCTURE (same rules as the rest of ``oracle/``).

Sources, from the abstracts on the pages:
* SparseSpec-L: the per-head attention statistics that full-context
  verification already produces serve as an importance signal for recalling
  critical history, with no extra forward pass.
* Dustin: verification restricted to the critical tokens of the history,
  selected per head from the target's historical attention.

Readings (the abstracts fix no formula; these are the plainest ones that fit
SpecStream's block-wise states, section 4.2, Eq. 7-8):
* The history is cut into blocks of `block_len` tokens; block j of request b
  is [j*block_len, min((j+1)*block_len, N_b)).
* The importance of block j for KV head g is the largest attention mass any
  row of that head (query i, head h of the group) puts on the block in the
  full round's softmax (history and candidates): max_r sum_{t in block j}
  p_t(r). Blocks past a request's end have importance 0.
* Selection keeps, per (request, KV head), the k blocks of largest importance
  among the request's blocks; ties go to the lower block index; the kept
  indices are listed in increasing order, padded with -1.
* Block-sparse verification attends, for every row of KV head g, the kept
  blocks of that head plus the candidate region (under its mask): softmax
  over that union, exactly as the full round does over everything.
"""

from __future__ import annotations

import numpy as np

from .verify_attention import NEG_INF, visibility


def _rows(q, b, g, group):
    """Query rows of KV head g of request b, as (i, h) pairs in row order."""
    nq = q.shape[1]
    return [(i, g * group + hh) for i in range(nq) for hh in range(group)]


def block_importance(q, k_hist, v_hist, hist_len, k_cand, cand_vis, scale, block_len, n_blocks):
    """[B][Hkv][n_blocks] float64: max over the head's rows of the softmax mass
    of each history block (softmax over history + visible candidates)."""
    n_b, nq, hq, d = q.shape
    hkv = k_cand.shape[1]
    group = hq // hkv
    out = np.zeros((n_b, hkv, n_blocks))
    for b in range(n_b):
        n = int(hist_len[b])
        for g in range(hkv):
            keys = np.concatenate([np.asarray(k_hist[b][g][:n], dtype=np.float64),
                                   np.asarray(k_cand[b, g], dtype=np.float64)])
            vis = visibility(n, cand_vis[b])  # [nq][n + nc]
            for i, h in _rows(q, b, g, group):
                s = scale * (keys @ np.asarray(q[b, i, h], dtype=np.float64))
                s = np.where(vis[i], s, NEG_INF)
                m = s.max()
                w = np.where(vis[i], np.exp(s - m), 0.0)
                p = w / w.sum()
                for j in range(n_blocks):
                    t0, t1 = j * block_len, min((j + 1) * block_len, n)
                    if t0 < t1:
                        out[b, g, j] = max(out[b, g, j], p[t0:t1].sum())
    return out


def select_blocks(importance, hist_len, block_len, k):
    """[B][Hkv][k] int32: per (request, KV head) the indices of the k most
    important of the request's blocks (ties: lower index first), listed in
    increasing order, padded with -1."""
    n_b, hkv, n_blocks = importance.shape
    out = np.full((n_b, hkv, k), -1, dtype=np.int32)
    for b in range(n_b):
        valid = min(n_blocks, -(-int(hist_len[b]) // block_len))
        for g in range(hkv):
            order = sorted(range(valid), key=lambda j: (-importance[b, g, j], j))
            kept = sorted(order[:k])
            out[b, g, :len(kept)] = kept
    return out


def gathered_attention(q, k_hist, v_hist, hist_len, block_len, blocks, k_cand, v_cand, cand_vis, scale):
    """O [B][nq][Hq][d], lse [B][nq][Hq] of block-sparse verification: each
    row of KV head g attends the blocks blocks[b][g] (entries < 0 or past the
    request's end are ignored) and the visible candidates."""
    n_b, nq, hq, d = q.shape
    hkv = k_cand.shape[1]
    group = hq // hkv
    o = np.zeros((n_b, nq, hq, d))
    lse = np.full((n_b, nq, hq), NEG_INF)
    for b in range(n_b):
        n = int(hist_len[b])
        for g in range(hkv):
            idx = []
            for j in sorted(set(int(x) for x in blocks[b][g])):
                if j >= 0:
                    idx.extend(range(j * block_len, min((j + 1) * block_len, n)))
            idx = np.array(idx, dtype=np.int64)
            kh = np.asarray(k_hist[b][g], dtype=np.float64)[idx] if len(idx) else np.zeros((0, d))
            vh = np.asarray(v_hist[b][g], dtype=np.float64)[idx] if len(idx) else np.zeros((0, d))
            keys = np.concatenate([kh, np.asarray(k_cand[b, g], dtype=np.float64)])
            vals = np.concatenate([vh, np.asarray(v_cand[b, g], dtype=np.float64)])
            vis = visibility(len(idx), cand_vis[b])
            for i, h in _rows(q, b, g, group):
                s = scale * (keys @ np.asarray(q[b, i, h], dtype=np.float64))
                s = np.where(vis[i], s, NEG_INF)
                m = s.max()
                if m == NEG_INF:
                    continue
                w = np.where(vis[i], np.exp(s - m), 0.0)
                l = w.sum()
                o[b, i, h] = (w @ vals) / l
                lse[b, i, h] = m + np.log(l)
    return o, lse
