"""fp64 CPU oracle for multi-query verification attention.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module. The product path (the HIP library
and its Python binding) never calls it, and this module imports nothing from
the product package.

What it computes is the plain definition, written out in float64:

* SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
  Serving"), section 4.2, Eq. (6): every query of a verification round attends,
  under one softmax, to the committed history followed by the GPU-resident
  candidate rows, with a mask M over the candidate rows. The history is
  visible to the whole query group; a candidate row is visible to a query only
  if the mask says so.
* Eq. (7): the local state (m, l, a) of a block of keys, with m the maximum
  score over the block, l the sum of exponentials relative to m and a the
  matching weighted sum of values.
* Eq. (8): the merge of two such states onto a common maximum.
* Eq. (9): a / l is the full softmax output over the visible keys.

Readings of points the pages leave open (each is also listed in the design
notes):

* Scores are scale * <q, k> with scale = 1 / sqrt(d_h) (section 4.2, the
  definition of S_j); the caller passes the scale it uses.
* lse is the natural log of the softmax denominator over scaled scores:
  lse = m + ln(l).
* GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
* Candidate visibility: chain (causal) = candidate j visible to query i iff
  j <= i (the diagonal is visible, as in the block-causal example of the
  Speculative Streaming post, section 2); tree = the ancestors of node i,
  itself included, found by walking parent pointers.
* A query that sees no key at all keeps the initial state (-inf, 0, 0)
  (section 4.2); its output is O = 0 and lse = -inf.
* Chunk j of a request with N committed tokens covers [j*C, min((j+1)*C, N)).

Layouts (logical; all arrays are numpy, any float dtype, upcast to float64):
  q       [B][nq][Hq][d]
  k_hist  per request b an array [Hkv][N_b][d] (a list, or a 4-D array whose
          third axis is at least N_b long)
  k_cand  [B][Hkv][nc][d]
  cand_vis[B][nq][nc] bool
  O       [B][nq][Hq][d],  lse [B][nq][Hq]
  state   m, l [B][nq][Hq],  acc [B][nq][Hq][d]
"""

from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# Masks and index tables (integer work: results must match bit for bit)
# ---------------------------------------------------------------------------

def chain_mask(n_cand: int) -> np.ndarray:
    """Causal visibility inside the candidate region (SpecStream section 4.2,
    the masked GPU region): query i sees candidate j iff j <= i."""
    i = np.arange(n_cand)[:, None]
    j = np.arange(n_cand)[None, :]
    return j <= i


def tree_mask(parents) -> np.ndarray:
    """Ancestor visibility for a candidate tree (single-pass tree verification
    of the Speculative Streaming post, section 3): node i sees itself and
    every node on its path to the root. parents[i] == -1 marks a root.

    The walk goes node by node up the parent pointers; it does not use the
    recursive bitmask construction the GPU path uses."""
    parents = [int(p) for p in parents]
    n = len(parents)
    vis = np.zeros((n, n), dtype=bool)
    for i in range(n):
        node = i
        steps = 0
        while node != -1:
            if not (0 <= node < n):
                raise ValueError(f"parent pointer {node} out of range")
            vis[i, node] = True
            node = parents[node]
            steps += 1
            if steps > n:
                raise ValueError("parent pointers contain a cycle")
    return vis


def tree_depths(parents) -> np.ndarray:
    """Depth (edges to the root) of every node, by walking parent pointers."""
    parents = [int(p) for p in parents]
    out = np.zeros(len(parents), dtype=np.int64)
    for i in range(len(parents)):
        node, depth = parents[i], 0
        while node != -1:
            depth += 1
            node = parents[node]
        out[i] = depth
    return out


def mask_to_bits(vis: np.ndarray) -> np.ndarray:
    """Pack a dense [n][n] visibility matrix (n <= 64) into one uint64 per
    row: bit j of row i is set iff row i sees candidate j."""
    n_rows, n_cols = vis.shape
    if n_cols > 64:
        raise ValueError("at most 64 candidates fit one 64-bit row")
    out = np.zeros(n_rows, dtype=np.uint64)
    for i in range(n_rows):
        word = 0
        for j in range(n_cols):
            if vis[i, j]:
                word |= 1 << j
        out[i] = np.uint64(word)
    return out


def chunk_list(req_len, chunk_len: int):
    """History chunking (SpecStream section 4.2): the committed history of
    request b is cut into contiguous chunks along token positions.
    Returns [(b, j, start, length)] in request order, then chunk order."""
    if chunk_len <= 0:
        raise ValueError("chunk_len must be positive")
    out = []
    for b, n in enumerate(req_len):
        n = int(n)
        j = 0
        while j * chunk_len < n:
            start = j * chunk_len
            out.append((b, j, start, min(chunk_len, n - start)))
            j += 1
    return out


def visibility(hist_len: int, cand_vis: np.ndarray) -> np.ndarray:
    """Full visibility row set [nq][hist_len + nc] of one request: the
    committed history is visible to every query of the round (SpecStream
    section 4.2), candidates follow the candidate mask."""
    nq = cand_vis.shape[0]
    return np.concatenate([np.ones((nq, hist_len), dtype=bool), cand_vis.astype(bool)], axis=1)


# ---------------------------------------------------------------------------
# Eq. (6): materialised softmax attention over history + candidates
# ---------------------------------------------------------------------------

def _hist_slice(k_hist, b: int, g: int, n: int) -> np.ndarray:
    return np.asarray(k_hist[b][g][:n], dtype=np.float64)


def attention_slice(q_rows, keys, vals, vis_rows, scale):
    """One (request, KV head) slice of Eq. (6), materialised.

    q_rows [R][d], keys/vals [T][d], vis_rows [R][T] bool.
    Returns O [R][d] and lse [R] in float64."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    vis_rows = np.asarray(vis_rows, dtype=bool)
    n_rows, d = q_rows.shape
    o = np.zeros((n_rows, d), dtype=np.float64)
    lse = np.full(n_rows, NEG_INF, dtype=np.float64)
    if keys.shape[0] == 0:
        return o, lse
    s = float(scale) * (q_rows @ keys.T)                 # [R][T]
    s = np.where(vis_rows, s, NEG_INF)
    m = s.max(axis=1)                                     # -inf where nothing visible
    seen = np.isfinite(m)
    w = np.zeros_like(s)
    w[seen] = np.where(vis_rows[seen], np.exp(s[seen] - m[seen, None]), 0.0)
    l = w.sum(axis=1)
    p = np.zeros_like(w)
    p[seen] = w[seen] / l[seen, None]
    o = p @ vals
    lse[seen] = m[seen] + np.log(l[seen])
    return o, lse


def attention_reference(q, k_hist, v_hist, hist_len, k_cand, v_cand, cand_vis, scale,
                        requests=None, kv_heads=None):
    """Eq. (6) for every request and head (or the listed subsets).

    Returns O [B][nq][Hq][d] and lse [B][nq][Hq] (float64); rows of requests
    or KV heads not listed are left at O = 0, lse = -inf."""
    q = np.asarray(q)
    n_b, nq, hq, d = q.shape
    hkv = int(k_cand.shape[1]) if k_cand is not None else len(k_hist[0])
    grp = hq // hkv
    o = np.zeros((n_b, nq, hq, d), dtype=np.float64)
    lse = np.full((n_b, nq, hq), NEG_INF, dtype=np.float64)
    reqs = range(n_b) if requests is None else requests
    heads = range(hkv) if kv_heads is None else kv_heads
    for b in reqs:
        n = int(hist_len[b])
        nc = 0 if k_cand is None else int(k_cand.shape[2])
        vis = visibility(n, np.asarray(cand_vis[b]) if nc else np.zeros((nq, 0), bool))
        for g in heads:
            keys = _hist_slice(k_hist, b, g, n)
            vals = _hist_slice(v_hist, b, g, n)
            if nc:
                keys = np.concatenate([keys, np.asarray(k_cand[b, g], dtype=np.float64)])
                vals = np.concatenate([vals, np.asarray(v_cand[b, g], dtype=np.float64)])
            # rows of the slice: (query i, head-in-group hh), query-major
            rows = np.asarray(q[b, :, g * grp:(g + 1) * grp, :], dtype=np.float64).reshape(nq * grp, d)
            vis_rows = np.repeat(vis, grp, axis=0)
            o_s, lse_s = attention_slice(rows, keys, vals, vis_rows, scale)
            o[b, :, g * grp:(g + 1) * grp, :] = o_s.reshape(nq, grp, d)
            lse[b, :, g * grp:(g + 1) * grp] = lse_s.reshape(nq, grp)
    return o, lse


# ---------------------------------------------------------------------------
# Eq. (7)-(9): partial states, merge, finalise
# ---------------------------------------------------------------------------

def empty_state(shape_rows, d):
    """The initial state (-inf, 0, 0) of section 4.2."""
    return (np.full(shape_rows, NEG_INF), np.zeros(shape_rows), np.zeros(tuple(shape_rows) + (d,)))


def local_state(q_rows, keys, vals, vis_rows, scale):
    """Eq. (7): the local state of one block of keys for each row, taken over
    the keys visible to that row. Rows that see none get (-inf, 0, 0)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    n_rows, d = q_rows.shape
    m = np.full(n_rows, NEG_INF)
    l = np.zeros(n_rows)
    acc = np.zeros((n_rows, d))
    keys = np.asarray(keys, dtype=np.float64)
    if keys.shape[0] == 0:
        return m, l, acc
    vals = np.asarray(vals, dtype=np.float64)
    vis_rows = np.asarray(vis_rows, dtype=bool)
    s = float(scale) * (q_rows @ keys.T)
    s = np.where(vis_rows, s, NEG_INF)
    m = s.max(axis=1)
    seen = np.isfinite(m)
    e = np.zeros_like(s)
    e[seen] = np.where(vis_rows[seen], np.exp(s[seen] - m[seen, None]), 0.0)
    l = e.sum(axis=1)
    acc = e @ vals
    return m, l, acc


def _scale_factor(m_old, m_new):
    """e^(m_old - m_new), taken as 0 where m_old is -inf (an empty state)."""
    out = np.zeros_like(m_old, dtype=np.float64)
    ok = np.isfinite(m_old)
    out[ok] = np.exp(m_old[ok] - m_new[ok])
    return out


def merge_states(state_a, state_b):
    """Eq. (8): rescale two states to the common maximum and add."""
    m_a, l_a, acc_a = state_a
    m_b, l_b, acc_b = state_b
    m_a = np.asarray(m_a, dtype=np.float64)
    m_b = np.asarray(m_b, dtype=np.float64)
    m_new = np.maximum(m_a, m_b)
    alpha = _scale_factor(m_a, m_new)
    beta = _scale_factor(m_b, m_new)
    l_new = alpha * l_a + beta * l_b
    acc_new = alpha[..., None] * acc_a + beta[..., None] * acc_b
    return m_new, l_new, acc_new


def finalize(state):
    """O = a / l (section 4.2, after the last block) and lse = m + ln l.
    A row with l == 0 saw nothing: O = 0, lse = -inf."""
    m, l, acc = state
    seen = l > 0
    o = np.zeros_like(acc)
    o[seen] = acc[seen] / l[seen][..., None]
    lse = np.full(m.shape, NEG_INF)
    lse[seen] = m[seen] + np.log(l[seen])
    return o, lse


def chunk_slot_states(q, k_hist, v_hist, hist_len, chunk_len, chunk_begin, n_chunks,
                      chunks_per_slot, scale, requests=None, kv_heads=None):
    """The per-slot history states a chunk call defines: slot s holds the
    local state (Eq. 7) over the union of chunks
    [chunk_begin + s*cps, chunk_begin + (s+1)*cps) of each request, clipped
    to [0, N_b). Every history key is visible to every query. A slot with no
    key is (-inf, 0, 0).

    Returns m, l [S][B][nq][Hq] and acc [S][B][nq][Hq][d]."""
    q = np.asarray(q)
    n_b, nq, hq, d = q.shape
    hkv = len(k_hist[0])
    grp = hq // hkv
    n_slots = -(-n_chunks // chunks_per_slot)
    m = np.full((n_slots, n_b, nq, hq), NEG_INF)
    l = np.zeros((n_slots, n_b, nq, hq))
    acc = np.zeros((n_slots, n_b, nq, hq, d))
    reqs = range(n_b) if requests is None else requests
    heads = range(hkv) if kv_heads is None else kv_heads
    for s in range(n_slots):
        c0 = chunk_begin + s * chunks_per_slot
        c1 = min(chunk_begin + n_chunks, c0 + chunks_per_slot)
        for b in reqs:
            n = int(hist_len[b])
            t0, t1 = min(c0 * chunk_len, n), min(c1 * chunk_len, n)
            for g in heads:
                rows = np.asarray(q[b, :, g * grp:(g + 1) * grp, :], dtype=np.float64).reshape(nq * grp, d)
                keys = np.asarray(k_hist[b][g][t0:t1], dtype=np.float64)
                vals = np.asarray(v_hist[b][g][t0:t1], dtype=np.float64)
                vis_rows = np.ones((nq * grp, t1 - t0), dtype=bool)
                ms, ls, accs = local_state(rows, keys, vals, vis_rows, scale)
                m[s, b, :, g * grp:(g + 1) * grp] = ms.reshape(nq, grp)
                l[s, b, :, g * grp:(g + 1) * grp] = ls.reshape(nq, grp)
                acc[s, b, :, g * grp:(g + 1) * grp, :] = accs.reshape(nq, grp, d)
    return m, l, acc


def candidate_state(q, k_cand, v_cand, cand_vis, scale, requests=None, kv_heads=None):
    """The state of the candidate region alone (section 4.2, GPU region under
    the candidate mask), one slot: m, l [B][nq][Hq], acc [B][nq][Hq][d]."""
    q = np.asarray(q)
    n_b, nq, hq, d = q.shape
    hkv = int(k_cand.shape[1])
    grp = hq // hkv
    m = np.full((n_b, nq, hq), NEG_INF)
    l = np.zeros((n_b, nq, hq))
    acc = np.zeros((n_b, nq, hq, d))
    reqs = range(n_b) if requests is None else requests
    heads = range(hkv) if kv_heads is None else kv_heads
    for b in reqs:
        vis_rows = np.repeat(np.asarray(cand_vis[b], dtype=bool), grp, axis=0)
        for g in heads:
            rows = np.asarray(q[b, :, g * grp:(g + 1) * grp, :], dtype=np.float64).reshape(nq * grp, d)
            ms, ls, accs = local_state(rows, k_cand[b, g], v_cand[b, g], vis_rows, scale)
            m[b, :, g * grp:(g + 1) * grp] = ms.reshape(nq, grp)
            l[b, :, g * grp:(g + 1) * grp] = ls.reshape(nq, grp)
            acc[b, :, g * grp:(g + 1) * grp, :] = accs.reshape(nq, grp, d)
    return m, l, acc


def merge_slots(m, l, acc, slots_per_req=None):
    """Fold slots [0, n) of every request with Eq. (8) in slot order, then
    finalise. m, l [S][B][nq][Hq]; acc [S][B][nq][Hq][d]; slots_per_req [B]
    (None = all S). Returns O [B][nq][Hq][d], lse [B][nq][Hq]."""
    n_s, n_b = m.shape[0], m.shape[1]
    d = acc.shape[-1]
    o = np.zeros(acc.shape[1:])
    lse = np.full(m.shape[1:], NEG_INF)
    for b in range(n_b):
        count = n_s if slots_per_req is None else int(slots_per_req[b])
        state = empty_state(m.shape[2:], d)
        for s in range(count):
            state = merge_states(state, (m[s, b], l[s, b], acc[s, b]))
        o[b], lse[b] = finalize(state)
    return o, lse


def chunked_attention(q, k_hist, v_hist, hist_len, k_cand, v_cand, cand_vis, scale,
                      chunk_len, order="forward", rng=None):
    """The streaming procedure of section 4.2, in float64: start from (-inf, 0, 0),
    fold in the local state of every history chunk (Eq. 7-8) in the given
    order, then the candidate region, then O = a / l.

    order: "forward", "reverse" or "random" (a permutation drawn from rng).
    Used to pin Eq. (9): the result must not depend on chunking or order."""
    q = np.asarray(q)
    n_b, nq, hq, d = q.shape
    hkv = len(k_hist[0])
    grp = hq // hkv
    o = np.zeros((n_b, nq, hq, d))
    lse = np.full((n_b, nq, hq), NEG_INF)
    for b in range(n_b):
        n = int(hist_len[b])
        starts = list(range(0, n, chunk_len))
        if order == "reverse":
            starts = starts[::-1]
        elif order == "random":
            starts = [starts[i] for i in rng.permutation(len(starts))]
        vis_c = np.repeat(np.asarray(cand_vis[b], dtype=bool), grp, axis=0)
        for g in range(hkv):
            rows = np.asarray(q[b, :, g * grp:(g + 1) * grp, :], dtype=np.float64).reshape(nq * grp, d)
            state = empty_state((nq * grp,), d)
            for t0 in starts:
                t1 = min(t0 + chunk_len, n)
                keys = np.asarray(k_hist[b][g][t0:t1], dtype=np.float64)
                vals = np.asarray(v_hist[b][g][t0:t1], dtype=np.float64)
                part = local_state(rows, keys, vals, np.ones((nq * grp, t1 - t0), bool), scale)
                state = merge_states(state, part)
            if k_cand is not None and k_cand.shape[2]:
                part = local_state(rows, k_cand[b, g], v_cand[b, g], vis_c, scale)
                state = merge_states(state, part)
            o_s, lse_s = finalize(state)
            o[b, :, g * grp:(g + 1) * grp, :] = o_s.reshape(nq, grp, d)
            lse[b, :, g * grp:(g + 1) * grp] = lse_s.reshape(nq, grp)
    return o, lse
