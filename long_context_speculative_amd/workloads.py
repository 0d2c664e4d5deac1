"""Seeded synthetic inputs for verification attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both the HIP path (through the tests and the benchmark)
and the fp64 oracle consume what it produces.

Recipe (every tensor is independent of the others and of the draw order):

* A config carries one integer seed. Each random stream is keyed by
  ``SeedSequence(seed, spawn_key=(stream, b))`` where ``stream`` names the
  tensor (see ``_STREAM``) and ``b`` is the request; lengths and trees draw
  from numpy PCG64 generators built from it.
* Ragged history lengths: integer uniform on [lo, hi], both ends included,
  one draw of B values from stream "len".
* Candidate trees: node 0 is the root (parent -1, depth 0); for i = 1..n-1 the
  parent is uniform over the earlier nodes whose depth is below the depth cap,
  so every node sits at depth <= cap and parent[i] < i (topological order).
* Values: float32 N(0, 1) from torch's CPU generator, one generator per
  (tensor, request) seeded with 63 bits of ``SeedSequence(seed,
  spawn_key=(stream, b)).generate_state``; drawn in the logical layout order
  of the tensor (a ragged history in [Hkv][N_b][d] order per request), then
  rounded to the config's dtype (bf16 by round-to-nearest-even through
  torch).

Logical layouts handed out:
  q        [B][nq][Hq][d]
  k_hist   uniform: [B][Hkv][N][d]; ragged: head-packed [Hkv][sum N_b][d]
           (or token-packed [sum N_b][Hkv][d]) with per-request element
           offsets ``hist_offset`` [B] (int64)
  k_cand   [B][Hkv][nc][d]
  parents  [B][nc] int32 (tree configs), -1 = root
  hist_len [B] int32
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_STREAM = {"len": 1, "tree": 2, "q": 3, "k_hist": 4, "v_hist": 5, "k_cand": 6, "v_cand": 7}


@dataclasses.dataclass(frozen=True)
class VerifyConfig:
    """One verification-round workload."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                  # "f32" or "bf16"
    hist_len: int               # uniform history length (ragged: upper bound)
    chunk_len: int
    n_queries: int              # k drafts + 1, or tree nodes
    mask: str                   # "causal" or "tree"
    seed: int
    ragged_lo: int = 0          # > 0 means ragged lengths in [ragged_lo, hist_len]
    tree_depth_cap: int = 8
    streamed: bool = False      # history sits in pinned host memory
    packing: str = "head"       # ragged layout: "head" [Hkv][sum N][d] or "token" [sum N][Hkv][d]
    score_scale: float = 0.0    # > 0: the score scale; else 1/sqrt(d)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def rows(self) -> int:
        """Rows per KV head: queries x heads of the group."""
        return self.n_queries * self.group

    @property
    def ragged(self) -> bool:
        return self.ragged_lo > 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        """score_scale if set, else 1/sqrt(d); rounded to float32 (the value
        the library receives)."""
        return float(np.float32(self.score_scale if self.score_scale > 0 else 1.0 / math.sqrt(self.head_dim)))

    def with_(self, **kw) -> "VerifyConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1_tiny_f32": VerifyConfig("c1_tiny_f32", 1, 4, 1, 64, "f32", 256, 64, 5, "causal", seed=1),
    "c2_qwen3_8b": VerifyConfig("c2_qwen3_8b", 16, 32, 8, 128, "bf16", 32768, 4096, 6, "causal", seed=2),
    "c3_internlm25_7b_ragged": VerifyConfig("c3_internlm25_7b_ragged", 32, 32, 8, 128, "bf16", 65536, 2048, 5,
                                            "causal", seed=3, ragged_lo=8192),
    "c4_tree_72b": VerifyConfig("c4_tree_72b", 4, 64, 8, 128, "bf16", 131072, 4096, 64, "tree", seed=4),
    "c5_streamed": VerifyConfig("c5_streamed", 8, 32, 8, 128, "bf16", 65536, 2048, 6, "causal", seed=5,
                                streamed=True),
}


def _rng(seed: int, stream: str, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(_STREAM[stream], b))))


def draw_lengths(cfg: VerifyConfig) -> np.ndarray:
    if not cfg.ragged:
        return np.full(cfg.batch, cfg.hist_len, dtype=np.int32)
    rng = _rng(cfg.seed, "len", 0)
    return rng.integers(cfg.ragged_lo, cfg.hist_len, size=cfg.batch, endpoint=True).astype(np.int32)


def draw_tree(seed: int, b: int, n: int, depth_cap: int) -> np.ndarray:
    rng = _rng(seed, "tree", b)
    parents = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        allowed = np.nonzero(depth[:i] < depth_cap)[0]
        p = int(allowed[rng.integers(0, len(allowed))])
        parents[i] = p
        depth[i] = depth[p] + 1
    return parents


def _torch_seed(seed: int, stream: str, b: int) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(_STREAM[stream], b))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _fill_normal(out: torch.Tensor, seed: int, stream: str, pieces) -> None:
    """Fill ``out`` (a CPU tensor) with N(0,1) values, piece by piece.

    pieces: list of (b, flat_start, count); piece b draws float32 normals from
    its own torch CPU generator, then they are rounded into ``out`` (bf16:
    round-to-nearest-even). Pieces run in parallel threads.
    """
    flat = out.view(-1)

    def work(piece):
        b, start, count = piece
        g = torch.Generator().manual_seed(_torch_seed(seed, stream, b))
        step = 1 << 24
        for off in range(0, count, step):
            n = min(step, count - off)
            vals = torch.randn(n, generator=g, dtype=torch.float32)
            flat[start + off:start + off + n].copy_(vals)

    threads = max(1, min(16, os.cpu_count() or 1))
    if len(pieces) == 1:
        work(pieces[0])
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, pieces))


def _fill_ragged(out: torch.Tensor, cfg: VerifyConfig, stream: str, lens, cum) -> None:
    """Ragged history: request b draws its [Hkv][N_b][d] block in that order
    from its own generator (the values do not depend on the packing), then
    the block is placed head-packed or token-packed."""
    hkv, d = cfg.n_kv_heads, cfg.head_dim

    def work(b):
        n = int(lens[b])
        g = torch.Generator().manual_seed(_torch_seed(cfg.seed, stream, b))
        block = torch.randn(hkv * n * d, generator=g, dtype=torch.float32).view(hkv, n, d)
        c0 = int(cum[b])
        if cfg.packing == "head":
            out[:, c0:c0 + n, :].copy_(block)
        else:
            out[c0:c0 + n].copy_(block.transpose(0, 1))

    threads = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(cfg.batch)))


@dataclasses.dataclass
class VerifyInputs:
    cfg: VerifyConfig
    q: torch.Tensor
    k_hist: torch.Tensor
    v_hist: torch.Tensor
    hist_len: np.ndarray          # [B] int32
    hist_offset: np.ndarray       # [B] int64 element offsets (ragged layout) or None
    k_cand: torch.Tensor
    v_cand: torch.Tensor
    parents: np.ndarray | None    # [B][nc] int32, tree configs only

    # ---- views for the oracle (numpy float32, exact copies of the values) ----
    def hist_per_request(self, which: str) -> "_HistView":
        """Indexable as view[b][g] -> numpy float32 [N_b][d] (converted lazily,
        one (request, KV head) slice at a time)."""
        return _HistView(self, which)


def input_digest(inp: VerifyInputs) -> str:
    """SHA-256 (hex) over the bytes of every input, in this order: q, the K
    and V history, the K and V candidates (each in its stored layout), the
    history lengths (int32) and, for trees, the parents (int32)."""
    h = hashlib.sha256()
    for t in (inp.q, inp.k_hist, inp.v_hist, inp.k_cand, inp.v_cand):
        h.update(t.contiguous().reshape(-1).view(torch.uint8).numpy().data)
    h.update(np.ascontiguousarray(inp.hist_len, dtype=np.int32).tobytes())
    if inp.parents is not None:
        h.update(np.ascontiguousarray(inp.parents, dtype=np.int32).tobytes())
    return h.hexdigest()


class _HistView:
    def __init__(self, inp: "VerifyInputs", which: str):
        self._inp = inp
        self._src = inp.k_hist if which == "k" else inp.v_hist

    def __len__(self):
        return self._inp.cfg.batch

    def __getitem__(self, b: int) -> "_HistHeads":
        return _HistHeads(self, int(b))


class _HistHeads:
    def __init__(self, view: _HistView, b: int):
        self._view, self._b = view, b

    def __len__(self):
        return self._view._inp.cfg.n_kv_heads

    def __getitem__(self, g: int) -> np.ndarray:
        inp, src, b = self._view._inp, self._view._src, self._b
        cfg = inp.cfg
        n = int(inp.hist_len[b])
        if cfg.ragged and cfg.packing == "head":
            t0 = int(inp.hist_offset[b]) // cfg.head_dim
            sl = src[int(g), t0:t0 + n, :]
        elif cfg.ragged:
            t0 = int(inp.hist_offset[b]) // (cfg.n_kv_heads * cfg.head_dim)
            sl = src[t0:t0 + n, int(g), :]
        else:
            sl = src[b, int(g), :n, :]
        return sl.float().numpy()


def make_inputs(cfg: VerifyConfig, with_history: bool = True) -> VerifyInputs:
    """Draw every input of one round on the CPU."""
    b_, hq, hkv, d, nq = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_queries
    dt = cfg.torch_dtype
    lens = draw_lengths(cfg)
    parents = None
    if cfg.mask == "tree":
        parents = np.stack([draw_tree(cfg.seed, b, nq, cfg.tree_depth_cap) for b in range(b_)])

    q = torch.empty((b_, nq, hq, d), dtype=dt)
    _fill_normal(q, cfg.seed, "q", [(b, b * nq * hq * d, nq * hq * d) for b in range(b_)])

    offsets = None
    if not with_history:
        k_hist = torch.empty(0, dtype=dt)
        v_hist = torch.empty(0, dtype=dt)
    elif cfg.ragged:
        total = int(lens.astype(np.int64).sum())
        cum = np.zeros(b_, dtype=np.int64)
        cum[1:] = np.cumsum(lens[:-1].astype(np.int64))
        if cfg.packing == "head":
            k_hist = torch.empty((hkv, total, d), dtype=dt)
            v_hist = torch.empty((hkv, total, d), dtype=dt)
            offsets = cum * d
        else:
            k_hist = torch.empty((total, hkv, d), dtype=dt)
            v_hist = torch.empty((total, hkv, d), dtype=dt)
            offsets = cum * hkv * d
        _fill_ragged(k_hist, cfg, "k_hist", lens, cum)
        _fill_ragged(v_hist, cfg, "v_hist", lens, cum)
    else:
        n = cfg.hist_len
        per = hkv * n * d
        k_hist = torch.empty((b_, hkv, n, d), dtype=dt)
        v_hist = torch.empty((b_, hkv, n, d), dtype=dt)
        pieces = [(b, b * per, per) for b in range(b_)]
        _fill_normal(k_hist, cfg.seed, "k_hist", pieces)
        _fill_normal(v_hist, cfg.seed, "v_hist", pieces)

    per_c = hkv * nq * d
    k_cand = torch.empty((b_, hkv, nq, d), dtype=dt)
    v_cand = torch.empty((b_, hkv, nq, d), dtype=dt)
    _fill_normal(k_cand, cfg.seed, "k_cand", [(b, b * per_c, per_c) for b in range(b_)])
    _fill_normal(v_cand, cfg.seed, "v_cand", [(b, b * per_c, per_c) for b in range(b_)])
    return VerifyInputs(cfg, q, k_hist, v_hist, lens, offsets, k_cand, v_cand, parents)


def to_chunk_major(k_hist: torch.Tensor, v_hist: torch.Tensor, chunk_len: int, out: torch.Tensor) -> None:
    """Re-lay a uniform history [B][Hkv][N][d] (K and V) into the chunk-major
    host layout [J][2][B][Hkv][C][d] used for streaming (one contiguous block
    per chunk). ``out`` is preallocated (pinned host memory)."""
    b_, hkv, n, d = k_hist.shape
    n_chunks = n // chunk_len
    kc = k_hist.view(b_, hkv, n_chunks, chunk_len, d).permute(2, 0, 1, 3, 4)
    vc = v_hist.view(b_, hkv, n_chunks, chunk_len, d).permute(2, 0, 1, 3, 4)
    out_v = out.view(n_chunks, 2, b_, hkv, chunk_len, d)
    out_v[:, 0].copy_(kc)
    out_v[:, 1].copy_(vc)
