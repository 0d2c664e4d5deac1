"""One verification round on the GPU, composed from the C-ABI calls.

ResidentRound: history resident in HBM -> ss_verify_candidates into slot 0,
the history into slots 1.. (ss_verify_chunk over fixed chunks, or
ss_verify_history's balanced cut), ss_merge_states -> O, lse (ragged chunked
rounds fold only the slots each request's history reaches). With the
candidate region fused, one ss_verify_history call writes all slots.
StreamedRound: history in pinned host memory -> ss_stream_history on a copy
and a compute stream, then candidates and merge on the compute stream.

Only device buffers and the order of calls live here; all arithmetic is in
the HIP library.
"""

from __future__ import annotations

import math

import torch

from . import ssverify as ss
from .workloads import VerifyInputs, to_chunk_major


def device_cus(device="cuda") -> int:
    return torch.cuda.get_device_properties(torch.device(device)).multi_processor_count


def auto_chunks_per_slot(cfg, hist_len, chunk_len, cus: int) -> int:
    """Chunks merged per state slot for a resident round. Wide row groups
    (compute-bound) take 4. Otherwise the slot count is chosen so that the
    chunk kernel launches about two work-groups per compute unit (one full
    wave of work-groups): fewer launches leave units idle, more leave
    partly filled rounds and cost a state slot each."""
    if cfg.rows > 32:
        return 4
    units = sum(-(-int(n) // chunk_len) for n in hist_len) * cfg.n_kv_heads
    return max(1, units // (2 * cus))


def auto_history_slots(cfg, hist_len, cus: int) -> int:
    """Slots per stream for ss_verify_history. Ragged lengths: enough that
    the longest stream does not force ranges longer than an even share of
    one wave of work-groups (two per compute unit), plus one for the range
    boundaries. Uniform lengths: one chunk per work-group of that wave. Wide
    row groups use the fixed cut of 4 chunks per slot."""
    pads = [-(-int(n) // 128) * 128 for n in hist_len]
    pad_max = max(pads, default=0)
    if cfg.rows > 32:
        return max(1, -(-pad_max // (4 * cfg.chunk_len)))
    if not cfg.ragged:
        return max(1, 2 * cus // (cfg.batch * cfg.n_kv_heads))
    total = sum(pads) * cfg.n_kv_heads
    if total == 0:
        return 2
    return max(2, -(-pad_max * 2 * cus // total) + 2)


def narrow_mfma(cfg, engine="auto") -> bool:
    """Whether the library runs this shape on its narrow MFMA kernels (the
    ones that can fold the candidate region into the history launch)."""
    return engine != "valu" and cfg.dtype == "bf16" and cfg.head_dim == 128 and cfg.rows <= 32


# Launch configuration of the resident round that the benchmark times.
BENCH_RESIDENT = dict(split="balanced", chunks_per_slot="auto", history_slots="auto", fuse_candidates="auto")


ENGINES = {"auto": ss.SS_ENGINE_AUTO, "valu": ss.SS_ENGINE_VALU, "mfma": ss.SS_ENGINE_MFMA}


def _problem(cfg, engine="auto") -> ss.Problem:
    return ss.make_problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_queries,
                           cfg.torch_dtype, cfg.scale, ENGINES[engine])


class ResidentRound:
    def __init__(self, inp: VerifyInputs, device="cuda", chunk_len=None, chunks_per_slot=1, engine="auto",
                 split="chunks", history_slots="auto", fuse_candidates=False):
        """split: "chunks" (ss_verify_chunk over chunks of chunk_len, merged
        chunks_per_slot at a time) or "balanced" (ss_verify_history with
        history_slots slots per stream).
        fuse_candidates (balanced split only): True, False or "auto" (when
        the narrow MFMA kernel serves the shape): pass the candidate region
        to ss_verify_history instead of a separate ss_verify_candidates.
        chunks_per_slot: an integer, or "auto" (auto_chunks_per_slot).
        history_slots: an integer >= 1, or "auto" (auto_history_slots).
        engine: "auto", "valu" or "mfma" (ss_problem_t.engine)."""
        cfg = inp.cfg
        self.cfg = cfg
        self.problem = _problem(cfg, engine)
        self.chunk_len = chunk_len or cfg.chunk_len
        if split not in ("chunks", "balanced"):
            raise ValueError(f"unknown split {split!r}")
        self.split = split
        if chunks_per_slot == "auto":
            chunks_per_slot = auto_chunks_per_slot(cfg, inp.hist_len, self.chunk_len, device_cus(device))
        self.cps = chunks_per_slot
        self.q = inp.q.to(device)
        self.k_hist = inp.k_hist.to(device)
        self.v_hist = inp.v_hist.to(device)
        self.max_len = int(inp.hist_len.max()) if len(inp.hist_len) else 0
        if cfg.ragged:
            self.hist_offset = torch.as_tensor(inp.hist_offset, dtype=torch.int64, device=device)
            self.hist_len = torch.as_tensor(inp.hist_len, dtype=torch.int32, device=device)
            if cfg.packing == "head":
                self.hist_view = ss.head_packed_view(self.k_hist, self.v_hist, self.hist_offset, self.hist_len,
                                                     self.max_len)
            else:
                self.hist_view = ss.token_major_view(self.k_hist, self.v_hist, self.hist_offset, self.hist_len,
                                                     self.max_len)
        else:
            self.hist_view = ss.head_major_view(self.k_hist, self.v_hist)
        self.k_cand = inp.k_cand.to(device)
        self.v_cand = inp.v_cand.to(device)
        self.cand_view = ss.head_major_view(self.k_cand, self.v_cand)
        self.parents = None
        if inp.parents is not None:
            self.parents = torch.as_tensor(inp.parents, dtype=torch.int32, device=device).contiguous()
        self.n_chunks = math.ceil(self.max_len / self.chunk_len)
        if fuse_candidates == "auto":
            fuse_candidates = narrow_mfma(cfg, engine)
        self.fused = bool(fuse_candidates) and split == "balanced"
        if split == "balanced":
            if history_slots == "auto":
                history_slots = auto_history_slots(cfg, inp.hist_len, device_cus(device))
            self.n_hist_slots = int(history_slots)
        else:
            self.n_hist_slots = math.ceil(self.n_chunks / self.cps)
        if self.fused:
            # one call writes every slot; outside the narrow kernel it gives
            # the first to the candidate region
            self.n_call_slots = self.n_hist_slots + (0 if narrow_mfma(cfg, engine) else 1)
            self.state = ss.StateBuffers(self.problem, self.n_call_slots, device)
        else:
            # slot 0: candidate region; slots 1 .. n_hist_slots: history
            self.state = ss.StateBuffers(self.problem, self.n_hist_slots + 1, device)
        self.slots_per_req = None
        if cfg.ragged and split == "chunks":
            per_slot = self.chunk_len * self.cps
            counts = [1 + math.ceil(int(n) / per_slot) for n in inp.hist_len]
            self.slots_per_req = torch.tensor(counts, dtype=torch.int32, device=device)
        self.mask_out = torch.zeros((cfg.batch, cfg.n_queries), dtype=torch.int64, device=device)
        self.o = torch.empty((cfg.batch, cfg.n_queries, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32,
                             device=device)
        self.lse = torch.empty((cfg.batch, cfg.n_queries, cfg.n_q_heads), dtype=torch.float32, device=device)

    def chunks(self, stream=None):
        if self.fused:                  # history and candidates, every slot written
            ss.ss_verify_history(self.problem, self.q, self.hist_view, self.cand_view, self.parents, self.mask_out,
                                 self.n_call_slots, self.state, 0, stream)
            return
        if self.split == "balanced":    # writes every history slot, even with no history
            ss.ss_verify_history(self.problem, self.q, self.hist_view, None, None, None, self.n_hist_slots,
                                 self.state, 1, stream)
            return
        if self.n_chunks == 0:          # no history at all: nothing to enqueue
            return
        ss.ss_verify_chunk(self.problem, self.q, self.hist_view, self.chunk_len, 0, self.n_chunks, self.cps,
                           self.state, 1, stream)

    def candidates(self, stream=None):
        if self.fused:                  # done inside the history launch
            return
        ss.ss_verify_candidates(self.problem, self.q, self.cand_view, self.parents, self.mask_out, self.state,
                                0, stream)

    def merge(self, stream=None):
        # ragged requests fold only the slots their history reaches
        ss.ss_merge_states(self.problem, self.state, self.slots_per_req, self.o, self.lse, stream)

    def run(self, stream=None):
        self.chunks(stream)
        self.candidates(stream)
        self.merge(stream)


class StreamedRound:
    def __init__(self, inp: VerifyInputs, device="cuda", n_buf=2, chunk_len=None):
        cfg = inp.cfg
        self.cfg = cfg
        self.problem = _problem(cfg)
        self.chunk_len = chunk_len or cfg.chunk_len
        n = int(inp.hist_len[0])
        if (inp.hist_len != n).any() or n % self.chunk_len:
            raise ValueError("streamed rounds need one history length, a multiple of the chunk length")
        self.n_chunks = n // self.chunk_len
        self.n_buf = n_buf
        b_, hkv, d = cfg.batch, cfg.n_kv_heads, cfg.head_dim
        self.chunk_elems = 2 * b_ * hkv * self.chunk_len * d
        self.host_kv = torch.empty((self.n_chunks, self.chunk_elems), dtype=cfg.torch_dtype, pin_memory=True)
        to_chunk_major(inp.k_hist, inp.v_hist, self.chunk_len, self.host_kv)
        self.staging = torch.empty((n_buf, self.chunk_elems), dtype=cfg.torch_dtype, device=device)
        self.q = inp.q.to(device)
        self.k_cand = inp.k_cand.to(device)
        self.v_cand = inp.v_cand.to(device)
        self.cand_view = ss.head_major_view(self.k_cand, self.v_cand)
        self.parents = None
        if inp.parents is not None:
            self.parents = torch.as_tensor(inp.parents, dtype=torch.int32, device=device).contiguous()
        self.state = ss.StateBuffers(self.problem, self.n_chunks + 1, device)
        self.o = torch.empty((b_, cfg.n_queries, cfg.n_q_heads, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((b_, cfg.n_queries, cfg.n_q_heads), dtype=torch.float32, device=device)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.compute_stream = torch.cuda.Stream(device=device)

    def run(self, record_timings=False):
        """Enqueues the whole round; the result is ready once compute_stream is."""
        cs = self.compute_stream
        cs.wait_stream(torch.cuda.current_stream())
        ss.ss_stream_history(self.problem, self.q, self.host_kv, self.chunk_len, self.n_chunks, self.staging,
                             self.n_buf, self.state, 0, self.copy_stream, cs, record_timings)
        ss.ss_verify_candidates(self.problem, self.q, self.cand_view, self.parents, None, self.state,
                                self.n_chunks, cs)
        ss.ss_merge_states(self.problem, self.state, None, self.o, self.lse, cs)
        torch.cuda.current_stream().wait_stream(cs)
