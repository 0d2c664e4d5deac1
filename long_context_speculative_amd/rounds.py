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


def wgs_per_cu(cfg, engine="auto") -> int:
    """Work-groups per compute unit in one launch: one for the narrow bf16
    and the fp32 MFMA kernels (two co-resident 4-wave work-groups progress
    unevenly, and the one left alone at the end streams slower), two for
    the other chunk kernels."""
    return 1 if narrow_mfma(cfg, engine) or f32_mfma(cfg, engine) else 2


def auto_chunks_per_slot(cfg, hist_len, chunk_len, cus: int, engine="auto") -> int:
    """Chunks merged per state slot for a resident round. Wide row groups
    (compute-bound) take 4. Otherwise the slot count is chosen so that the
    chunk kernel launches about wgs_per_cu work-groups per compute unit:
    fewer leave units idle, more leave partly filled rounds and cost a state
    slot each."""
    if cfg.rows > 32:
        return 4
    units = sum(-(-int(n) // chunk_len) for n in hist_len) * cfg.n_kv_heads
    return max(1, units // (wgs_per_cu(cfg, engine) * cus))


# Line positions the balanced cut charges per stream for starting a piece
# (kPlanCharge of the library's plan, at its 128-token alignment).
PLAN_CHARGE = 512


def one_piece_per_stream(max_len: int, streams: int, cus: int) -> bool:
    """Whether ragged histories on the narrow MFMA kernel run faster as one
    piece per stream (one slot: a work-group per (request, KV head), all in
    parallel) than under the balanced cut, whose work-groups run two or
    three short pieces one after another, each paying its start and merge.
    Measured on MI355X (256 CUs), lengths uniform in [n/8, n], history and
    merge launches: one piece per stream is 1.07-1.33x faster at n <= 2048
    with 192 to 1024 streams, even at 3072-4096 and slower beyond; with
    fewer streams it leaves CUs idle. (The library's own slot choice for
    ss_verify_round, whose one-slot rounds also skip the merge launch, takes
    one slot up to 4096 tokens when every CU has a stream.)"""
    return max_len <= 2048 and 4 * streams >= 3 * cus


def auto_history_slots(cfg, hist_len, cus: int, engine="auto") -> int:
    """Slots per stream for ss_verify_history. Ragged lengths on the narrow
    MFMA kernel: one when one_piece_per_stream holds, else (and on the other
    kernels) as many as the longest stream has pieces when every work-group
    of the launch (wgs_per_cu per compute unit) takes an even share of the
    line. Uniform lengths: one chunk per work-group of that
    launch. Wide row groups on the MFMA kernel: one wave of work-groups
    (8-wave groups of 256 rows, one per compute unit, or 4-wave groups of 128
    rows, two per unit), the slot count ss_verify_round picks; other wide
    shapes use the fixed cut of 4 chunks per slot."""
    pads = [-(-int(n) // 128) * 128 for n in hist_len]
    pad_max = max(pads, default=0)
    if cfg.rows > 32 and mfma_fuses_candidates(cfg, engine):
        per_group, per_cu = (256, 1) if cfg.rows > 128 else (128, 2)
        groups = -(-cfg.rows // per_group)
        return min(64, max(1, per_cu * cus // (cfg.batch * cfg.n_kv_heads * groups)))
    if cfg.rows > 32:
        return max(1, -(-pad_max // (4 * cfg.chunk_len)))
    wave = wgs_per_cu(cfg, engine) * cus
    if not cfg.ragged:
        return max(1, wave // (cfg.batch * cfg.n_kv_heads))
    if not any(pads):
        return 2
    # the line also holds a gap of PLAN_CHARGE positions after every stream
    total = (sum(pads) + PLAN_CHARGE * len(pads)) * cfg.n_kv_heads
    if narrow_mfma(cfg, engine) and one_piece_per_stream(max((int(n) for n in hist_len), default=0),
                                                          cfg.batch * cfg.n_kv_heads, cus):
        return 1
    # Tokens per work-group of the balanced cut (an even share, rounded up to
    # 128): a stream of pad tokens then spans at most ceil(pad / L) work-group
    # ranges, plus one when it straddles a boundary. With that many slots the
    # cut's cap pad_max / (slots - 1) stays below L, so L is the even share.
    piece = max(128, -(-(-(-total // wave)) // 128) * 128)
    return max(2, -(-pad_max // piece) + 1)


def narrow_mfma(cfg, engine="auto") -> bool:
    """Whether the library runs this shape on its narrow MFMA kernels
    (bf16, head_dim 128 or 64, up to 32 rows per KV head)."""
    return engine != "valu" and cfg.dtype == "bf16" and cfg.head_dim in (64, 128) and cfg.rows <= 32


def f32_mfma(cfg, engine="auto") -> bool:
    """Whether the library runs this shape on its fp32 MFMA kernel (every
    fp32 shape outside the forced VALU engine; one work-group per piece up to
    32 rows per KV head, one per row group of 32 beyond)."""
    return engine != "valu" and cfg.dtype == "f32"


def mfma_fuses_candidates(cfg, engine="auto") -> bool:
    """Whether ss_verify_history folds the candidate region into the history
    launch (the MFMA kernels, narrow and wide-row) instead of giving it a
    slot of its own."""
    return narrow_mfma(cfg, engine) or (engine != "valu" and cfg.dtype == "bf16" and cfg.head_dim in (64, 128))


# Launch configuration of the resident round that the benchmark times.
BENCH_RESIDENT = dict(split="balanced", chunks_per_slot="auto", history_slots="auto", fuse_candidates="auto",
                      kv_layout="interleaved")


ENGINES = {"auto": ss.SS_ENGINE_AUTO, "valu": ss.SS_ENGINE_VALU, "mfma": ss.SS_ENGINE_MFMA}


def _problem(cfg, engine="auto") -> ss.Problem:
    return ss.make_problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_queries,
                           cfg.torch_dtype, cfg.scale, ENGINES[engine])


def interleave_kv(k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    """One device tensor holding the K row and the V row of every (token, KV
    head) next to each other: the shape of k with an axis of 2 inserted
    before the feature axis (index 0 = K, 1 = V), so one history stream is
    one run of memory instead of two."""
    return torch.stack((k, v), dim=-2).contiguous()


class ResidentRound:
    def __init__(self, inp: VerifyInputs, device="cuda", chunk_len=None, chunks_per_slot=1, engine="auto",
                 split="chunks", history_slots="auto", fuse_candidates=False, kv_layout="separate"):
        """split: "chunks" (ss_verify_chunk over chunks of chunk_len, merged
        chunks_per_slot at a time) or "balanced" (ss_verify_history with
        history_slots slots per stream).
        kv_layout: "separate" (K and V in two tensors of the input layout)
        or "interleaved" (one tensor, each token's K and V rows adjacent;
        the view's strides and offsets step over both).
        fuse_candidates (balanced split only): True, False or "auto" (when
        an MFMA kernel serves the shape): pass the candidate region to
        ss_verify_history instead of a separate ss_verify_candidates.
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
            chunks_per_slot = auto_chunks_per_slot(cfg, inp.hist_len, self.chunk_len, device_cus(device), engine)
        self.cps = chunks_per_slot
        if kv_layout not in ("separate", "interleaved"):
            raise ValueError(f"unknown kv_layout {kv_layout!r}")
        self.kv_layout = kv_layout
        self.q = inp.q.to(device)
        self.max_len = int(inp.hist_len.max()) if len(inp.hist_len) else 0
        if cfg.ragged:
            self.hist_offset = torch.as_tensor(inp.hist_offset, dtype=torch.int64, device=device)
            self.hist_len = torch.as_tensor(inp.hist_len, dtype=torch.int32, device=device)
        if kv_layout == "separate":
            self.k_hist = inp.k_hist.to(device)
            self.v_hist = inp.v_hist.to(device)
            if not cfg.ragged:
                self.hist_view = ss.head_major_view(self.k_hist, self.v_hist)
            elif cfg.packing == "head":
                self.hist_view = ss.head_packed_view(self.k_hist, self.v_hist, self.hist_offset, self.hist_len,
                                                     self.max_len)
            else:
                self.hist_view = ss.token_major_view(self.k_hist, self.v_hist, self.hist_offset, self.hist_len,
                                                     self.max_len)
        else:
            # [B][Hkv][N][2][d], head-packed [Hkv][sum N][2][d] or
            # token-packed [sum N][Hkv][2][d]
            self.kv_hist = interleave_kv(inp.k_hist.to(device), inp.v_hist.to(device))
            kv = self.kv_hist
            v_at = kv.narrow(-2, 1, 1)  # the V rows: head_dim elements after each K row
            if not cfg.ragged:
                sb, sh, st = kv.stride(0), kv.stride(1), kv.stride(2)
                self.hist_view = ss.make_view(kv, v_at, sb, sh, st, kv.shape[2])
            else:
                self.hist_offset2 = self.hist_offset * 2  # element offsets count K and V rows
                if cfg.packing == "head":
                    sh, st = kv.stride(0), kv.stride(1)
                else:
                    st, sh = kv.stride(0), kv.stride(1)
                self.hist_view = ss.make_view(kv, v_at, 0, sh, st, self.max_len, self.hist_offset2, self.hist_len)
        self.k_cand = inp.k_cand.to(device)
        self.v_cand = inp.v_cand.to(device)
        self.cand_view = ss.head_major_view(self.k_cand, self.v_cand)
        self.parents = None
        if inp.parents is not None:
            self.parents = torch.as_tensor(inp.parents, dtype=torch.int32, device=device).contiguous()
        self.n_chunks = math.ceil(self.max_len / self.chunk_len)
        if fuse_candidates == "auto":
            fuse_candidates = mfma_fuses_candidates(cfg, engine)
        self.fused = bool(fuse_candidates) and split == "balanced"
        if split == "balanced":
            if history_slots == "auto":
                history_slots = auto_history_slots(cfg, inp.hist_len, device_cus(device), engine)
            self.n_hist_slots = int(history_slots)
        else:
            self.n_hist_slots = math.ceil(self.n_chunks / self.cps)
        if self.fused:
            # one call writes every slot; the VALU engines give the first to
            # the candidate region
            self.n_call_slots = self.n_hist_slots + (0 if mfma_fuses_candidates(cfg, engine) else 1)
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
        self.stats = None               # a BlockStatsBuffer: balanced split records block statistics
        self.o = torch.empty((cfg.batch, cfg.n_queries, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32,
                             device=device)
        self.lse = torch.empty((cfg.batch, cfg.n_queries, cfg.n_q_heads), dtype=torch.float32, device=device)

    def chunks(self, stream=None):
        if self.fused:                  # history and candidates, every slot written
            ss.ss_verify_history(self.problem, self.q, self.hist_view, self.cand_view, self.parents, self.mask_out,
                                 self.n_call_slots, self.state, 0, stream, stats=self.stats)
            return
        if self.split == "balanced":    # writes every history slot, even with no history
            ss.ss_verify_history(self.problem, self.q, self.hist_view, None, None, None, self.n_hist_slots,
                                 self.state, 1, stream, stats=self.stats)
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
    def __init__(self, inp: VerifyInputs, device="cuda", n_buf=2, chunk_len=None, chunks_per_copy=1):
        cfg = inp.cfg
        self.cfg = cfg
        self.problem = _problem(cfg)
        self.chunk_len = chunk_len or cfg.chunk_len
        n = int(inp.hist_len[0])
        if (inp.hist_len != n).any() or n % self.chunk_len:
            raise ValueError("streamed rounds need one history length, a multiple of the chunk length")
        self.n_chunks = n // self.chunk_len
        self.n_buf = n_buf
        self.chunks_per_copy = chunks_per_copy
        b_, hkv, d = cfg.batch, cfg.n_kv_heads, cfg.head_dim
        self.chunk_elems = 2 * b_ * hkv * self.chunk_len * d
        self.host_kv = torch.empty((self.n_chunks, self.chunk_elems), dtype=cfg.torch_dtype, pin_memory=True)
        to_chunk_major(inp.k_hist, inp.v_hist, self.chunk_len, self.host_kv)
        self.staging = torch.empty((n_buf, chunks_per_copy * self.chunk_elems), dtype=cfg.torch_dtype,
                                   device=device)
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

    def run(self, record_timings=False, checks=0):
        """Enqueues the whole round; the result is ready once compute_stream is.
        checks: ordering diagnostics of ss_stream_history (SS_STREAM_POISON,
        SS_STREAM_DELAY)."""
        cs = self.compute_stream
        cs.wait_stream(torch.cuda.current_stream())
        ss.ss_stream_history(self.problem, self.q, self.host_kv, self.chunk_len, self.n_chunks, self.staging,
                             self.n_buf, self.state, 0, self.copy_stream, cs, record_timings,
                             chunks_per_copy=self.chunks_per_copy, checks=checks)
        ss.ss_verify_candidates(self.problem, self.q, self.cand_view, self.parents, None, self.state,
                                self.n_chunks, cs)
        ss.ss_merge_states(self.problem, self.state, None, self.o, self.lse, cs)
        torch.cuda.current_stream().wait_stream(cs)


def exposed_wait(timings) -> float:
    """The compute stream's wait for data in one streaming call, in ms: the
    first chunk's arrival after the call, then every chunk that lands after
    the previous chunk's attention finished (SpecStream section 3.2's
    compute bubble)."""
    c0, c1, k0, k1 = timings
    return max(0.0, c1[0]) + sum(max(0.0, c1[j] - k1[j - 1]) for j in range(1, len(c1)))


class LayeredStreamedRound:
    """A verification round through L layers, each with its own host-resident
    history (SpecStream section 4.2: the target reads each layer's history
    layer by layer). Between layers the compute stream runs the rest of the
    layer (output projection and feed-forward), stood in for here by a
    square bf16 matrix product chain of a chosen size. With prefetch the
    staging ring continues across layers (SS_STREAM_CONTINUE), so the next
    layer's first chunks are copied while the current layer finishes."""

    def __init__(self, inputs, device="cuda", n_buf=2, chunks_per_copy=1, rest_dim=4096, rest_reps=4):
        self.layers = [StreamedRound.__new__(StreamedRound) for _ in inputs]
        first = StreamedRound(inputs[0], device, n_buf, None, chunks_per_copy)
        self.layers[0] = first
        for i, inp in enumerate(inputs[1:], 1):
            lay = StreamedRound.__new__(StreamedRound)
            lay.__dict__.update(first.__dict__)     # same geometry, staging ring and streams
            lay.host_kv = torch.empty_like(first.host_kv, pin_memory=True)
            to_chunk_major(inp.k_hist, inp.v_hist, lay.chunk_len, lay.host_kv)
            lay.q = inp.q.to(device)
            lay.k_cand = inp.k_cand.to(device)
            lay.v_cand = inp.v_cand.to(device)
            lay.cand_view = ss.head_major_view(lay.k_cand, lay.v_cand)
            lay.parents = None if inp.parents is None else torch.as_tensor(inp.parents, dtype=torch.int32,
                                                                           device=device).contiguous()
            lay.state = ss.StateBuffers(first.problem, first.n_chunks + 1, device)
            lay.o = torch.empty_like(first.o)
            lay.lse = torch.empty_like(first.lse)
            self.layers[i] = lay
        self.rest_a = torch.randn((rest_dim, rest_dim), device=device).to(torch.bfloat16)
        self.rest_b = torch.randn((rest_dim, rest_dim), device=device).to(torch.bfloat16)
        self.rest_reps = rest_reps

    def run(self, prefetch=True, record_timings=False):
        first = self.layers[0]
        cs = first.compute_stream
        cs.wait_stream(torch.cuda.current_stream())
        for i, lay in enumerate(self.layers):
            ss.ss_stream_history(lay.problem, lay.q, lay.host_kv, lay.chunk_len, lay.n_chunks, lay.staging,
                                 lay.n_buf, lay.state, 0, lay.copy_stream, cs, record_timings,
                                 chunks_per_copy=lay.chunks_per_copy, continue_ring=prefetch and i > 0)
            ss.ss_verify_candidates(lay.problem, lay.q, lay.cand_view, lay.parents, None, lay.state, lay.n_chunks, cs)
            ss.ss_merge_states(lay.problem, lay.state, None, lay.o, lay.lse, cs)
            with torch.cuda.stream(cs):       # the rest of the layer
                x = self.rest_a
                for _ in range(self.rest_reps):
                    x = torch.mm(x, self.rest_b)
        torch.cuda.current_stream().wait_stream(cs)

    def layer_waits(self):
        """Exposed wait of every layer of the last timed run, in ms."""
        n = len(self.layers)
        return [exposed_wait(ss.ss_stream_timings(self.layers[i].n_chunks, back=n - 1 - i)) for i in range(n)]


class TieredRound:
    """Commit-aware KV tiering around the verification round (SpecStream
    section 4.1, Eq. 4-5), one request per batch row:

      Sealed History [0, H_b)   pinned host store, chunk-major
                                [J][2][B][Hkv][C][d]; streamed every round
                                (ss_stream_history with per-request lengths)
      Active Tail [H_b, C_b)    device tail buffer, row 0 = token H_b
      Speculative Frontier      the round's candidate rows (device)

    verify() runs one round: streamed sealed history into slots [0, J),
    the tail with the candidate region folded in (ss_verify_history) into
    the following slots, then the merge. commit() moves the accepted
    candidates into the tail (the rest is simply not kept: rollback stays on
    the GPU). migrate() applies Eq. (5) through the library, copies [H_b,
    E_b) to the host store on the copy stream and, ordered after those
    copies, compacts the tail into the second tail buffer; H_b becomes E_b.
    """

    def __init__(self, cfg, hist_k, hist_v, tail_target=512, gran=256, chunk_len=512, max_tokens=None,
                 q_max=None, device="cuda", n_buf=2, tail_slots=2, overlap_migration=False):
        """hist_k, hist_v: per-request CPU tensors [Hkv][N_b][d] of the
        initial committed history (cfg.torch_dtype).
        overlap_migration: migrate() only starts the device-to-host copies,
        on a stream of their own, and returns; the next verify() runs while
        they are in flight (reading the tail rows they copy), and H moves to
        E, with the tail compacted, once they have landed (finalize(), called
        by verify() after it has enqueued its work)."""
        self.cfg = cfg
        self.problem = _problem(cfg)
        self.device = device
        b_, hkv, d = cfg.batch, cfg.n_kv_heads, cfg.head_dim
        dt = cfg.torch_dtype
        self.tail_target, self.gran, self.chunk_len = tail_target, gran, chunk_len
        self.n_buf, self.tail_slots = n_buf, tail_slots
        q_max = q_max or cfg.n_queries
        lens = [int(k.shape[1]) for k in hist_k]
        max_tokens = max_tokens or (max(lens) + 64 * q_max)
        self.n_chunks_cap = -(-max_tokens // chunk_len)
        # tail capacity: T + g of committed rows after migration stays below
        # T + g; one round adds at most q_max
        self.cap = -(-(tail_target + 2 * gran + q_max) // 128) * 128
        chunk_elems = 2 * b_ * hkv * chunk_len * d
        self.host_kv = torch.zeros((self.n_chunks_cap, chunk_elems), dtype=dt, pin_memory=True)
        self.staging = torch.empty((n_buf, chunk_elems), dtype=dt, device=device)
        self.tails = [(torch.zeros((b_, hkv, self.cap, d), dtype=dt, device=device),
                       torch.zeros((b_, hkv, self.cap, d), dtype=dt, device=device)) for _ in range(2)]
        self.cur = 0
        self.copy_stream = torch.cuda.Stream(device=device)
        self.compute_stream = torch.cuda.Stream(device=device)
        self.overlap = overlap_migration
        self.migrate_stream = torch.cuda.Stream(device=device) if overlap_migration else None
        self.pending = None              # (E, copies-landed event) of a migration in flight
        self.last_migration = None       # (start, end) timing events of the last migration copy
        self.state = ss.StateBuffers(self.problem, self.n_chunks_cap + tail_slots, device)
        self.o = torch.empty((b_, cfg.n_queries, cfg.n_q_heads, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((b_, cfg.n_queries, cfg.n_q_heads), dtype=torch.float32, device=device)
        self.mask_out = torch.zeros((b_, cfg.n_queries), dtype=torch.int64, device=device)

        # Initial placement: the whole committed history goes to the device
        # once, Eq. (5) decides what is sealed, the sealed part is migrated to
        # the host store and the rest becomes the tail.
        n0 = max(max(lens), 1)
        full_k = torch.zeros((b_, hkv, n0, d), dtype=dt)
        full_v = torch.zeros((b_, hkv, n0, d), dtype=dt)
        for b in range(b_):
            full_k[b, :, :lens[b]] = hist_k[b]
            full_v[b, :, :lens[b]] = hist_v[b]
        full_k, full_v = full_k.to(device), full_v.to(device)
        full = self._view(full_k, full_v, n0)
        self.H = [0] * b_
        self.C = list(lens)
        ends = [ss.ss_tier_migration_end(0, c, tail_target, gran) for c in self.C]
        stream = torch.cuda.current_stream()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        ss.ss_tier_migrate(self.problem, full, [0] * b_, [0] * b_, ends, self.host_kv, chunk_len,
                           self.n_chunks_cap, stream)
        ev1.record(stream)
        ss.ss_kv_copy_rows(self.problem, full, ends, self.tail_view(), [0] * b_,
                           [c - e for c, e in zip(self.C, ends)], stream)
        torch.cuda.synchronize()
        # the bulk migration of the initial history (device to host)
        self.init_migrate_ms = ev0.elapsed_time(ev1)
        self.init_migrated_bytes = 2 * sum(ends) * hkv * d * cfg.elem_bytes
        self.H = ends
        self._check_capacity()

    # ---- views --------------------------------------------------------------
    def _view(self, k, v, rows, req_len=None):
        b_, hkv, cap, d = k.shape
        return ss.make_view(k, v, hkv * cap * d, cap * d, d, rows, None, req_len)

    def tail_view(self, req_len=None):
        k, v = self.tails[self.cur]
        return self._view(k, v, self.cap, req_len)

    def _check_capacity(self):
        for h, c in zip(self.H, self.C):
            if not (0 <= h <= c and c - h <= self.cap):
                raise RuntimeError(f"tail of {c - h} rows exceeds the buffer ({self.cap})")

    # ---- one round ----------------------------------------------------------
    def verify(self, q, k_cand, v_cand, parents=None):
        """q [B][nq][Hq][d], k_cand/v_cand [B][Hkv][nq][d] (device). Result in
        self.o / self.lse once the current stream has caught up."""
        cfg = self.cfg
        cs = self.compute_stream
        cs.wait_stream(torch.cuda.current_stream())
        self.q = q
        self.cand_view = ss.head_major_view(k_cand, v_cand)
        self.k_cand, self.v_cand = k_cand, v_cand
        self.sealed_len = torch.tensor(self.H, dtype=torch.int32, device=self.device)
        self.tail_len = torch.tensor([c - h for c, h in zip(self.C, self.H)], dtype=torch.int32,
                                     device=self.device)
        n_chunks = -(-max(self.H) // self.chunk_len)
        n_slots = n_chunks + self.tail_slots
        st = ss.StateBuffers.__new__(ss.StateBuffers)
        st.acc, st.m, st.l, st.n_slots = self.state.acc, self.state.m, self.state.l, n_slots
        st.struct = ss.State(self.state.acc.data_ptr(), self.state.m.data_ptr(), self.state.l.data_ptr(), n_slots)
        if n_chunks:
            ss.ss_stream_history(self.problem, q, self.host_kv, self.chunk_len, n_chunks, self.staging, self.n_buf,
                                 st, 0, self.copy_stream, cs, req_len=self.sealed_len)
        ss.ss_verify_history(self.problem, q, self.tail_view(self.tail_len), self.cand_view, parents,
                             self.mask_out, self.tail_slots, st, n_chunks, cs)
        ss.ss_merge_states(self.problem, st, None, self.o, self.lse, cs)
        torch.cuda.current_stream().wait_stream(cs)
        self.finalize()
        return self.o, self.lse

    def commit(self, accepted):
        """accepted[b]: how many of request b's candidates (a prefix) the
        target accepted. Their KV joins the tail; the rest is dropped."""
        src_rows = [0] * self.cfg.batch
        dst_rows = [c - h for c, h in zip(self.C, self.H)]
        cand = ss.head_major_view(self.k_cand, self.v_cand)
        ss.ss_kv_copy_rows(self.problem, cand, src_rows, self.tail_view(), dst_rows, list(accepted),
                           torch.cuda.current_stream())
        self.C = [c + int(a) for c, a in zip(self.C, accepted)]
        self._check_capacity()

    def migrate(self, overlap=None):
        """Eq. (5) for every request; [H_b, E_b) goes to the host store, then
        the tail is compacted so that row 0 is token E_b. Returns E. With
        overlap (default: overlap_migration) the copies are only started
        (see __init__)."""
        overlap = self.overlap if overlap is None else overlap
        self.finalize()
        ends = [ss.ss_tier_migration_end(h, c, self.tail_target, self.gran) for h, c in zip(self.H, self.C)]
        if all(e == h for e, h in zip(ends, self.H)):
            return ends
        cur = torch.cuda.current_stream()
        if overlap and self.migrate_stream is None:
            self.migrate_stream = torch.cuda.Stream(device=self.device)
        stream = self.migrate_stream if overlap else self.copy_stream
        stream.wait_stream(cur)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        ss.ss_tier_migrate(self.problem, self.tail_view(), self.H, self.H, ends, self.host_kv, self.chunk_len,
                           self.n_chunks_cap, stream)
        t1.record(stream)
        self.last_migration = (t0, t1)
        self.pending = (ends, t1)
        if not overlap:
            self.finalize()
        return ends

    def finalize(self):
        """Completes a migration whose copies were started: once they have
        landed (stream order, no host wait), the tail is compacted so that
        row 0 is token E_b, and H becomes E (section 4.1: H moves only after
        the copy)."""
        if self.pending is None:
            return
        ends, landed = self.pending
        cur = torch.cuda.current_stream()
        # the sealed range is reclaimed on the GPU only after its copy landed
        cur.wait_event(landed)
        nxt = 1 - self.cur
        k, v = self.tails[nxt]
        ss.ss_kv_copy_rows(self.problem, self.tail_view(), [e - h for e, h in zip(ends, self.H)],
                           self._view(k, v, self.cap), [0] * self.cfg.batch,
                           [c - e for c, e in zip(self.C, ends)], cur)
        self.cur = nxt
        self.H = ends
        self.pending = None

    # ---- inspection (tests) -------------------------------------------------
    def sealed_rows(self, b, which):
        """Host-store rows [0, H_b) of request b: CPU tensor [Hkv][H_b][d]."""
        cfg = self.cfg
        j = -(-self.H[b] // self.chunk_len)
        kv = 0 if which == "k" else 1
        blocks = self.host_kv[:j].view(j, 2, cfg.batch, cfg.n_kv_heads, self.chunk_len, cfg.head_dim)
        rows = blocks[:, kv, b].permute(1, 0, 2, 3).reshape(cfg.n_kv_heads, j * self.chunk_len, cfg.head_dim)
        return rows[:, :self.H[b]]

    def tail_rows(self, b, which):
        """Device tail rows [H_b, C_b) of request b, on the CPU."""
        k, v = self.tails[self.cur]
        t = k if which == "k" else v
        return t[b, :, :self.C[b] - self.H[b]].cpu()


class SparseRound:
    """Block statistics and block-sparse verification on a resident history
    (the SparseSpec-L and Dustin abstracts on the pages, over SpecStream's
    block-wise states):

      full()    the full round -> O, lse. With stats=False: one state slot
                per block of block_len tokens (ss_verify_chunk,
                chunks_per_slot 1), the candidate region in slot 0, merge.
                With stats=True: the resident round as benchmarked (balanced
                cut, candidates fused) recording block statistics as it goes
                (narrow MFMA kernel, block_len a multiple of 128);
      select()  per-(request, KV head) importance of every block
                (ss_block_importance from the block slots, or
                ss_block_importance_stats from the statistics) and the k most
                important blocks (ss_select_blocks);
      sparse()  verification of the selected blocks only
                (ss_verify_chunk_gathered, gather_per_slot selected blocks
                merged per slot) with the candidate region, merge.

    gather_per_slot: an integer, or "auto": on the narrow MFMA kernel as
    many as give about one work-group per compute unit, else 1.
    """

    def __init__(self, inp: VerifyInputs, block_len: int, k: int, device="cuda", engine="auto", stats=False,
                 gather_per_slot="auto"):
        cfg = inp.cfg
        self.use_stats = bool(stats)
        if self.use_stats:
            if not narrow_mfma(cfg, engine):
                raise ValueError("block statistics need the narrow MFMA kernel")
            self.full_round = ResidentRound(inp, device, chunk_len=block_len, engine=engine, **BENCH_RESIDENT)
        else:
            self.full_round = ResidentRound(inp, device, chunk_len=block_len, chunks_per_slot=1, engine=engine)
        fr = self.full_round
        self.cfg, self.problem, self.block_len, self.k = cfg, fr.problem, block_len, k
        self.n_blocks = fr.n_chunks
        if self.use_stats and self.n_blocks > 0:
            fr.stats = ss.BlockStatsBuffer(self.problem, block_len, self.n_blocks, device)
        b_, hkv = cfg.batch, cfg.n_kv_heads
        self.importance = torch.zeros((b_, hkv, max(self.n_blocks, 1)), dtype=torch.float32, device=device)
        self.selected = torch.full((b_, hkv, k), -1, dtype=torch.int32, device=device)
        self.len_dev = fr.hist_len if cfg.ragged else None
        if gather_per_slot == "auto":
            gather_per_slot = 1
            if narrow_mfma(cfg, engine) and block_len % 32 == 0:
                units = k * b_ * hkv
                gather_per_slot = max(1, min(k, 64, -(-units // (wgs_per_cu(cfg, engine) * device_cus(device)))))
        self.gather_per_slot = int(gather_per_slot)
        self.n_sparse_slots = -(-k // self.gather_per_slot)
        self.state = ss.StateBuffers(self.problem, self.n_sparse_slots + 1, device)
        self.o = torch.empty_like(fr.o)
        self.lse = torch.empty_like(fr.lse)

    def full(self, stream=None):
        self.full_round.run(stream)

    def select(self, stream=None):
        fr = self.full_round
        if self.n_blocks == 0:
            self.selected.fill_(-1)
            return
        if self.use_stats:
            ss.ss_block_importance_stats(self.problem, fr.stats, self.len_dev, fr.max_len, fr.lse, self.importance,
                                         stream)
        else:
            ss.ss_block_importance(self.problem, fr.state, 1, self.n_blocks, fr.lse, self.importance, stream)
        ss.ss_select_blocks(self.problem, self.importance, self.len_dev, fr.max_len, self.block_len, self.k,
                            self.selected, stream)

    def sparse(self, stream=None):
        fr = self.full_round
        ss.ss_verify_chunk_gathered(self.problem, fr.q, fr.hist_view, self.block_len, self.selected, self.state, 1,
                                    stream, chunks_per_slot=self.gather_per_slot)
        ss.ss_verify_candidates(self.problem, fr.q, fr.cand_view, fr.parents, None, self.state, 0, stream)
        ss.ss_merge_states(self.problem, self.state, None, self.o, self.lse, stream)
