"""ctypes binding of libssverify (the C ABI in include/ss_verify.h).

Argument marshalling only: every step of the computation runs in the HIP
library. torch supplies device memory and stream handles. The library is
loaded on first use; if it is missing, every call raises (there is no other
implementation to fall back to).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# The in-tree build; SS_VERIFY_LIB names another build of the same library
# (the host AddressSanitizer build of build.py --asan, for the CPU tests).
LIB_PATH = os.environ.get("SS_VERIFY_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libssverify.so")

SS_OK = 0
SS_ERR_INVALID_ARG = -1
SS_ERR_UNSUPPORTED = -2
SS_ERR_HIP = -3

SS_F32 = 0
SS_BF16 = 1

SS_STREAM_TIMINGS = 1
SS_STREAM_CONTINUE = 2
SS_STREAM_POISON = 4
SS_STREAM_DELAY = 8

SS_ENGINE_AUTO = 0
SS_ENGINE_VALU = 1
SS_ENGINE_MFMA = 2

EXPORTED = ("ss_abi_version", "ss_last_error", "ss_state_bytes", "ss_verify_chunk", "ss_verify_history",
            "ss_verify_candidates", "ss_merge_states", "ss_stream_history", "ss_stream_timings", "ss_tree_mask_host",
            "ss_slot_tokens_host", "ss_history_plan_host", "ss_tier_migration_end", "ss_tier_migrate",
            "ss_kv_copy_rows", "ss_verify_chunk_gathered", "ss_block_importance", "ss_select_blocks",
            "ss_read_probe", "ss_block_stats_bytes", "ss_block_importance_stats", "ss_verify_round",
            "ss_verify_round_noalloc", "ss_mfma_probe")


class SSError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libssverify error {code}: {message}")
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_queries", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("engine", ctypes.c_int32)]


class KVView(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64), ("req_offset", ctypes.c_void_p),
                ("req_len", ctypes.c_void_p), ("max_len", ctypes.c_int32)]


class BlockStats(ctypes.Structure):
    _fields_ = [("buf", ctypes.c_void_p), ("block_len", ctypes.c_int32), ("n_blocks", ctypes.c_int32)]


class State(ctypes.Structure):
    _fields_ = [("acc", ctypes.c_void_p), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m long_context_speculative_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, I32, I64 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.ss_abi_version.restype = I32
        L.ss_abi_version.argtypes = []
        L.ss_last_error.restype = ctypes.c_char_p
        L.ss_last_error.argtypes = []
        L.ss_state_bytes.restype = I64
        L.ss_state_bytes.argtypes = [P(Problem), I32]
        L.ss_verify_chunk.restype = I32
        L.ss_verify_chunk.argtypes = [P(Problem), VP, P(KVView), I32, I32, I32, I32, P(State), I32, VP]
        L.ss_verify_history.restype = I32
        L.ss_verify_history.argtypes = [P(Problem), VP, P(KVView), P(KVView), VP, VP, P(BlockStats), I32,
                                        P(State), I32, VP]
        L.ss_verify_round.restype = I32
        L.ss_verify_round.argtypes = [P(Problem), VP, P(KVView), P(KVView), VP, VP, I32, P(State), VP, VP, VP]
        L.ss_verify_round_noalloc.restype = I32
        L.ss_verify_round_noalloc.argtypes = [P(Problem), VP, P(KVView), P(KVView), VP, VP, VP, VP, VP]
        L.ss_verify_candidates.restype = I32
        L.ss_verify_candidates.argtypes = [P(Problem), VP, P(KVView), VP, VP, P(State), I32, VP]
        L.ss_merge_states.restype = I32
        L.ss_merge_states.argtypes = [P(Problem), P(State), VP, VP, VP, VP]
        L.ss_stream_history.restype = I32
        L.ss_stream_history.argtypes = [P(Problem), VP, VP, VP, I32, I32, I32, VP, I32, P(State), I32, VP, VP, I32]
        L.ss_stream_timings.restype = I32
        L.ss_stream_timings.argtypes = [I32, I32, VP, VP, VP, VP]
        L.ss_tree_mask_host.restype = I32
        L.ss_tree_mask_host.argtypes = [VP, I32, VP]
        L.ss_slot_tokens_host.restype = I32
        L.ss_slot_tokens_host.argtypes = [I32, I32, I32, I32, I32, I32, P(I64), P(I64)]
        L.ss_history_plan_host.restype = I32
        L.ss_history_plan_host.argtypes = [VP, I32, I32, I32, I32, I32, VP, P(I64)]
        L.ss_tier_migration_end.restype = I32
        L.ss_tier_migration_end.argtypes = [I64, I64, I64, I64, P(I64)]
        L.ss_tier_migrate.restype = I32
        L.ss_tier_migrate.argtypes = [P(Problem), P(KVView), VP, VP, VP, VP, I32, I32, VP]
        L.ss_kv_copy_rows.restype = I32
        L.ss_kv_copy_rows.argtypes = [P(Problem), P(KVView), VP, P(KVView), VP, VP, VP]
        L.ss_verify_chunk_gathered.restype = I32
        L.ss_verify_chunk_gathered.argtypes = [P(Problem), VP, P(KVView), I32, VP, I32, I32, P(State), I32, VP]
        L.ss_block_importance.restype = I32
        L.ss_block_importance.argtypes = [P(Problem), P(State), I32, I32, VP, VP, VP]
        L.ss_block_stats_bytes.restype = I64
        L.ss_block_stats_bytes.argtypes = [P(Problem), I32]
        L.ss_block_importance_stats.restype = I32
        L.ss_block_importance_stats.argtypes = [P(Problem), P(BlockStats), VP, I32, VP, VP, VP]
        L.ss_select_blocks.restype = I32
        L.ss_select_blocks.argtypes = [P(Problem), VP, I32, VP, I32, I32, I32, VP, VP]
        L.ss_read_probe.restype = I32
        L.ss_read_probe.argtypes = [VP, I64, I32, VP, VP]
        L.ss_mfma_probe.restype = I32
        L.ss_mfma_probe.argtypes = [VP, I64, I32, I32, VP, VP]
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != SS_OK:
        raise SSError(rc, lib().ss_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# struct builders
# ---------------------------------------------------------------------------

def make_problem(batch, n_q_heads, n_kv_heads, head_dim, n_queries, dtype, scale, engine=SS_ENGINE_AUTO) -> Problem:
    if isinstance(dtype, torch.dtype):
        dtype = SS_F32 if dtype == torch.float32 else SS_BF16
    return Problem(batch, n_q_heads, n_kv_heads, head_dim, n_queries, dtype, scale, engine)


def make_view(k: torch.Tensor, v: torch.Tensor, stride_b: int, stride_h: int, stride_t: int, max_len: int,
              req_offset: Optional[torch.Tensor] = None, req_len: Optional[torch.Tensor] = None) -> KVView:
    return KVView(k.data_ptr(), v.data_ptr(), stride_b, stride_h, stride_t, _ptr(req_offset), _ptr(req_len), max_len)


def head_major_view(k: torch.Tensor, v: torch.Tensor, req_len: Optional[torch.Tensor] = None,
                    max_len: Optional[int] = None) -> KVView:
    """View of [B][Hkv][N][d] tensors (contiguous in the last three axes)."""
    sb, sh, st, sx = k.stride()
    return make_view(k, v, sb, sh, st, k.shape[2] if max_len is None else max_len, None, req_len)


def head_packed_view(k: torch.Tensor, v: torch.Tensor, req_offset: torch.Tensor, req_len: torch.Tensor,
                     max_len: int) -> KVView:
    """View of packed ragged [Hkv][sum N_b][d] tensors (each head's tokens of
    all requests back to back) with device offsets (elements) and lengths."""
    sh, st, sx = k.stride()
    return make_view(k, v, 0, sh, st, max_len, req_offset, req_len)


def token_major_view(k: torch.Tensor, v: torch.Tensor, req_offset: torch.Tensor, req_len: torch.Tensor,
                     max_len: int) -> KVView:
    """View of packed ragged [sum N_b][Hkv][d] tensors with device offsets
    (elements) and lengths per request."""
    st, sh, sx = k.stride()
    return make_view(k, v, 0, sh, st, max_len, req_offset, req_len)


class StateBuffers:
    """Device tensors of n_slots state slots plus the C struct over them."""

    def __init__(self, problem: Problem, n_slots: int, device="cuda"):
        rows = (n_slots, problem.batch, problem.n_queries, problem.n_q_heads)
        self.acc = torch.empty(rows + (problem.head_dim,), dtype=torch.float32, device=device)
        self.m = torch.empty(rows, dtype=torch.float32, device=device)
        self.l = torch.empty(rows, dtype=torch.float32, device=device)
        self.n_slots = n_slots
        self.struct = State(self.acc.data_ptr(), self.m.data_ptr(), self.l.data_ptr(), n_slots)


# ---------------------------------------------------------------------------
# the calls (same names as the C ABI)
# ---------------------------------------------------------------------------

def ss_abi_version() -> int:
    return lib().ss_abi_version()


def ss_state_bytes(problem: Problem, n_slots: int) -> int:
    r = lib().ss_state_bytes(ctypes.byref(problem), n_slots)
    if r < 0:
        _check(int(r))
    return int(r)


def ss_verify_chunk(problem: Problem, q: torch.Tensor, hist: KVView, chunk_len: int, chunk_begin: int,
                    n_chunks: int, chunks_per_slot: int, out: StateBuffers, slot_begin: int, stream=None) -> None:
    _check(lib().ss_verify_chunk(ctypes.byref(problem), q.data_ptr(), ctypes.byref(hist), chunk_len, chunk_begin,
                                 n_chunks, chunks_per_slot, ctypes.byref(out.struct), slot_begin, _stream(stream)))


def ss_verify_history(problem: Problem, q: torch.Tensor, hist: KVView, cand: Optional[KVView],
                      parents: Optional[torch.Tensor], mask_out: Optional[torch.Tensor], n_slots: int,
                      out: StateBuffers, slot_begin: int, stream=None, stats: Optional["BlockStatsBuffer"] = None
                      ) -> None:
    _check(lib().ss_verify_history(ctypes.byref(problem), q.data_ptr(), ctypes.byref(hist),
                                   None if cand is None else ctypes.byref(cand), _ptr(parents), _ptr(mask_out),
                                   None if stats is None else ctypes.byref(stats.struct), n_slots,
                                   ctypes.byref(out.struct), slot_begin, _stream(stream)))


def ss_verify_candidates(problem: Problem, q: torch.Tensor, cand: KVView, parents: Optional[torch.Tensor],
                         mask_out: Optional[torch.Tensor], out: StateBuffers, slot: int, stream=None) -> None:
    _check(lib().ss_verify_candidates(ctypes.byref(problem), q.data_ptr(), ctypes.byref(cand), _ptr(parents),
                                      _ptr(mask_out), ctypes.byref(out.struct), slot, _stream(stream)))


def ss_merge_states(problem: Problem, states: StateBuffers, slots_per_req: Optional[torch.Tensor],
                    o: torch.Tensor, lse: torch.Tensor, stream=None) -> None:
    _check(lib().ss_merge_states(ctypes.byref(problem), ctypes.byref(states.struct), _ptr(slots_per_req),
                                 o.data_ptr(), lse.data_ptr(), _stream(stream)))


def ss_verify_round(problem: Problem, q: torch.Tensor, hist: KVView, cand: KVView, parents: Optional[torch.Tensor],
                    mask_out: Optional[torch.Tensor], n_slots: int, work: StateBuffers, o: torch.Tensor,
                    lse: torch.Tensor, stream=None) -> None:
    _check(lib().ss_verify_round(ctypes.byref(problem), q.data_ptr(), ctypes.byref(hist), ctypes.byref(cand),
                                 _ptr(parents), _ptr(mask_out), n_slots, ctypes.byref(work.struct), o.data_ptr(),
                                 lse.data_ptr(), _stream(stream)))


def ss_verify_round_noalloc(problem: Problem, q: torch.Tensor, hist: KVView, cand: KVView,
                            parents: Optional[torch.Tensor], mask_out: Optional[torch.Tensor], o: torch.Tensor,
                            lse: torch.Tensor, stream=None) -> None:
    _check(lib().ss_verify_round_noalloc(ctypes.byref(problem), q.data_ptr(), ctypes.byref(hist),
                                         ctypes.byref(cand), _ptr(parents), _ptr(mask_out), o.data_ptr(),
                                         lse.data_ptr(), _stream(stream)))


def ss_stream_history(problem: Problem, q: torch.Tensor, host_kv: torch.Tensor, chunk_len: int, n_chunks: int,
                      staging: torch.Tensor, n_buf: int, out: StateBuffers, slot_begin: int, copy_stream,
                      compute_stream, record_timings: bool = False, req_len: Optional[torch.Tensor] = None,
                      chunks_per_copy: int = 1, continue_ring: bool = False, checks: int = 0) -> None:
    """checks: SS_STREAM_POISON and/or SS_STREAM_DELAY (ordering diagnostics)."""
    flags = (SS_STREAM_TIMINGS if record_timings else 0) | (SS_STREAM_CONTINUE if continue_ring else 0) | checks
    _check(lib().ss_stream_history(ctypes.byref(problem), q.data_ptr(), host_kv.data_ptr(), _ptr(req_len), chunk_len,
                                   n_chunks, chunks_per_copy, staging.data_ptr(), n_buf, ctypes.byref(out.struct),
                                   slot_begin, _stream(copy_stream), _stream(compute_stream), flags))


def ss_stream_timings(n_chunks: int, back: int = 0):
    """Per-chunk (copy_begin, copy_end, compute_begin, compute_end) in ms from
    the compute stream's frontier at the timed call `back` calls ago."""
    bufs = [(ctypes.c_float * n_chunks)() for _ in range(4)]
    _check(lib().ss_stream_timings(back, n_chunks, *[ctypes.addressof(b) for b in bufs]))
    return [list(b) for b in bufs]


def ss_tree_mask_host(parents) -> list:
    n = len(parents)
    par = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in parents])
    out = (ctypes.c_uint64 * max(n, 1))()
    _check(lib().ss_tree_mask_host(ctypes.addressof(par), n, ctypes.addressof(out)))
    return [int(out[i]) for i in range(n)]


def ss_slot_tokens_host(length: int, chunk_len: int, chunk_begin: int, n_chunks: int, chunks_per_slot: int,
                        s: int):
    t0, t1 = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ss_slot_tokens_host(length, chunk_len, chunk_begin, n_chunks, chunks_per_slot, s,
                                     ctypes.byref(t0), ctypes.byref(t1)))
    return t0.value, t1.value


def ss_history_plan_host(lens, n_kv_heads: int, max_len: int, n_wg: int, n_slots: int):
    """The balanced cut of ss_verify_history: (plan, piece_len) with plan an
    int64 array [batch][n_kv_heads][n_slots][4] of {work-group, t0, t1,
    writes}."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    plan = np.empty((len(lens), n_kv_heads, n_slots, 4), dtype=np.int64)
    piece = ctypes.c_int64()
    _check(lib().ss_history_plan_host(lens.ctypes.data, len(lens), n_kv_heads, max_len, n_wg, n_slots,
                                      plan.ctypes.data, ctypes.byref(piece)))
    return plan, piece.value


def _i64(values):
    import numpy as np
    return np.ascontiguousarray(np.asarray(values, dtype=np.int64))


def ss_tier_migration_end(h: int, c: int, tail: int, gran: int) -> int:
    e = ctypes.c_int64()
    _check(lib().ss_tier_migration_end(h, c, tail, gran, ctypes.byref(e)))
    return e.value


def ss_tier_migrate(problem: Problem, tail: KVView, tail_first, begin, end, host_kv: torch.Tensor, chunk_len: int,
                    n_chunks: int, stream=None) -> None:
    a, b_, e = _i64(tail_first), _i64(begin), _i64(end)
    _check(lib().ss_tier_migrate(ctypes.byref(problem), ctypes.byref(tail), a.ctypes.data, b_.ctypes.data,
                                 e.ctypes.data, host_kv.data_ptr(), chunk_len, n_chunks, _stream(stream)))


def ss_kv_copy_rows(problem: Problem, src: KVView, src_row, dst: KVView, dst_row, n_rows, stream=None) -> None:
    a, b_, n = _i64(src_row), _i64(dst_row), _i64(n_rows)
    _check(lib().ss_kv_copy_rows(ctypes.byref(problem), ctypes.byref(src), a.ctypes.data, ctypes.byref(dst),
                                 b_.ctypes.data, n.ctypes.data, _stream(stream)))


def ss_verify_chunk_gathered(problem: Problem, q: torch.Tensor, hist: KVView, chunk_len: int, chunk_idx: torch.Tensor,
                             out: StateBuffers, slot_begin: int, stream=None, chunks_per_slot: int = 1) -> None:
    """chunk_idx: device int32 [B][Hkv][n_sel]; slot slot_begin + s merges
    entries [s * chunks_per_slot, (s + 1) * chunks_per_slot)."""
    _check(lib().ss_verify_chunk_gathered(ctypes.byref(problem), q.data_ptr(), ctypes.byref(hist), chunk_len,
                                          chunk_idx.data_ptr(), chunk_idx.shape[-1], chunks_per_slot,
                                          ctypes.byref(out.struct), slot_begin, _stream(stream)))


def ss_block_importance(problem: Problem, states: StateBuffers, slot_begin: int, n_blocks: int, lse: torch.Tensor,
                        importance: torch.Tensor, stream=None) -> None:
    _check(lib().ss_block_importance(ctypes.byref(problem), ctypes.byref(states.struct), slot_begin, n_blocks,
                                     lse.data_ptr(), importance.data_ptr(), _stream(stream)))


def ss_block_stats_bytes(problem: Problem, n_blocks: int) -> int:
    r = lib().ss_block_stats_bytes(ctypes.byref(problem), n_blocks)
    _check(int(r) if r < 0 else 0)
    return int(r)


class BlockStatsBuffer:
    """Device buffer for the block statistics ss_verify_history records."""

    def __init__(self, problem: Problem, block_len: int, n_blocks: int, device="cuda"):
        n = ss_block_stats_bytes(problem, n_blocks)
        self.buf = torch.empty(n // 4, dtype=torch.float32, device=device)
        self.struct = BlockStats(self.buf.data_ptr(), block_len, n_blocks)
        self.block_len, self.n_blocks = block_len, n_blocks


def ss_block_importance_stats(problem: Problem, stats: BlockStatsBuffer, req_len: Optional[torch.Tensor], max_len: int,
                              lse: torch.Tensor, importance: torch.Tensor, stream=None) -> None:
    """req_len / max_len: the lengths of the history view the statistics were
    recorded over (req_len device int32 [B], or None: all max_len)."""
    _check(lib().ss_block_importance_stats(ctypes.byref(problem), ctypes.byref(stats.struct), _ptr(req_len), max_len,
                                           lse.data_ptr(), importance.data_ptr(), _stream(stream)))


def ss_select_blocks(problem: Problem, importance: torch.Tensor, req_len: Optional[torch.Tensor], max_len: int,
                     block_len: int, k: int, out: torch.Tensor, stream=None) -> None:
    """importance: device float32 [B][Hkv][n_blocks]; out: device int32 [B][Hkv][k]."""
    _check(lib().ss_select_blocks(ctypes.byref(problem), importance.data_ptr(), importance.shape[-1], _ptr(req_len),
                                  max_len, block_len, k, out.data_ptr(), _stream(stream)))


def ss_read_probe(src: torch.Tensor, n_work_groups: int, sink: torch.Tensor, stream=None) -> None:
    """Reads all of src (a 16-byte multiple) with n_work_groups contiguous spans."""
    _check(lib().ss_read_probe(src.data_ptr(), src.numel() * src.element_size(), n_work_groups, sink.data_ptr(),
                               _stream(stream)))


MFMA_PROBE_FLOPS_PER_WAVE_ITER = 8 * 16384  # eight 16x16x32 products per wave and iteration


def ss_mfma_probe(operands: torch.Tensor, iters: int, n_work_groups: int, sink: torch.Tensor, stream=None) -> int:
    """Matrix-core probe over bf16 operands (>= 8192 elements); returns the
    launch's floating-point operation count (work-groups of four waves)."""
    _check(lib().ss_mfma_probe(operands.data_ptr(), operands.numel(), iters, n_work_groups, sink.data_ptr(),
                               _stream(stream)))
    return n_work_groups * 4 * iters * MFMA_PROBE_FLOPS_PER_WAVE_ITER
