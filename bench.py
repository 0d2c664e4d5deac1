"""Benchmark of one verification round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole resident hot path over one batch of
synthetic input already in HBM: ss_verify_history over every request's
committed history (with the candidate region folded into the same launch on
the MFMA kernels, narrow and wide-row, else ss_verify_candidates after it)
and ss_merge_states. The headline workload is the largest single-GPU one,
the InternLM2.5-7B-like layer: 32 requests with ragged committed histories
(uniform in [8192, 65536] tokens, seed-drawn), 32 query heads over 8 KV
heads, head_dim 128, bf16, 5 queries (4 drafts + 1) under a causal
candidate mask. The same line carries sub-records for the Qwen3-8B-like
layer (uniform 32768 tokens, HBM-bound) and the 72B-like tree workload
(64-node candidate tree under 8-way GQA, bound by the matrix cores).

Prints ONE JSON line. value = effective KV GB/s = (history + candidate K/V
bytes) / time per step. Also reported: verified query-tokens/s, the history
launch's roofline (algorithmic bytes, or FLOPs for wide row groups, per
launch / its event-timed duration; for the MFMA-bound launch also against
a same-run matrix-core probe on N(0,1) bf16 operands, whose rate sets the
attainable ceiling for such data), the streamed path on the streamed
workload (host-link GB/s against a plain pinned H2D copy of the same bytes),
and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_speculative_amd import rounds  # noqa: E402
from long_context_speculative_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
CSRC = "long_context_speculative_amd/csrc/"


def chunk_kernel_sources(cfg, engine="auto"):
    """Source files of the chunk kernel that serves cfg (mirrors the library's
    engine choice)."""
    bf16_128 = cfg.dtype == "bf16" and cfg.head_dim == 128
    mfma_bf16 = cfg.dtype == "bf16" and cfg.head_dim in (64, 128)
    if engine != "valu" and cfg.dtype == "f32":
        main = "ss_mfma_f32.hip"
    elif engine == "valu" or not mfma_bf16:
        main = "ss_valu_small.hip" if bf16_128 and cfg.rows < 16 else "ss_valu.hip"
    elif cfg.rows <= 32:
        main = "ss_mfma.hip"
    else:
        main = "ss_mfma_wide.hip"
    return [CSRC + main, CSRC + "ss_common.h", "long_context_speculative_amd/build.py"]


def kv_bytes(cfg, hist_len) -> tuple[int, int]:
    row = 2 * cfg.n_kv_heads * cfg.head_dim * cfg.elem_bytes
    return int(np.asarray(hist_len, dtype=np.int64).sum()) * row, cfg.batch * cfg.n_queries * row


def chunk_kernel_bytes(cfg, hist_len, n_slots, with_cand=False) -> int:
    """Algorithmic bytes of one history-kernel launch: the history K and V
    once, Q once, the state slots written (acc + m + l, fp32), and the
    candidate K and V when the launch also attends the candidate region."""
    hist, cand = kv_bytes(cfg, hist_len)
    q = cfg.batch * cfg.n_queries * cfg.n_q_heads * cfg.head_dim * cfg.elem_bytes
    states = n_slots * cfg.batch * cfg.n_queries * cfg.n_q_heads * (cfg.head_dim + 2) * 4
    return hist + q + states + (cand if with_cand else 0)


def launch_bytes(cfg, hist_len, rnd) -> int:
    """Algorithmic bytes of the timed history launch of a resident round."""
    if rnd.fused:
        return chunk_kernel_bytes(cfg, hist_len, rnd.n_call_slots, with_cand=True)
    return chunk_kernel_bytes(cfg, hist_len, rnd.n_hist_slots)


def chunk_kernel_flops(cfg, hist_len) -> int:
    """Algorithmic FLOPs of one chunk-kernel launch: S = Q K^T and O = P V,
    2 * d FLOPs each per (query head, query, history key)."""
    return 4 * cfg.n_q_heads * cfg.n_queries * cfg.head_dim * int(np.asarray(hist_len, dtype=np.int64).sum())


def source_hash(cfg, engine="auto") -> str:
    h = hashlib.sha256()
    for p in chunk_kernel_sources(cfg, engine):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_matches(text, cfg, split, fused, slots) -> bool:
    """Whether a committed counter summary was taken on the current kernel
    source with the same history cut, candidate placement and slot count."""
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_split = re.search(r"history_split:\s*(\w+)", text)
    m_fused = re.search(r"fused_candidates:\s*(\w+)", text)
    m_slots = re.search(r"history_slots:\s*(\d+)", text)
    if not m_hash or m_hash.group(1) != source_hash(cfg):
        return False
    if (m_split.group(1) if m_split else "chunks") != split:
        return False
    if (m_fused.group(1) == "True" if m_fused else False) != fused:
        return False
    return m_slots is not None and int(m_slots.group(1)) == slots


def read_traffic(cfg, split, fused, slots):
    """HBM bytes per chunk-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source with the same
    history cut, candidate placement and slot count; else None."""
    path = os.path.join(ROOT, "profiles", f"chunk_kernel_{cfg.name}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_bytes or not profile_matches(text, cfg, split, fused, slots):
        return None
    return float(m_bytes.group(1))


def read_profile_value(cfg, key, split, fused, slots):
    """A number recorded in the committed counter summary of cfg's history
    launch, if it was taken in the same configuration (profile_matches);
    else None."""
    path = os.path.join(ROOT, "profiles", f"chunk_kernel_{cfg.name}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(re.escape(key) + r":\s*([0-9.eE+]+)", text)
    if not m or not profile_matches(text, cfg, split, fused, slots):
        return None
    return float(m.group(1))


def make_round(cfg, inp, cps="auto", engine="auto", split="balanced"):
    """The resident round in the launch configuration the benchmark times
    (rounds.BENCH_RESIDENT unless overridden)."""
    kw = dict(rounds.BENCH_RESIDENT)
    kw.update(chunks_per_slot=cps, split=split)
    return rounds.ResidentRound(inp, engine=engine, **kw)


# Sustained load after idle makes the device's clock and power management
# swing for tens of milliseconds: traced on MI355X, the history launch runs
# up to 40% slower a few milliseconds into a burst and returns to its steady
# duration after about 30 ms. Every timed loop is therefore preceded by this
# much untimed device work of the same kind.
SETTLE_S = 0.3


def settle(fn, seconds=SETTLE_S):
    """Runs fn (an enqueue of device work) untimed for `seconds` of wall
    time, synchronising every few calls."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_resident(cfg, steps, warmup, cps="auto", engine="auto", split="balanced"):
    """Step time over `steps` timed steps (events only at the two ends, so no
    marker sits between the launches), then the history launch's own
    duration from HIP events around each launch over another `steps` steps
    on the same stream. Before each: `warmup` steps and the settle time."""
    inp = wl.make_inputs(cfg)
    rnd = make_round(cfg, inp, cps, engine, split)
    rnd.inputs_sha256 = wl.input_digest(inp)
    del inp
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        rnd.run()
    settle(rnd.run)
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for _ in range(steps):
        rnd.run()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_begin.elapsed_time(t_end) / steps
    settle(rnd.run, 0.1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        rnd.chunks()
        ev[k][1].record(stream)
        rnd.candidates()
        rnd.merge()
    torch.cuda.synchronize()
    ms_chunk = sum(a.elapsed_time(b) for a, b in ev) / steps
    hist_len = np.full(cfg.batch, cfg.hist_len) if not cfg.ragged else rnd.hist_len.cpu().numpy()
    return rnd, hist_len, ms_step, ms_chunk


def time_streamed(cfg, reps=3):
    """The streamed round (one copy per 64 MiB chunk, two staging buffers)
    against a plain pinned H2D copy of the same chunks, and the same round
    with two chunks per copy (fewer copy-engine starts and event waits)."""
    inp = wl.make_inputs(cfg)
    srd = rounds.StreamedRound(inp, n_buf=2)
    grouped = rounds.StreamedRound(inp, n_buf=2, chunks_per_copy=2)
    del inp
    srd.run()
    torch.cuda.synchronize()
    walls = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        srd.run(record_timings=True)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    from long_context_speculative_amd import ssverify as ss
    c0, c1, k0, k1 = ss.ss_stream_timings(srd.n_chunks)
    bubble = rounds.exposed_wait((c0, c1, k0, k1))
    # plain pinned H2D copy of the same bytes, same chunking, one stream
    dst = srd.staging
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s = srd.copy_stream
    with torch.cuda.stream(s):
        for j in range(srd.n_chunks):
            dst[j % srd.n_buf].copy_(srd.host_kv[j], non_blocking=True)
    torch.cuda.synchronize()
    copy_wall = time.perf_counter() - t0
    hist_bytes = srd.host_kv.numel() * srd.host_kv.element_size()
    wall = min(walls)
    grouped.run()
    torch.cuda.synchronize()
    g_walls = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        grouped.run()
        torch.cuda.synchronize()
        g_walls.append(time.perf_counter() - t0)
    g_wall = min(g_walls)
    del grouped
    torch.cuda.empty_cache()
    return {
        "workload": cfg.name,
        "host_link_GBps": hist_bytes / wall / 1e9,
        "plain_h2d_GBps": hist_bytes / copy_wall / 1e9,
        "frac_of_plain_h2d": copy_wall / wall,
        "ms_per_round": wall * 1e3,
        "exposed_wait_ms": bubble,
        "chunk_compute_ms_mean": float(np.mean([k1[j] - k0[j] for j in range(srd.n_chunks)])),
        "chunk_copy_ms_mean": float(np.mean([c1[j] - c0[j] for j in range(srd.n_chunks)])),
        "query_tokens_per_s": cfg.batch * cfg.n_queries / wall,
        "two_chunks_per_copy": {"host_link_GBps": hist_bytes / g_wall / 1e9, "frac_of_plain_h2d": copy_wall / g_wall,
                                "ms_per_round": g_wall * 1e3},
    }


def time_layered(cfg, n_layers=4, hist_len=16384, rest_dim=8192, rest_reps=2, reps=3):
    """Cross-layer prefetch and grouped transfers (SpecStream section 4.2):
    n_layers layers of the streamed workload's shape (history cut to
    hist_len tokens per layer), each followed on the compute stream by a
    stand-in for the rest of the layer (bf16 matrix products), with the
    staging ring continued across layers (the next layer's chunks are copied
    while the current one finishes) or restarted per layer."""
    lcfg = cfg.with_(hist_len=hist_len)
    inputs = [wl.make_inputs(lcfg.with_(seed=lcfg.seed + 100 * i)) for i in range(n_layers)]
    lr = rounds.LayeredStreamedRound(inputs, n_buf=2, chunks_per_copy=2, rest_dim=rest_dim, rest_reps=rest_reps)
    del inputs
    out = {"workload": f"{n_layers} layers of {cfg.name} with {hist_len} history tokens each, "
                       f"rest of layer = {rest_reps} bf16 {rest_dim}^2 matrix products",
           "chunks_per_copy": 2, "n_buf": 2}
    for prefetch in (False, True):
        lr.run(prefetch=prefetch)
        torch.cuda.synchronize()
        walls = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            lr.run(prefetch=prefetch, record_timings=True)
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t0)
        key = "prefetch" if prefetch else "no_prefetch"
        out[key] = {"ms_per_round": min(walls) * 1e3,
                    "exposed_wait_ms_per_layer": [round(w, 3) for w in lr.layer_waits()]}
    # the rest-of-layer stand-in alone
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(lr.layers[0].compute_stream):
        x = lr.rest_a
        for _ in range(rest_reps * n_layers):
            x = torch.mm(x, lr.rest_b)
    torch.cuda.synchronize()
    out["rest_of_layers_ms"] = (time.perf_counter() - t0) * 1e3
    out["round_speedup_from_prefetch"] = out["no_prefetch"]["ms_per_round"] / out["prefetch"]["ms_per_round"]
    return out


def read_probe(n_bytes=2 << 30, reps=10):
    """Same-run HBM read reference (ss_read_probe): the history kernels' load
    shape over n_bytes of N(0,1) bf16 data (like the KV history), with one
    work-group per CU (their launch shape) and with eight."""
    from long_context_speculative_amd import ssverify as ss
    cus = rounds.device_cus()
    src = torch.randn(n_bytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    out = {"bytes": n_bytes}
    for name, wgs in (("one_per_cu_GBps", cus), ("eight_per_cu_GBps", 8 * cus)):
        settle(lambda: ss.ss_read_probe(src, wgs, sink), 0.2)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            ss.ss_read_probe(src, wgs, sink)
        b.record()
        torch.cuda.synchronize()
        out[name] = round(n_bytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9, 1)
    del src
    torch.cuda.empty_cache()
    return out


def mfma_probe(iters=4096, reps=20):
    """Same-run matrix-core reference (ss_mfma_probe): bf16 MFMA products and
    nothing else, two work-groups of four waves per CU (two waves per SIMD, as
    the wide-row kernel runs), on N(0,1) bf16 operands like the attention
    inputs. The clock the chip holds depends on the operand values, so this is
    the attainable rate for such data; the published peak assumes 2.4 GHz."""
    from long_context_speculative_amd import ssverify as ss
    cus = rounds.device_cus()
    ops = torch.randn(1 << 22, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    wgs = 2 * cus
    settle(lambda: ss.ss_mfma_probe(ops, iters, wgs, sink), 0.2)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        flops = ss.ss_mfma_probe(ops, iters, wgs, sink)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tflops = flops / (ms * 1e-3) / 1e12
    del ops
    torch.cuda.empty_cache()
    return {"TFLOPs": round(tflops, 1), "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "ms_per_launch": round(ms, 4), "work_groups": wgs, "operands": "N(0,1) bf16"}


def hold(workload, seconds, probe=False):
    """Back-to-back calls of one workload's resident round (or of the
    matrix-core probe) for `seconds`, synchronising every 8 calls; prints a
    line when the loop starts and one with the time per call at the end."""
    from long_context_speculative_amd import ssverify as ss
    if probe:
        ops = torch.randn(1 << 22, dtype=torch.bfloat16, device="cuda")
        sink = torch.zeros(256, dtype=torch.float32, device="cuda")
        wgs = 2 * rounds.device_cus()
        fn, name = (lambda: ss.ss_mfma_probe(ops, 4096, wgs, sink)), "mfma_probe"
    else:
        cfg = wl.CONFIGS[workload]
        inp = wl.make_inputs(cfg)
        rnd = make_round(cfg, inp)
        del inp
        fn, name = rnd.run, workload
    fn()
    torch.cuda.synchronize()
    print(json.dumps({"hold": name, "seconds": seconds, "state": "running"}), flush=True)
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
    print(json.dumps({"hold": name, "calls": n, "ms_per_call": round((time.perf_counter() - t0) / n * 1e3, 4)}),
          flush=True)


def time_sparse(cfg, block_len=512, k=16, reps=20):
    """Block statistics and block-sparse verification on the resident
    workload, with the importance signal taken two ways: from a full round
    with one state slot per block (ss_verify_chunk), and from the block
    statistics that the benchmarked full round (balanced cut, candidates
    fused) records as it goes. Then the per-head top-k selection and the
    sparse round over the kept blocks; the sparse result is compared with
    the full one on the GPU."""
    inp = wl.make_inputs(cfg)
    modes = {"block_slots": rounds.SparseRound(inp, block_len, k),
             "stats": rounds.SparseRound(inp, block_len, k, stats=True)}
    plain = rounds.ResidentRound(inp, **rounds.BENCH_RESIDENT)
    del inp
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        settle(fn, 0.1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ms_plain = timed(plain.run)
    hist_b, cand_b = kv_bytes(cfg, np.full(cfg.batch, cfg.hist_len))
    out = {"full_round_plain_ms": ms_plain}
    for name, sr in modes.items():
        ms_full = timed(sr.full)
        ms_select = timed(sr.select)
        ms_sparse = timed(sr.sparse)
        torch.cuda.synchronize()
        o_full, o_sparse = sr.full_round.o, sr.o
        kept = (sr.selected >= 0).sum().item() / (cfg.batch * cfg.n_kv_heads)
        kept_b = hist_b * kept / sr.n_blocks
        out["workload"] = (f"{cfg.name}, blocks of {block_len} tokens, {k} of {sr.n_blocks} kept per "
                           f"(request, KV head)")
        out[name] = {
            "full_round_ms": ms_full,
            "importance_and_select_ms": ms_select,
            "sparse_round_ms": ms_sparse,
            "sparse_kept_KV_GBps": (kept_b + cand_b) / (ms_sparse * 1e-3) / 1e9,
            "speedup_vs_plain_full_round": ms_plain / ms_sparse,
            "max_abs_O_sparse_vs_full": float((o_sparse - o_full).abs().max().item()),
            "mean_abs_O_sparse_vs_full": float((o_sparse - o_full).abs().mean().item()),
        }
    out["stats_recording_overhead"] = out["stats"]["full_round_ms"] / ms_plain - 1.0
    # the two importance signals round differently: near-ties at the k-th
    # place may fall either way
    a, b = modes["stats"].selected, modes["block_slots"].selected
    common = (a.unsqueeze(-1) == b.unsqueeze(-2)) & (a >= 0).unsqueeze(-1)
    out["selected_blocks_overlap"] = common.any(-1).sum().item() / max(1, (a >= 0).sum().item())
    return out


def time_tiered(cfg, n_rounds=8, tail=512, gran=16):
    """Commit-aware tiering (SpecStream section 4.1) on the streamed
    workload's shape: every request starts with its whole committed history,
    Eq. (5) seals all but the Active Tail into the pinned host store (the
    bulk migration is timed), then rounds stream the sealed history, attend
    the tail and the candidates, commit a random prefix of the candidates and
    migrate per Eq. (5), whose small granularity makes migrations fire inside
    the timed rounds. Two passes of n_rounds: migrations serialised after
    each round's verification, then overlapped with the next round's (the
    copies run on a stream of their own, H moves once they landed); a round
    is timed to the end of its own work on the current stream."""
    inp = wl.make_inputs(cfg)
    b_, hkv, d, nq = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_queries
    hist_k = [inp.k_hist[b] for b in range(b_)]
    hist_v = [inp.v_hist[b] for b in range(b_)]
    tr = rounds.TieredRound(cfg, hist_k, hist_v, tail_target=tail, gran=gran, chunk_len=cfg.chunk_len,
                            max_tokens=cfg.hist_len + 4 * nq * (2 * n_rounds + 2))
    del inp, hist_k, hist_v
    # a plain pinned device-to-host copy of the same bytes, for reference
    n_bytes = tr.init_migrated_bytes
    src = torch.empty(n_bytes // cfg.elem_bytes, dtype=cfg.torch_dtype, device="cuda")
    dst = torch.empty_like(src, device="cpu").pin_memory()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    plain_d2h = n_bytes / (time.perf_counter() - t0) / 1e9
    del src, dst
    gen = torch.Generator().manual_seed(cfg.seed)
    rng = np.random.default_rng(cfg.seed)
    cur = torch.cuda.current_stream()
    out = {"workload": f"{cfg.name} with commit-aware tiering (T={tail}, g={gran})"}
    for mode in ("serialised", "overlapped"):
        overlap = mode == "overlapped"
        walls, verify_ms, mig_ms, sealed = [], [], [], []
        migrated = 0
        for r in range(n_rounds + 1):
            q = torch.randn((b_, nq, cfg.n_q_heads, d), generator=gen).to(cfg.torch_dtype).cuda()
            kc = torch.randn((b_, hkv, nq, d), generator=gen).to(cfg.torch_dtype).cuda()
            vc = torch.randn((b_, hkv, nq, d), generator=gen).to(cfg.torch_dtype).cuda()
            acc = [int(x) for x in rng.integers(0, nq + 1, size=b_)]
            cur.synchronize()
            t0 = time.perf_counter()
            tr.verify(q, kc, vc)
            cur.synchronize()
            t1 = time.perf_counter()
            h0 = list(tr.pending[0]) if tr.pending is not None else list(tr.H)
            tr.commit(acc)
            tr.migrate(overlap=overlap)
            cur.synchronize()                   # this round's own work; overlapped copies run on
            t2 = time.perf_counter()
            moved = sum(e - h for e, h in zip(tr.pending[0] if tr.pending else tr.H, h0))
            if r > 0:                           # the first round warms up
                walls.append(t2 - t0)
                verify_ms.append((t1 - t0) * 1e3)
                sealed.append(sum(tr.H))
                migrated += moved
            if moved and r > 0:
                mig_ms.append(tr.last_migration)
        tr.finalize()
        torch.cuda.synchronize()
        mig_ms = [a.elapsed_time(b) for a, b in mig_ms]
        out[mode] = {"ms_per_round": float(np.mean(walls)) * 1e3, "verify_ms": float(np.mean(verify_ms)),
                     "tokens_migrated_in_rounds": int(migrated), "migrations": len(mig_ms),
                     "migration_copy_ms_mean": float(np.mean(mig_ms)) if mig_ms else None}
    wall = out["overlapped"]["ms_per_round"] * 1e-3
    chunk_bytes = tr.host_kv[0].numel() * tr.host_kv.element_size()
    streamed = -(-max(tr.H) // cfg.chunk_len) * chunk_bytes
    out.update({
        "host_link_GBps": streamed / (out["overlapped"]["verify_ms"] * 1e-3) / 1e9,
        "sealed_tokens_per_request": float(sum(tr.H)) / b_,
        "active_tail_tokens_per_request": float(np.mean([c - h for c, h in zip(tr.C, tr.H)])),
        "bulk_migration_GBps": n_bytes / (tr.init_migrate_ms * 1e-3) / 1e9,
        "plain_d2h_GBps": plain_d2h,
        "tokens_migrated_in_rounds": out["overlapped"]["tokens_migrated_in_rounds"]
        + out["serialised"]["tokens_migrated_in_rounds"],
        "query_tokens_per_s": b_ * nq / wall,
    })
    return out


def cpu_baseline(cfg, budget_s=15.0):
    """The fp64 oracle, as it stands, on (request, KV head) slices of the same
    workload until about budget_s seconds of CPU time are spent."""
    import oracle
    from threadpoolctl import threadpool_info
    inp = wl.make_inputs(cfg.with_(batch=min(cfg.batch, 2)))
    vis = np.stack([oracle.chain_mask(cfg.n_queries)] * inp.cfg.batch) if cfg.mask != "tree" else \
        np.stack([oracle.tree_mask(inp.parents[b]) for b in range(inp.cfg.batch)])
    q = inp.q.float().numpy()
    kc, vc = inp.k_cand.float().numpy(), inp.v_cand.float().numpy()
    kh, vh = inp.hist_per_request("k"), inp.hist_per_request("v")
    done, slices, keys = 0.0, 0, 0
    t0 = time.perf_counter()
    while done < budget_s:
        b, g = divmod(slices % (inp.cfg.batch * cfg.n_kv_heads), cfg.n_kv_heads)
        oracle.attention_reference(q, kh, vh, inp.hist_len, kc, vc, vis, cfg.scale, requests=[b], kv_heads=[g])
        slices += 1
        keys += int(inp.hist_len[b]) + cfg.n_queries
        done = time.perf_counter() - t0
    row = 2 * cfg.head_dim * cfg.elem_bytes
    kv = keys * row
    cores = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    # the whole tiny fp32 round (c1) on one thread
    from threadpoolctl import threadpool_limits
    c1 = wl.CONFIGS["c1_tiny_f32"]
    inp1 = wl.make_inputs(c1)
    vis1 = np.stack([oracle.chain_mask(c1.n_queries)] * c1.batch)
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        oracle.attention_reference(inp1.q.float().numpy(), inp1.hist_per_request("k"), inp1.hist_per_request("v"),
                                   inp1.hist_len, inp1.k_cand.float().numpy(), inp1.v_cand.float().numpy(), vis1,
                                   c1.scale)
        c1_ms = (time.perf_counter() - t1) * 1e3
    return {"value": kv / done / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "c1_round_one_thread_ms": round(c1_ms, 3),
            "sample": f"{slices} (request, KV head) slices of {cfg.name}, fp64 NumPy, {done:.1f} s",
            "query_tokens_per_s": slices / (cfg.batch * cfg.n_kv_heads) * cfg.batch * cfg.n_queries / done,
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def counters_pass(cfg, cps="auto", engine="auto", split="balanced", settle_s=0.0):
    """One calibration kernel of known traffic (torch.neg over 2^30 bytes of
    bf16: reads 1 GiB, writes 1 GiB), then one step of the workload; with
    settle_s > 0, that many seconds of the same steps before the last one (so
    the last dispatches run in the steady state the timed loops measure)."""
    src = torch.randn(1 << 29, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    inp = wl.make_inputs(cfg)
    rnd = make_round(cfg, inp, cps, engine, split)
    del inp
    torch.cuda.synchronize()
    if settle_s > 0:
        settle(rnd.run, settle_s)
    rnd.run()
    cps = rnd.cps
    torch.cuda.synchronize()
    hist_len = np.full(cfg.batch, cfg.hist_len) if not cfg.ragged else rnd.hist_len.cpu().numpy()
    print(json.dumps({"counters_pass": cfg.name, "calibration_bytes": 1 << 30, "chunks_per_slot": cps,
                      "split": rnd.split, "history_slots": rnd.n_hist_slots,
                      "fused_candidates": rnd.fused,
                      "chunk_kernel_algorithmic_bytes": launch_bytes(cfg, hist_len, rnd)}),
          flush=True)


DEFAULT_WORKLOAD = "c3_internlm25_7b_ragged"


def workload_desc(cfg) -> str:
    return (f"{cfg.name}: B={cfg.batch}, Hq={cfg.n_q_heads}, Hkv={cfg.n_kv_heads}, d={cfg.head_dim}, "
            f"history={'U[%d, %d]' % (cfg.ragged_lo, cfg.hist_len) if cfg.ragged else cfg.hist_len}"
            f" ({'ragged' if cfg.ragged else 'uniform'}), chunk={cfg.chunk_len}, q={cfg.n_queries}, mask={cfg.mask}")


def resident_record(cfg, steps, warmup, cps, engine, split, probe):
    """Step and history-launch times of one resident workload, with the
    launch's roofline (HBM bytes, or MFMA FLOPs for wide row groups)."""
    rnd, hist_len, ms_step, ms_chunk = time_resident(cfg, steps, warmup, cps, engine, split)
    kernel = "ss_verify_history" if rnd.split == "balanced" else "ss_verify_chunk"
    hist_b, cand_b = kv_bytes(cfg, hist_len)
    gbs = (hist_b + cand_b) / (ms_step * 1e-3) / 1e9
    alg = launch_bytes(cfg, hist_len, rnd)
    traffic = read_traffic(cfg, rnd.split, rnd.fused, rnd.n_hist_slots) if engine == "auto" else None
    if cfg.rows > 32:
        # wide row groups: the chunk kernel is bound by the matrix cores (the
        # dense peak of the input type)
        flops = chunk_kernel_flops(cfg, hist_len)
        tflops = flops / (ms_chunk * 1e-3) / 1e12
        peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                "traffic": None if traffic is None else int(traffic), "kernel": kernel,
                "ms_per_launch": round(ms_chunk, 4), "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": alg,
                "hbm_GBps_algorithmic": round(alg / (ms_chunk * 1e-3) / 1e9, 2)}
        cycles = read_profile_value(cfg, "grbm_active_cycles_per_xcd", rnd.split, rnd.fused, rnd.n_hist_slots)
        if cycles:
            # The launch's active GPU cycles (rocprofv3 GRBM_GUI_ACTIVE, per
            # XCD) over its duration here is the clock it sustained; the dense
            # peak scales with the clock (2.5 PFLOP/s at 2.4 GHz).
            clock = cycles / (ms_chunk * 1e-3) / 1e9
            roof["sustained_clock_GHz"] = round(clock, 3)
            roof["frac_at_sustained_clock"] = round(tflops / (peak * clock / 2.4), 4)
    else:
        achieved = alg / (ms_chunk * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if traffic is None else int(traffic),
                "kernel": kernel, "ms_per_launch": round(ms_chunk, 4), "algorithmic_bytes_per_launch": alg}
        if probe:
            roof["frac_of_read_probe"] = round(achieved / max(probe["one_per_cu_GBps"], probe["eight_per_cu_GBps"]),
                                               4)
    rec = {
        "config": {"workload": workload_desc(cfg), "seed": cfg.seed, "inputs_sha256": rnd.inputs_sha256,
                   "batch": cfg.batch, "history_tokens": cfg.hist_len,
                   "history_tokens_total": int(hist_b // (2 * cfg.n_kv_heads * cfg.head_dim * cfg.elem_bytes)),
                   "queries": cfg.n_queries,
                   "split": rnd.split, "history_slots": rnd.n_hist_slots, "fused_candidates": rnd.fused,
                   "chunks_per_slot": rnd.cps if rnd.split == "chunks" else None, "engine": engine},
        "ms_per_step": round(ms_step, 4),
        "effective_KV_GBps": round(gbs, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "query_tokens_per_s": round(cfg.batch * cfg.n_queries / (ms_step * 1e-3), 1),
        "roofline": roof,
    }
    del rnd
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=[k for k in wl.CONFIGS if not wl.CONFIGS[k].streamed])
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the c2 and c4 sub-records of the default run")
    ap.add_argument("--chunks-per-slot", type=int, default=0,
                    help="chunks merged per state slot (0: automatic, about two work-groups per compute unit)")
    ap.add_argument("--split", default=rounds.BENCH_RESIDENT["split"], choices=["balanced", "chunks"],
                    help="history cut: ss_verify_history's balanced cut, or ss_verify_chunk over fixed chunks")
    ap.add_argument("--engine", default="auto", choices=list(rounds.ENGINES),
                    help="chunk-kernel engine (ss_problem_t.engine)")
    ap.add_argument("--queries", type=int, default=0, help="override the workload's queries per request")
    ap.add_argument("--head-dim", type=int, default=0, choices=[0, 64, 128], help="override the workload's head_dim")
    ap.add_argument("--dtype", default="", choices=["", "bf16", "f32"], help="override the workload's input type")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streamed", action="store_true", help="skip the streamed, tiered and layered legs")
    ap.add_argument("--no-sparse", action="store_true", help="skip the block-statistics / sparse leg")
    ap.add_argument("--streamed-only", action="store_true",
                    help="run only the streamed leg (c5_streamed) and print its record (for traces of that path)")
    ap.add_argument("--mfma-probe-only", action="store_true",
                    help="only the matrix-core reference (ss_mfma_probe) on N(0,1) bf16 operands")
    ap.add_argument("--hold", type=float, default=0.0,
                    help="run the workload's resident round (with --mfma-probe-only: the probe) back to back for "
                         "this many seconds and print its time per call; for power and clock readings taken "
                         "meanwhile by another tool")
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection pass: one plain elementwise copy of 1 GiB (the calibration kernel "
                         "of known size), then one step of the workload; prints nothing else")
    ap.add_argument("--counters-settle", type=float, default=0.0,
                    help="with --counters: seconds of the same steps before the last one (steady-state dispatches)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the verification path runs on a "
              f"single MI355X; sharding across GPUs is described, not built).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.hold > 0:
        hold(args.workload, args.hold, args.mfma_probe_only)
        return
    if args.mfma_probe_only:
        print(json.dumps({"mfma_probe": mfma_probe()}), flush=True)
        return
    if args.streamed_only:
        print(json.dumps({"streamed": time_streamed(wl.CONFIGS["c5_streamed"])}), flush=True)
        return
    cfg = wl.CONFIGS[args.workload]
    if args.queries:
        cfg = cfg.with_(n_queries=args.queries, name=f"{cfg.name}_q{args.queries}")
    if args.head_dim and args.head_dim != cfg.head_dim:
        cfg = cfg.with_(head_dim=args.head_dim, name=f"{cfg.name}_d{args.head_dim}")
    if args.dtype and args.dtype != cfg.dtype:
        cfg = cfg.with_(dtype=args.dtype, name=f"{cfg.name}_{args.dtype}")
    overridden = cfg.name != args.workload
    cps = args.chunks_per_slot or "auto"
    if args.counters:
        counters_pass(cfg, cps, args.engine, args.split, args.counters_settle)
        return
    # the read reference first, while the device is in the state the timed
    # steps start from (after seconds of streaming it reads measurably slower)
    probe = read_probe()
    head = resident_record(cfg, args.steps, args.warmup, cps, args.engine, args.split, probe)
    out = {
        "metric": "verification-attn effective KV GB/s (% of HBM peak) + verified query-tokens/s",
        "value": head["effective_KV_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded N(0,1), {cfg.dtype})",
        "config": head["config"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "query_tokens_per_s": head["query_tokens_per_s"],
        "roofline": head["roofline"],
        "hbm_read_probe": probe,
    }
    # the other resident workloads of the round, each in its own launch
    # configuration: the uniform HBM-bound layer and the MFMA-bound tree
    if not args.no_extra_workloads and args.workload == DEFAULT_WORKLOAD and not overridden:
        for key, name in (("c2", "c2_qwen3_8b"), ("c4", "c4_tree_72b")):
            rec = resident_record(wl.CONFIGS[name], args.steps, args.warmup, "auto", args.engine, args.split, probe)
            out[key] = {k: rec[k] for k in ("config", "ms_per_step", "effective_KV_GBps", "pct_hbm_peak",
                                             "query_tokens_per_s", "roofline")}
            torch.cuda.empty_cache()
        # the matrix-core reference after the timed launches (it heats the chip)
        out["mfma_probe"] = mfma_probe()
        roof = out["c4"]["roofline"]
        roof["frac_of_mfma_probe"] = round(roof["achieved"] / out["mfma_probe"]["TFLOPs"], 4)
    if not args.no_sparse:
        out["sparse"] = time_sparse(wl.CONFIGS["c2_qwen3_8b"])
        torch.cuda.empty_cache()
    if not args.no_streamed:
        out["streamed"] = time_streamed(wl.CONFIGS["c5_streamed"])
        torch.cuda.empty_cache()
        out["tiered"] = time_tiered(wl.CONFIGS["c5_streamed"])
        torch.cuda.empty_cache()
        out["layered"] = time_layered(wl.CONFIGS["c5_streamed"])
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
