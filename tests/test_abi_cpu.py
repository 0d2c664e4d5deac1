"""CPU-only checks of the C-ABI library: it loads, exports every call the
header declares, rejects bad arguments before touching a device, and its
host-side integer rules (tree mask, chunk-to-slot token ranges) agree bit for
bit with the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from long_context_speculative_amd import ssverify as ss
from long_context_speculative_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss_verify.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SS_API\s+[\w\s\*]*?\b(ss_\w+)\s*\(", text)))


def test_library_exports_every_declared_call():
    names = header_functions()
    assert len(names) >= 10
    L = ss.lib()
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(ss.EXPORTED)


def test_missing_library_fails_loudly():
    """Without the built library every call raises; nothing falls back to
    another implementation (checked in a fresh interpreter, whose binding has
    not loaded the library yet)."""
    import subprocess
    import sys
    code = (
        "import sys\n"
        "from long_context_speculative_amd import ssverify as ss\n"
        "ss.LIB_PATH = '/nonexistent/libssverify.so'\n"
        "for call in (ss.ss_abi_version, lambda: ss.ss_tier_migration_end(0, 0, 512, 128)):\n"
        "    try:\n"
        "        call()\n"
        "    except RuntimeError as e:\n"
        "        assert 'missing' in str(e), e\n"
        "    else:\n"
        "        sys.exit('a call returned without the library')\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


def test_abi_version_matches_header():
    m = re.search(r"#define\s+SS_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert ss.ss_abi_version() == int(m.group(1))


def _problem(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_queries=6, dtype=ss.SS_BF16, scale=0.088,
                engine=ss.SS_ENGINE_AUTO)
    base.update(kw)
    return ss.Problem(**base)


def test_state_bytes():
    p = _problem()
    assert ss.ss_state_bytes(p, 3) == 3 * 2 * 6 * 8 * (128 + 2) * 4
    with pytest.raises(ss.SSError) as e:
        ss.ss_state_bytes(_problem(head_dim=96), 1)
    assert e.value.code == ss.SS_ERR_UNSUPPORTED


class _Fake:
    """Something with a data_ptr(), for calls that must fail validation
    before any device work (the pointers are never dereferenced)."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _view(max_len=64, stride_t=128, k=4096, v=8192):
    return ss.KVView(k, v, 0, 0, stride_t, None, None, max_len)


def _state(n_slots=4):
    st = ss.StateBuffers.__new__(ss.StateBuffers)
    st.struct = ss.State(4096, 8192, 12288, n_slots)
    return st


@pytest.mark.parametrize("case,code", [
    ("null_problem", ss.SS_ERR_INVALID_ARG),
    ("bad_heads", ss.SS_ERR_INVALID_ARG),
    ("head_dim_96", ss.SS_ERR_UNSUPPORTED),
    ("null_q", ss.SS_ERR_INVALID_ARG),
    ("misaligned_k", ss.SS_ERR_INVALID_ARG),
    ("zero_chunk", ss.SS_ERR_INVALID_ARG),
    ("slot_overflow", ss.SS_ERR_INVALID_ARG),
    ("bad_cps", ss.SS_ERR_INVALID_ARG),
    ("bad_stride", ss.SS_ERR_INVALID_ARG),
    ("bad_engine", ss.SS_ERR_INVALID_ARG),
    ("negative_scale", ss.SS_ERR_INVALID_ARG),
])
def test_verify_chunk_rejects(case, code):
    L = ss.lib()
    p = _problem()
    q = 4096
    view = _view()
    st = _state(4)
    args = dict(chunk_len=64, chunk_begin=0, n_chunks=4, cps=1, slot_begin=0)
    if case == "null_problem":
        rc = L.ss_verify_chunk(None, q, ctypes.byref(view), 64, 0, 4, 1, ctypes.byref(st.struct), 0, None)
        assert rc == code
        return
    if case == "bad_heads":
        p = _problem(n_q_heads=7)
    if case == "head_dim_96":
        p = _problem(head_dim=96)
    if case == "null_q":
        q = None
    if case == "misaligned_k":
        view = _view(k=4098)
    if case == "zero_chunk":
        args["chunk_len"] = 0
    if case == "slot_overflow":
        args["slot_begin"] = 1
    if case == "bad_cps":
        args["cps"] = 0
    if case == "bad_stride":
        view = _view(stride_t=100)
    if case == "bad_engine":
        p = _problem(engine=7)
    if case == "negative_scale":
        p = _problem(scale=-0.1)
    rc = L.ss_verify_chunk(ctypes.byref(p), q, ctypes.byref(view), args["chunk_len"], args["chunk_begin"],
                           args["n_chunks"], args["cps"], ctypes.byref(st.struct), args["slot_begin"], None)
    assert rc == code
    assert L.ss_last_error().decode()


def test_candidates_and_stream_reject():
    L = ss.lib()
    p = _problem(n_queries=65)
    rc = L.ss_verify_candidates(ctypes.byref(p), 4096, ctypes.byref(_view(max_len=65)), None, None,
                                ctypes.byref(_state().struct), 0, None)
    assert rc == ss.SS_ERR_UNSUPPORTED
    p = _problem()
    rc = L.ss_verify_candidates(ctypes.byref(p), 4096, ctypes.byref(_view(max_len=5)), None, None,
                                ctypes.byref(_state().struct), 0, None)
    assert rc == ss.SS_ERR_INVALID_ARG          # max_len must equal n_queries
    rc = L.ss_verify_candidates(ctypes.byref(p), 4096, ctypes.byref(_view(max_len=6)), None, None,
                                ctypes.byref(_state(2).struct), 2, None)
    assert rc == ss.SS_ERR_INVALID_ARG          # slot out of range
    # equal copy and compute streams
    rc = L.ss_stream_history(ctypes.byref(p), 4096, 4096, None, 64, 4, 1, 8192, 2, ctypes.byref(_state(4).struct), 0,
                             None, None, 0)
    assert rc == ss.SS_ERR_INVALID_ARG
    rc = L.ss_stream_history(ctypes.byref(p), 4096, 4096, None, 64, 5, 1, 8192, 2, ctypes.byref(_state(4).struct), 0,
                             1, 2, 0)
    assert rc == ss.SS_ERR_INVALID_ARG          # 5 chunks, 4 slots
    rc = L.ss_stream_history(ctypes.byref(p), 4096, 4096, None, 64, 4, 0, 8192, 2, ctypes.byref(_state(4).struct), 0,
                             1, 2, 0)
    assert rc == ss.SS_ERR_INVALID_ARG          # chunks_per_copy 0
    rc = L.ss_stream_history(ctypes.byref(p), 4096, 4096, None, 64, 4, 1, 8192, 2, ctypes.byref(_state(4).struct), 0,
                             1, 2, 16)
    assert rc == ss.SS_ERR_INVALID_ARG          # unknown flag
    rc = L.ss_merge_states(ctypes.byref(p), ctypes.byref(_state().struct), None, None, 4096, None)
    assert rc == ss.SS_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(6))
def test_tree_mask_host_matches_oracle(seed):
    n = [1, 5, 17, 33, 63, 64][seed]
    parents = workloads.draw_tree(seed, 0, n, 8)
    got = ss.ss_tree_mask_host(parents)
    want = [int(x) for x in oracle.mask_to_bits(oracle.tree_mask(parents))]
    assert got == want


def test_tree_mask_host_chain_and_invalid_parents():
    for n in (1, 2, 6, 64):
        assert ss.ss_tree_mask_host([-1] + list(range(n - 1))) == [int(x) for x in
                                                                     oracle.mask_to_bits(oracle.chain_mask(n))]
    # pointers that do not point strictly backwards are read as roots
    assert ss.ss_tree_mask_host([-1, 5, 1, -7, 0]) == [0b1, 0b10, 0b110, 0b1000, 0b10001]


def test_slot_tokens_host_tile_history():
    rng = np.random.default_rng(5)
    for _ in range(40):
        c = int(rng.choice([1, 7, 64, 2048, 4096]))
        n = int(rng.integers(0, min(20000, 60 * c)))
        cps = int(rng.integers(1, 5))
        n_chunks = -(-n // c) if n else 0
        ref = oracle.chunk_list([n], c)
        covered = []
        for s in range(-(-n_chunks // cps) if n_chunks else 0):
            t0, t1 = ss.ss_slot_tokens_host(n, c, 0, n_chunks, cps, s)
            # the slot's range is exactly the union of its chunks in the oracle's list
            mine = [(st, ln) for (_, j, st, ln) in ref if s * cps <= j < (s + 1) * cps]
            assert (t0, t1) == (mine[0][0], mine[-1][0] + mine[-1][1])
            covered.append((t0, t1))
        if covered:
            assert covered[0][0] == 0 and covered[-1][1] == n
            assert all(a[1] == b[0] for a, b in zip(covered, covered[1:]))
    # a chunk beyond the request's length gives an empty range
    assert ss.ss_slot_tokens_host(100, 64, 2, 1, 1, 0) == (100, 100)
    # a sub-range of chunks
    assert ss.ss_slot_tokens_host(1000, 64, 3, 5, 2, 1) == (5 * 64, 7 * 64)
    assert ss.ss_slot_tokens_host(1000, 64, 3, 5, 2, 2) == (7 * 64, 8 * 64)


CHARGE = 512  # line positions the cut charges per stream (kPlanCharge)


def _check_plan(lens, hkv, max_len, n_wg, n_slots):
    """Invariants of the balanced cut of ss_verify_history: every slot of
    every stream is written exactly once; the computed pieces of a stream
    come first and tile [0, len) in order; the rest are empty fills; no
    work-group outside the grid is used; no work-group gets more than
    piece_len (padded) tokens, nor more line positions than piece_len plus
    one charge when the charge of every stream it finishes is counted; the
    ranges are an even share of the line (tokens and charges) plus one
    alignment step unless the slot budget needs more."""
    plan, piece_len = ss.ss_history_plan_host(lens, hkv, max_len, n_wg, n_slots)
    lens_c = np.clip(np.asarray(lens, dtype=np.int64), 0, max_len)
    pad = -(-lens_c // 128) * 128
    total = (int(pad.sum()) + CHARGE * len(lens_c)) * hkv
    assert piece_len % 128 == 0 and piece_len >= 128
    # the cut grows past an even share only to respect the slot budget
    even = -(-total // n_wg)
    cap = -(-int(pad.max(initial=0)) // (n_slots - 1))
    assert piece_len < max(even, cap, 128) + 128
    assert (plan[..., 3] == 1).all(), "a slot written zero or several times"
    load = {}
    charged = {}
    for b, n in enumerate(lens_c):
        for g in range(hkv):
            e = plan[b, g]
            computed = [k for k in range(n_slots) if e[k, 1] >= 0]
            assert computed == list(range(len(computed)))
            if n == 0:
                assert not computed
                # the work-group whose range holds the stream's line position
                o = (int(pad[:b].sum()) + CHARGE * b) * hkv + g * CHARGE
                assert (e[:, 0] == min(o // piece_len, n_wg - 1)).all()
                continue
            assert computed, "a non-empty stream without pieces"
            assert e[0, 1] == 0 and e[computed[-1], 2] == n
            for k in computed[1:]:
                assert e[k, 1] == e[k - 1, 2]
            for k in computed:
                wg = int(e[k, 0])
                assert 0 <= wg < n_wg
                # padded extent of the piece inside the work-group's range
                t0, t1 = int(e[k, 1]), int(e[k, 2])
                end = int(pad[b]) if k == computed[-1] else t1
                load[wg] = load.get(wg, 0) + (end - t0)
            # consecutive pieces go to consecutive work-groups
            wgs = [int(e[k, 0]) for k in computed]
            assert wgs == list(range(wgs[0], wgs[0] + len(wgs)))
            charged[wgs[-1]] = charged.get(wgs[-1], 0) + CHARGE
    assert all(v <= piece_len for v in load.values())
    assert all(v + charged.get(w, 0) <= piece_len + CHARGE for w, v in load.items())
    return plan, piece_len


@pytest.mark.parametrize("seed", range(8))
def test_history_plan_host_random(seed):
    rng = np.random.default_rng(100 + seed)
    batch = int(rng.choice([1, 3, 32, 70, 200]))
    hkv = int(rng.choice([1, 2, 8]))
    max_len = int(rng.choice([1, 127, 1000, 65536]))
    lens = rng.integers(0, max_len + 1, size=batch)
    lens[rng.random(batch) < 0.2] = 0
    n_wg = int(rng.choice([1, 7, 64, 512]))
    n_slots = int(rng.choice([2, 3, 5, 16]))
    _check_plan(lens, hkv, max_len, n_wg, n_slots)


def test_history_plan_host_cases():
    # uniform lengths: equal ranges, about one stream per pair of work-groups
    plan, L = _check_plan([32768] * 16, 8, 32768, 256, 4)
    # (32768 + 512) * 128 / 256 positions per range; the last stream's tokens end in range 255
    assert L == 16640 and int(plan[..., 0].max()) == (127 * (32768 + CHARGE) + 32768 - 1) // L
    # the ragged long-history shape: every work-group gets an even share
    lens = workloads.draw_lengths(workloads.CONFIGS["c3_internlm25_7b_ragged"]).astype(np.int64)
    plan, L = _check_plan(lens, 8, int(max(lens)), 512, 6)
    assert L == -(-(-(-((-(-lens // 128) * 128).sum() + CHARGE * len(lens)) * 8 // 512)) // 128) * 128
    # a range holding more stream starts gets fewer tokens: 64 streams of
    # 1000 tokens (1024 padded, 1536 with the charge) on 22 work-groups
    plan, L = _check_plan([1000] * 64, 1, 1000, 22, 3)
    assert L == -(-(-(-64 * (1024 + CHARGE) // 22)) // 128) * 128 == 4480
    # a slot budget too small for an even cut widens the ranges
    plan, L = _check_plan([100000], 1, 100000, 512, 2)
    assert L >= 100096 // 1 and (plan[0, 0, :, 1] >= 0).sum() <= 2
    # only empty requests: every slot filled empty, each stream by the
    # work-group whose range holds its charge
    plan, L = _check_plan([0, 0, 0], 4, 10, 8, 3)
    assert (plan[..., 1] == -1).all() and int(plan[..., 0].max()) > 0
    # lengths past max_len are clamped, negative ones read as empty
    _check_plan([5000, -3, 10**6], 2, 4096, 16, 4)
    with pytest.raises(ss.SSError):
        ss.ss_history_plan_host([10], 1, 10, 4, 1)


def test_verify_history_rejects():
    L = ss.lib()
    p = _problem()
    view = _view(max_len=1000)
    def call(problem, q, n_slots, n_state, slot_begin, cand=None, stats=None):
        return L.ss_verify_history(ctypes.byref(problem), q, ctypes.byref(view),
                                   None if cand is None else ctypes.byref(cand), None, None,
                                   None if stats is None else ctypes.byref(stats), n_slots,
                                   ctypes.byref(_state(n_state).struct), slot_begin, None)
    assert call(p, 4096, 0, 4, 0) == ss.SS_ERR_INVALID_ARG             # n_slots < 1
    assert call(p, 4096, 4, 4, 1) == ss.SS_ERR_INVALID_ARG             # slots [1, 5) of 4
    assert call(p, None, 2, 4, 0) == ss.SS_ERR_INVALID_ARG             # no q
    assert call(_problem(head_dim=96), 4096, 2, 4, 0) == ss.SS_ERR_UNSUPPORTED
    # candidate views are checked like ss_verify_candidates'
    assert call(p, 4096, 2, 4, 0, cand=_view(max_len=5)) == ss.SS_ERR_INVALID_ARG    # max_len != n_queries
    assert call(p, 4096, 2, 4, 0, cand=_view(max_len=6, k=4098)) == ss.SS_ERR_INVALID_ARG
    assert call(_problem(n_queries=65), 4096, 2, 4, 0, cand=_view(max_len=65)) == ss.SS_ERR_UNSUPPORTED
    # outside the narrow MFMA kernel the candidates need a slot of their own
    assert call(_problem(engine=ss.SS_ENGINE_VALU), 4096, 1, 4, 0, cand=_view(max_len=6)) == ss.SS_ERR_INVALID_ARG
    # block statistics: narrow MFMA kernel only, block_len a positive multiple of 128, a buffer
    assert call(_problem(engine=ss.SS_ENGINE_VALU), 4096, 2, 4, 0,
                stats=ss.BlockStats(4096, 128, 8)) == ss.SS_ERR_UNSUPPORTED
    assert call(p, 4096, 2, 4, 0, stats=ss.BlockStats(4096, 100, 8)) == ss.SS_ERR_INVALID_ARG
    assert call(p, 4096, 2, 4, 0, stats=ss.BlockStats(4096, 0, 8)) == ss.SS_ERR_INVALID_ARG
    assert call(p, 4096, 2, 4, 0, stats=ss.BlockStats(4096, 256, 0)) == ss.SS_ERR_INVALID_ARG
    assert call(p, 4096, 2, 4, 0, stats=ss.BlockStats(None, 256, 8)) == ss.SS_ERR_INVALID_ARG


def test_gathered_chunks_per_slot_rejects():
    L = ss.lib()
    view = _view(max_len=1000)
    def call(problem, chunk_len, n_sel, cps, n_state):
        return L.ss_verify_chunk_gathered(ctypes.byref(problem), 4096, ctypes.byref(view), chunk_len, 4096, n_sel,
                                          cps, ctypes.byref(_state(n_state).struct), 0, None)
    assert call(_problem(), 128, 8, 0, 8) == ss.SS_ERR_INVALID_ARG          # chunks_per_slot < 1
    assert call(_problem(), 128, 8, 4, 1) == ss.SS_ERR_INVALID_ARG          # 2 slots needed
    assert call(_problem(), 100, 8, 4, 2) == ss.SS_ERR_INVALID_ARG          # chunk_len % 32
    assert call(_problem(engine=ss.SS_ENGINE_VALU), 128, 8, 4, 2) == ss.SS_ERR_UNSUPPORTED
    assert call(_problem(), 128, 130, 65, 2) == ss.SS_ERR_UNSUPPORTED      # more than 64 per slot
    assert L.ss_verify_chunk_gathered(ctypes.byref(_problem()), 4096, ctypes.byref(view), 128, None, 8, 4,
                                      ctypes.byref(_state(2).struct), 0, None) == ss.SS_ERR_INVALID_ARG


def test_block_stats_bytes_and_rejects():
    p = _problem()
    # four wave quarters x rows x blocks x (m, l) floats
    rows = p.batch * p.n_queries * p.n_q_heads
    assert ss.ss_block_stats_bytes(p, 8) == 4 * rows * 8 * 2 * 4
    with pytest.raises(ss.SSError):
        ss.ss_block_stats_bytes(p, 0)
    L = ss.lib()
    st = ss.BlockStats(4096, 256, 8)
    def imp(stats, max_len=1000, lse=4096, out=4096):
        return L.ss_block_importance_stats(ctypes.byref(p), None if stats is None else ctypes.byref(stats), None,
                                           max_len, lse, out, None)
    assert imp(None) == ss.SS_ERR_INVALID_ARG
    assert imp(st, lse=None) == ss.SS_ERR_INVALID_ARG
    assert imp(st, out=None) == ss.SS_ERR_INVALID_ARG
    assert imp(ss.BlockStats(4096, 256, 0)) == ss.SS_ERR_INVALID_ARG
    assert imp(ss.BlockStats(4096, 100, 8)) == ss.SS_ERR_INVALID_ARG       # block_len not a multiple of 128
    assert imp(st, max_len=-1) == ss.SS_ERR_INVALID_ARG


def test_tier_migration_end_matches_oracle():
    """The library's Eq. (5) against the oracle's, bit for bit, and against
    the hand-worked cases."""
    from oracle import tiering
    rng = np.random.default_rng(11)
    for _ in range(2000):
        g = int(rng.choice([1, 128, 256, 4096]))
        t = int(rng.choice([0, 512, 3000]))
        h = g * int(rng.integers(0, 50))
        c = h + int(rng.integers(0, 30 * g + t))
        assert ss.ss_tier_migration_end(h, c, t, g) == tiering.migration_end(h, c, t, g)
    path = os.path.join(ROOT, "tests", "golden", "tiering_eq5_cases.txt")
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if line:
            h, c, t, g, e = (int(x) for x in line)
            assert ss.ss_tier_migration_end(h, c, t, g) == e
    for bad in ((5, 4, 0, 1), (-1, 4, 0, 1), (0, 4, 0, 0), (0, 4, -1, 1)):
        with pytest.raises(ss.SSError):
            ss.ss_tier_migration_end(*bad)


def test_tier_copies_reject():
    L = ss.lib()
    p = _problem(batch=2)
    tail = ss.KVView(4096, 8192, 2 * 1024 * 128, 1024 * 128, 128, None, None, 1024)
    rows = lambda *v: (ctypes.c_int64 * 2)(*v)
    host = 65536
    ok = L.ss_tier_migrate(ctypes.byref(p), ctypes.byref(tail), rows(100, 100), rows(100, 300), rows(100, 300),
                           host, 512, 4, None)
    assert ok == ss.SS_OK                       # empty and in-range: nothing enqueued, nothing rejected
    # a range that leaves the tail view, one before the tail's first row, one past the host store
    assert L.ss_tier_migrate(ctypes.byref(p), ctypes.byref(tail), rows(0, 0), rows(0, 0), rows(1025, 0), host, 4096,
                             4, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_tier_migrate(ctypes.byref(p), ctypes.byref(tail), rows(50, 0), rows(40, 0), rows(60, 0), host, 512,
                             4, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_tier_migrate(ctypes.byref(p), ctypes.byref(tail), rows(0, 0), rows(0, 0), rows(0, 2049), host, 512,
                             4, None) == ss.SS_ERR_INVALID_ARG
    # views must be addressable from the host with contiguous rows
    bad = ss.KVView(4096, 8192, 2 * 1024 * 128, 1024 * 128, 256, None, None, 1024)
    assert L.ss_tier_migrate(ctypes.byref(p), ctypes.byref(bad), rows(0, 0), rows(0, 0), rows(1, 1), host, 512, 4,
                             None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_kv_copy_rows(ctypes.byref(p), ctypes.byref(tail), rows(0, 0), ctypes.byref(tail), rows(1000, 0),
                             rows(30, 0), None) == ss.SS_ERR_INVALID_ARG      # past the destination rows
    assert L.ss_kv_copy_rows(ctypes.byref(p), ctypes.byref(tail), rows(0, 0), ctypes.byref(tail), rows(0, 0),
                             rows(-1, 0), None) == ss.SS_ERR_INVALID_ARG


def test_probes_reject():
    L = ss.lib()
    # read probe: NULL buffers, misalignment, no bytes, no work-groups
    assert L.ss_read_probe(None, 4096, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_read_probe(4096, 4096, 1, None, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_read_probe(4100, 4096, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_read_probe(4096, 8, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_read_probe(4096, 4096, 0, 4096, None) == ss.SS_ERR_INVALID_ARG
    # matrix-core probe: a wave needs a window of 8192 bf16 operands
    assert L.ss_mfma_probe(None, 8192, 1, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_mfma_probe(4096, 8192, 1, 1, None, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_mfma_probe(4104, 8192, 1, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_mfma_probe(4096, 8191, 1, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_mfma_probe(4096, 8192, 0, 1, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert L.ss_mfma_probe(4096, 8192, 1, 0, 4096, None) == ss.SS_ERR_INVALID_ARG
    assert "8192" in L.ss_last_error().decode()


def test_input_digest_follows_the_seed():
    """The seeded inputs are a function of the config alone: the same seed
    gives the same bytes (digest), another seed other bytes; ragged lengths
    and tree parents enter the digest."""
    for cfg in (workloads.CONFIGS["c1_tiny_f32"],
                workloads.CONFIGS["c3_internlm25_7b_ragged"].with_(batch=3, hist_len=700, ragged_lo=1, chunk_len=128),
                workloads.CONFIGS["c4_tree_72b"].with_(batch=2, hist_len=300, chunk_len=128)):
        a = workloads.input_digest(workloads.make_inputs(cfg))
        assert a == workloads.input_digest(workloads.make_inputs(cfg))
        assert a != workloads.input_digest(workloads.make_inputs(cfg.with_(seed=cfg.seed + 1)))
        assert len(a) == 64


def test_auto_history_slots_keep_the_even_cut():
    """The resident round's slot count for ragged lengths on the narrow
    kernels is the least that keeps the balanced cut at an even share of the
    line: with it, the plan's tokens per work-group are the even share
    (rounded up to 128) and every slot is written once; with one slot fewer
    the cut's cap would lengthen the ranges."""
    from long_context_speculative_amd import rounds
    base = workloads.CONFIGS["c3_internlm25_7b_ragged"]
    rng = np.random.default_rng(5)
    for _ in range(200):
        b, hkv, mx = int(rng.integers(1, 80)), int(rng.integers(1, 9)), int(rng.integers(1, 70000))
        lens = rng.integers(0, mx + 1, size=b).astype(np.int32)
        if rng.random() < 0.2:
            lens[:] = 0
            lens[0] = mx
        cfg = base.with_(batch=b, n_kv_heads=hkv, n_q_heads=4 * hkv, hist_len=mx, ragged_lo=1)
        n_wg = int(rng.choice([64, 128, 256, 304]))
        slots = rounds.auto_history_slots(cfg, lens, n_wg)
        if rounds.one_piece_per_stream(int(lens.max()), b * hkv, n_wg) and lens.any():
            assert slots == 1
            continue
        total = sum(-(-int(n) // 128) * 128 + CHARGE for n in lens) * hkv
        even = max(128, -(-(-(-total // n_wg)) // 128) * 128)
        plan, piece = ss.ss_history_plan_host(lens, hkv, mx, n_wg, slots)
        assert (plan[..., 3] == 1).all()
        if total:
            assert piece == even, (b, hkv, mx, n_wg, slots)
        if slots > 2:
            assert ss.ss_history_plan_host(lens, hkv, mx, n_wg, slots - 1)[1] > even


def test_short_ragged_histories_take_one_piece_per_stream():
    """The slot rule for ragged histories on the narrow MFMA kernel: one slot
    (a work-group per stream) when the longest history is at most 2048 tokens
    with at least three streams per four compute units; the balanced cut
    otherwise, and always on the VALU engine."""
    from long_context_speculative_amd import rounds
    base = workloads.CONFIGS["c3_internlm25_7b_ragged"]  # 8 KV heads, 20 rows per KV head
    cus = 256
    cases = [(32, 2048, 1), (32, 2049, None), (32, 512, 1), (24, 2048, 1), (23, 2048, None), (24, 3072, None),
             (16, 2048, None), (128, 2048, 1), (128, 4096, None)]
    for batch, mx, want in cases:
        cfg = base.with_(batch=batch, hist_len=mx, ragged_lo=1)
        lens = np.full(batch, mx // 2, dtype=np.int32)
        lens[0] = mx
        assert rounds.one_piece_per_stream(mx, batch * 8, cus) == (want == 1), (batch, mx)
        slots = rounds.auto_history_slots(cfg, lens, cus)
        if want == 1:
            assert slots == 1, (batch, mx)
        else:
            assert slots >= 2, (batch, mx)
    # the VALU engine keeps the balanced count
    assert rounds.auto_history_slots(base.with_(batch=32, hist_len=2048), np.full(32, 2048), cus, "valu") >= 2


def test_view_token_stride_limit():
    """A token stride above 2^24 elements is refused before anything is
    enqueued (keys inside a tile are addressed by 32-bit offsets)."""
    L = ss.lib()
    p = _problem()
    st = ctypes.byref(_state(4).struct)
    big = ss.KVView(4096, 8192, 0, 0, (1 << 24) + 8, None, None, 1024)
    assert L.ss_verify_chunk(ctypes.byref(p), 4096, ctypes.byref(big), 64, 0, 4, 1, st, 0, None) == ss.SS_ERR_UNSUPPORTED
    assert "2^24" in L.ss_last_error().decode()


def _gpu_present() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(_gpu_present(), reason="passes fake device pointers past validation: only where no GPU can "
                                           "run them")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("rows", [(1, 4), (6, 4), (10, 4), (64, 8)])
@pytest.mark.parametrize("engine", ["auto", "mfma", "valu"])
def test_candidate_placement_mirror(dtype, head_dim, rows, engine):
    """The binding's mirror of the library's engine choice
    (rounds.mfma_fuses_candidates: the bf16 MFMA kernels, narrow and
    wide-row, attend the candidate region inside the history launch; the
    fp32 and VALU engines give it a slot of its own) agrees with the library:
    with one slot and a candidate view, ss_verify_history refuses the call
    (SS_ERR_INVALID_ARG, before any device work) exactly when the engine does
    not fold the candidates in; otherwise it passes validation and fails only
    at the device (there is none here: SS_ERR_HIP)."""
    from long_context_speculative_amd import rounds
    q, group = rows
    cfg = workloads.CONFIGS["c2_qwen3_8b"].with_(dtype=dtype, head_dim=head_dim, n_queries=q,
                                                 n_q_heads=2 * group, n_kv_heads=2)
    p = _problem(dtype=ss.SS_F32 if dtype == "f32" else ss.SS_BF16, head_dim=head_dim, n_queries=q,
                 n_q_heads=2 * group, n_kv_heads=2, engine=rounds.ENGINES[engine])
    es = 4 if dtype == "f32" else 2
    stride = 256 // es * ((head_dim * es + 255) // 256)  # a multiple of 16 bytes and >= head_dim
    view = _view(max_len=1000, stride_t=stride)
    cand = _view(max_len=q, stride_t=stride)
    L = ss.lib()
    rc = L.ss_verify_history(ctypes.byref(p), 4096, ctypes.byref(view), ctypes.byref(cand), None, None, None, 1,
                             ctypes.byref(_state(4).struct), 0, None)
    fused = rounds.mfma_fuses_candidates(cfg, engine)
    assert rc == (ss.SS_ERR_HIP if fused else ss.SS_ERR_INVALID_ARG), (rc, L.ss_last_error().decode())
