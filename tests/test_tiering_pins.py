"""Pins for the commit-aware tiering oracle (CPU only).

SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
Serving"), section 4.1: the target KV cache of a request is split at
0 <= H <= C <= L into Sealed History [0, H) on the host, Active Tail [H, C)
and Speculative Frontier [C, L) on the GPU (Eq. 4); the next migration ends
at E = max(H, g * floor(max(0, C - T) / g)) (Eq. 5); after verification the
committed prefix becomes C' in [C, L] and [C', L) is reclaimed, which never
touches [0, H).

The oracle is checked against hand-worked Eq. (5) cases (a cited fixture),
against a brute-force reading of Eq. (5) (the largest block boundary that
leaves at least T committed tokens on the GPU), and against the invariants
of random round trajectories; planted mistakes must each fail a pin.
"""

import os

import numpy as np
import pytest

from oracle import tiering

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiering_eq5_cases.txt")


def load_cases():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(tuple(int(x) for x in line.split()))
    return rows


def brute_force_end(h, c, tail, gran):
    """Walk the block boundaries above H one by one and keep the last one
    that still leaves at least `tail` committed tokens on the GPU."""
    e = h
    b = h + gran
    while b + tail <= c:
        e = b
        b += gran
    return e


def test_eq5_hand_worked_cases():
    cases = load_cases()
    assert len(cases) >= 10
    for h, c, t, g, e in cases:
        assert tiering.migration_end(h, c, t, g) == e, (h, c, t, g, e)


def test_eq5_matches_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(3000):
        g = int(rng.choice([1, 64, 128, 256, 4096]))
        t = int(rng.choice([0, 1, 100, 512, 2048]))
        h = g * int(rng.integers(0, 40))
        c = h + int(rng.integers(0, 20 * max(g, 1) + t))
        assert tiering.migration_end(h, c, t, g) == brute_force_end(h, c, t, g), (h, c, t, g)


def simulate(rng, steps, tail, gran, q_max, fn=None):
    """A request through rounds: q candidates are appended, a of them are
    accepted, the rest are reclaimed, then the tail migrates per Eq. (5).
    Returns the trajectory of (H, C, L, C', reclaimed, E)."""
    fn = fn or tiering.migration_end
    h, c = 0, int(rng.integers(0, 3 * tail + 2 * gran + 1))
    out = []
    for _ in range(steps):
        q = int(rng.integers(1, q_max + 1))
        l = c + q
        tiering.regions(h, c, l)
        a = int(rng.integers(0, q + 1))
        h2, c_new, l_new, reclaimed = tiering.commit(h, c, l, c + a)
        assert h2 == h and l_new == c_new
        e = fn(h, c_new, tail, gran)
        out.append((h, c, l, c_new, reclaimed, e))
        h, c = e, c_new
    return out


@pytest.mark.parametrize("seed", range(6))
def test_trajectory_invariants(seed):
    rng = np.random.default_rng(seed)
    tail = int(rng.choice([0, 128, 512]))
    gran = int(rng.choice([64, 128, 256]))
    for h, c, l, c_new, (r0, r1), e in simulate(rng, 400, tail, gran, 9):
        assert 0 <= h <= c <= c_new <= l
        # rollback stays on the GPU: the reclaimed suffix misses the host history
        assert (r0, r1) == (c_new, l) and not tiering.overlaps((r0, r1), (0, h))
        assert e >= h and e % gran == 0 and e <= max(c_new, h)
        if e > h:
            assert c_new - e >= tail                 # the tail keeps at least T tokens
        assert c_new - e < tail + gran or c_new < tail   # and never grows past T + g


def test_region_and_commit_checks():
    assert tiering.regions(0, 0, 0) == ((0, 0), (0, 0), (0, 0))
    assert tiering.regions(2, 5, 9) == ((0, 2), (2, 5), (5, 9))
    for bad in ((3, 2, 9), (0, 5, 4), (-1, 0, 0)):
        with pytest.raises(ValueError):
            tiering.regions(*bad)
    with pytest.raises(ValueError):
        tiering.commit(0, 10, 14, 9)                 # C' < C: a committed token rejected
    with pytest.raises(ValueError):
        tiering.commit(0, 10, 14, 15)                # C' > L
    assert tiering.commit(4, 10, 14, 12) == (4, 12, 12, (12, 14))
    with pytest.raises(ValueError):
        tiering.migration_end(0, 10, 0, 0)
    assert not tiering.overlaps((5, 9), (0, 5)) and tiering.overlaps((4, 9), (0, 5))


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _ceil_blocks(h, c, t, g):
    return max(h, g * (-(-max(0, c - t) // g)))


def _no_floor_at_h(h, c, t, g):
    return g * (max(0, c - t) // g)


def _ignores_tail(h, c, t, g):
    return max(h, g * (c // g))


@pytest.mark.parametrize("mutant", [_ceil_blocks, _no_floor_at_h, _ignores_tail])
def test_pins_catch_planted_mistakes(mutant):
    failed = False
    for h, c, t, g, e in load_cases():
        if mutant(h, c, t, g) != e:
            failed = True
    rng = np.random.default_rng(3)
    try:
        for hh, cc, ll, cn, (r0, r1), ee in simulate(rng, 300, 512, 256, 9, fn=mutant):
            if ee < hh or (ee > hh and cn - ee < 512):
                failed = True
                break
    except ValueError:
        failed = True
    assert failed

