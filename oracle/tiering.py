"""Plain integer oracle for commit-aware KV tiering.

TEST INFRASTRUCTURE (same rules as the rest of ``oracle/``).

SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
Serving"), section 4.1:

* Eq. (4): a request's target KV cache is split into the Sealed History
  [0, H) (migrated to host memory), the Active Tail [H, C) (committed, on the
  GPU) and the Speculative Frontier [C, L) (unverified candidates, on the
  GPU), with 0 <= H <= C <= L.
* Eq. (5): the end of the next migration is E = max(H, g * floor(max(0, C - T)
  / g)) for tail target T and granularity g; [H, E) migrates when E > H, and H
  becomes E only once that copy has completed.
* After verification the committed prefix becomes C' (C <= C' <= L); the
  rejected suffix [C', L) is reclaimed on the GPU. Because H <= C <= C', the
  reclaimed range never overlaps the host-resident history [0, H).

Every function here is a direct transcription of those definitions with
explicit checks; the pins in the test suite compare them with hand-worked
cases and random trajectories.
"""

from __future__ import annotations


def regions(h: int, c: int, l: int):
    """Eq. (4): (sealed, tail, frontier) as half-open ranges."""
    if not (0 <= h <= c <= l):
        raise ValueError(f"tier boundaries out of order: H={h}, C={c}, L={l}")
    return (0, h), (h, c), (c, l)


def migration_end(h: int, c: int, tail: int, gran: int) -> int:
    """Eq. (5): E = max(H, g * floor(max(0, C - T) / g))."""
    if gran <= 0 or tail < 0:
        raise ValueError("granularity must be positive and the tail target non-negative")
    if not (0 <= h <= c):
        raise ValueError("need 0 <= H <= C")
    return max(h, gran * (max(0, c - tail) // gran))


def commit(h: int, c: int, l: int, c_new: int):
    """End of a round: the committed prefix moves to C' and the frontier
    [C', L) is reclaimed. Returns (H, C', L' = C', reclaimed range)."""
    regions(h, c, l)
    if not (c <= c_new <= l):
        raise ValueError(f"new commit boundary {c_new} outside [{c}, {l}]")
    reclaimed = (c_new, l)
    return h, c_new, c_new, reclaimed


def overlaps(a, b) -> bool:
    """Whether two half-open ranges share a position."""
    return max(a[0], b[0]) < min(a[1], b[1])
