"""Bit-exact comparators between the oracle and the GPU path (used by the tests)."""
import numpy as np


class Mismatch(AssertionError):
    pass


def compare_starts(expected, got, data=None):
    """Piece boundaries (uint64 start offsets followed by the batch end)."""
    e = np.asarray(expected, dtype=np.uint64)
    g = np.asarray(got, dtype=np.uint64)
    if e.shape == g.shape and np.array_equal(e, g):
        return
    k = int(np.argmax(e[: min(e.size, g.size)] != g[: min(e.size, g.size)])) if min(e.size, g.size) else 0
    if min(e.size, g.size) and e[k] == g[k]:
        k = min(e.size, g.size)
    ctx = ""
    if data is not None and k < e.size:
        b = int(e[k])
        ctx = f" near bytes {bytes(np.asarray(data)[max(0, b - 24):b + 24])!r}"
    raise Mismatch(f"piece starts differ at piece {k}: expected {e[k] if k < e.size else None}, "
                   f"got {g[k] if k < g.size else None} (expected {e.size - 1} pieces, got {g.size - 1}){ctx}")


def compare_ids(exp_ids, exp_offsets, got_ids, got_offsets):
    """Token IDs and per-document token offsets, bit for bit."""
    ei = np.asarray(exp_ids, dtype=np.uint32)
    gi = np.asarray(got_ids, dtype=np.uint32)
    eo = np.asarray(exp_offsets, dtype=np.uint64)
    go = np.asarray(got_offsets, dtype=np.uint64)
    if not np.array_equal(eo, go):
        d = int(np.argmax(eo != go)) if eo.shape == go.shape else -1
        raise Mismatch(f"document offsets differ (first at doc {d}): expected {eo[:8]}..., got {go[:8]}...")
    if ei.shape != gi.shape:
        raise Mismatch(f"token count differs: expected {ei.size}, got {gi.size}")
    if not np.array_equal(ei, gi):
        k = int(np.argmax(ei != gi))
        doc = int(np.searchsorted(eo, k, side="right")) - 1
        raise Mismatch(f"token {k} (doc {doc}) differs: expected {ei[max(0, k - 4):k + 4].tolist()}, "
                       f"got {gi[max(0, k - 4):k + 4].tolist()}")
