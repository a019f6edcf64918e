"""Oracle character classes, probed out of the `regex` engine (TEST INFRASTRUCTURE ONLY).

The TokTier paper (arXiv 2607.29678, exactness section on the Unicode-table skew) states that
character-class tables must be probed directly out of the reference regex engine rather than taken
from library data, because stdlib tables lagged the engine's Unicode version. The oracle follows that:
every code point is classified by asking `regex` which property class matches it.

Codes (one byte per code point, index = code point):
    1 LU  letter, uppercase or titlecase  (\\p{Lu} | \\p{Lt})
    2 LL  letter, lowercase               (\\p{Ll})
    3 LO  letter, modifier or other       (\\p{Lm} | \\p{Lo})
    4 N   number                          (\\p{N})
    5 W   whitespace                      (what `\\s` matches)
    6 M   mark                            (\\p{M}; "other" in the 4-class split, a letter for o200k)
    7 O   everything else: controls, format characters, private use, unassigned, surrogates
    8 PS  punctuation or symbol           (\\p{P} | \\p{S}; "other" in the 4-class split)

This module is only imported by tests, by the smoke check and by the benchmark's CPU-baseline leg.
"""
import hashlib

import numpy as np

MAXCP = 0x110000
LU, LL, LO, N, W, M, O, PS = 1, 2, 3, 4, 5, 6, 7, 8

_PROBES = (
    (LU, r"[\p{Lu}\p{Lt}]"),
    (LL, r"\p{Ll}"),
    (LO, r"[\p{Lm}\p{Lo}]"),
    (N, r"\p{N}"),
    (W, r"\s"),
    (M, r"\p{M}"),
    (PS, r"[\p{P}\p{S}]"),
)

_cache = None


def class_table() -> np.ndarray:
    """Return the frozen uint8[0x110000] class table (computed once per process)."""
    global _cache
    if _cache is not None:
        return _cache
    import regex

    every = "".join(map(chr, range(MAXCP)))
    table = np.full(MAXCP, O, dtype=np.uint8)
    seen = np.zeros(MAXCP, dtype=bool)
    for code, pat in _PROBES:
        idx = np.fromiter((m.start() for m in regex.finditer(pat, every)), dtype=np.int64)
        if seen[idx].any():
            raise RuntimeError(f"class probe {pat} overlaps an earlier class")
        seen[idx] = True
        table[idx] = code
    _cache = table
    return table


def table_sha256() -> str:
    return hashlib.sha256(class_table().tobytes()).hexdigest()
