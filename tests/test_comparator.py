"""The parity comparator must catch planted faults (CPU only).

TokTier (arXiv 2607.29678, shadow-verifier paragraph) validates its comparator by planting faults:
ID substitution, deletion, duplication, adjacent swap and a same-length tail re-split -- the silent
shape of a history-dependent tokenizer bug.  Every planted fault must be flagged.
"""
import numpy as np
import pytest

import oracle
from parity import Mismatch, compare_ids, compare_starts
from workloads import textgen


@pytest.fixture(scope="module")
def reference():
    merges = oracle.train("cl100k", textgen.agent_transcript(31, 200_000).encode(), 3000)
    data, offs = textgen.to_batch([textgen.agent_transcript(32 + i, 3000) for i in range(5)])
    ids, oo = oracle.encode_batch("cl100k", merges, data, offs)
    return merges, data, offs, ids, oo


def _faults(ids, oo, rng):
    out = []
    k = int(rng.integers(5, ids.size - 5))
    sub = ids.copy(); sub[k] = (sub[k] + 1) % 3000
    out.append(("substitution", sub, oo))
    dele = np.delete(ids, k); oo2 = oo.copy(); oo2[np.searchsorted(oo, k, side="right"):] -= 1
    out.append(("deletion", dele, oo2))
    dup = np.insert(ids, k, ids[k]); oo3 = oo.copy(); oo3[np.searchsorted(oo, k, side="right"):] += 1
    out.append(("duplication", dup, oo3))
    j = k
    while ids[j] == ids[j + 1]:
        j += 1
    sw = ids.copy(); sw[j], sw[j + 1] = sw[j + 1], sw[j]
    out.append(("adjacent swap", sw, oo))
    # same-length tail re-split: the last two tokens of a document replaced by two different ones
    # of the same total count
    rs = ids.copy(); e = int(oo[1]); rs[e - 2], rs[e - 1] = rs[e - 1] ^ 1, rs[e - 2] ^ 2
    out.append(("same-length resplit", rs, oo))
    return out


def test_clean_passes(reference):
    _, _, _, ids, oo = reference
    compare_ids(ids, oo, ids.copy(), oo.copy())


def test_planted_faults_caught(reference):
    _, _, _, ids, oo = reference
    rng = np.random.default_rng(0)
    caught = 0
    for trial in range(40):
        for name, bad_ids, bad_oo in _faults(ids, oo, rng):
            with pytest.raises(Mismatch):
                compare_ids(ids, oo, bad_ids, bad_oo)
            caught += 1
    assert caught == 200


def test_split_comparator_catches_moved_boundary(reference):
    _, data, offs, _, _ = reference
    st = oracle.pretokenize("cl100k", data, offs)
    compare_starts(st, st.copy())
    moved = st.copy(); moved[10] += 1
    with pytest.raises(Mismatch):
        compare_starts(st, moved, data)
    merged = np.delete(st, 10)
    with pytest.raises(Mismatch):
        compare_starts(st, merged, data)
