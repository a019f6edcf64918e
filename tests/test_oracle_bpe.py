"""Pins for the oracle's BPE encoder E and trainer T (CPU only).

E is pinned to the exhaustive textbook loop on tiny inputs (brute force), to hand-worked cases, and
to the invariants: decode(encode(x)) = x, no adjacent pair left in the merge table, every ID below
256 + n_merges, and the seam inequality tok(" pipe")||tok("line") != tok(" pipeline") (TokTier,
arXiv 2607.29678, Figure 4).  The round schedule the GPU kernels use -- merge every leftmost
non-overlapping occurrence of the minimum-rank pair at once (paper, GPU BPE paragraph) -- is checked
against the same textbook loop for rank-consistent merge lists.
"""
import collections

import numpy as np
import pytest

import oracle
from workloads import textgen


def random_consistent_merges(rng, n, alphabet):
    """Merge r joins two IDs that exist before it (< 256 + r); no duplicate pairs."""
    ids = list(alphabet)
    seen, merges = set(), []
    while len(merges) < n:
        a = ids[int(rng.integers(0, len(ids)))]
        b = ids[int(rng.integers(0, len(ids)))]
        if (a, b) in seen:
            continue
        seen.add((a, b))
        merges.append((a, b))
        ids.append(255 + len(merges))
    return np.array(merges, dtype=np.uint32)


def round_bpe(merges, piece):
    """The GPU's schedule written plainly: find the minimum rank; merge all of its leftmost
    non-overlapping occurrences left to right; repeat."""
    rank = {(int(a), int(b)): r for r, (a, b) in enumerate(merges)}
    seq = list(piece)
    while True:
        rs = [rank.get((seq[i], seq[i + 1])) for i in range(len(seq) - 1)]
        live = [r for r in rs if r is not None]
        if not live:
            return seq
        r = min(live)
        out, i = [], 0
        while i < len(seq):
            if i + 1 < len(seq) and rs[i] == r:
                out.append(256 + r)
                i += 2
            else:
                out.append(seq[i])
                i += 1
        seq = out


def test_hand_worked():
    a, b, c = ord("a"), ord("b"), ord("c")
    m = np.array([(a, a), (256, 256), (a, b), (258, c)], dtype=np.uint32)
    enc = lambda s: oracle.bpe_encode(m, s, [0, len(s)])[0].tolist()
    assert enc(b"aaa") == [256, a]            # leftmost of the overlapping (a, a)
    assert enc(b"aaaa") == [257]              # aa + aa
    assert enc(b"aaaaa") == [257, a]
    assert enc(b"abc") == [259]
    assert enc(b"aabc") == [256, b, c]        # (a,a) has the lower rank, so (a,b) never forms
    assert enc(b"") == []


def test_pq_matches_textbook_on_random_lists():
    rng = np.random.default_rng(3)
    for trial in range(300):
        alpha = [97, 98, 99, 100][: int(rng.integers(2, 5))]
        merges = random_consistent_merges(rng, int(rng.integers(1, 40)), alpha)
        pieces = [bytes(int(x) for x in rng.choice(alpha, int(rng.integers(1, 14)))) for _ in range(20)]
        starts = np.concatenate([[0], np.cumsum([len(p) for p in pieces])])
        ids, ntok = oracle.bpe_encode(merges, b"".join(pieces), starts)
        exp = [oracle.textbook_bpe(merges, p) for p in pieces]
        assert ntok.tolist() == [len(e) for e in exp]
        assert ids.tolist() == [x for e in exp for x in e]


def test_round_schedule_equals_textbook_for_consistent_lists():
    rng = np.random.default_rng(4)
    for _ in range(2000):
        alpha = [97, 98, 99][: int(rng.integers(1, 4))]
        merges = random_consistent_merges(rng, int(rng.integers(1, 30)), alpha)
        p = bytes(int(x) for x in rng.choice(alpha, int(rng.integers(1, 16))))
        assert round_bpe(merges, p) == oracle.textbook_bpe(merges, p)


def test_round_schedule_needs_rank_consistency():
    # rank 0 uses ID 257, which rank 1 creates: the schedules diverge, so such lists are rejected
    a, b = 97, 98
    m = np.array([(257, a), (a, b), (b, a)], dtype=np.uint32)   # 256=(257,a) 257=(a,b) 258=(b,a)
    p = b"ababa"
    # serial: (a,b) at 0 -> 257, then (257,a) -> 256 at once, later (b,a) -> 258; the round merges
    # both (a,b) first, so its later (257,a) takes the second 257's right neighbour instead
    assert oracle.textbook_bpe(m, p) == [256, 258]
    assert round_bpe(m, p) == [257, 256]
    diffs = 0
    rng = np.random.default_rng(5)
    for _ in range(3000):
        n = int(rng.integers(2, 8))
        ids = [97, 98]
        mm = []
        for r in range(n):
            mm.append((int(rng.integers(97, 256 + n)) if rng.random() < 0.5 else 97,
                       int(rng.choice([97, 98]))))
        mm = np.array(mm, dtype=np.uint32)
        if len({tuple(x) for x in mm.tolist()}) != n:
            continue
        q = bytes(int(x) for x in rng.choice([97, 98], int(rng.integers(2, 12))))
        if round_bpe(mm, q) != oracle.textbook_bpe(mm, q):
            diffs += 1
    assert diffs > 0


def test_seam_pipeline():
    # merges that build " pipe", "line" and " pipeline" (the paper's Figure 4 example)
    toks = {}
    merges = []

    def mk(a, b):
        ida = toks[a] if len(a) > 1 else a[0]
        idb = toks[b] if len(b) > 1 else b[0]
        merges.append((ida, idb))
        toks[a + b] = 255 + len(merges)

    for a, b in [(b" ", b"p"), (b"i", b"p"), (b" p", b"ip"), (b" pip", b"e"), (b"l", b"i"), (b"n", b"e"),
                 (b"li", b"ne"), (b" pipe", b"line")]:
        mk(a, b)
    m = np.array(merges, dtype=np.uint32)
    for fam in ("gpt2", "cl100k", "o200k"):
        whole = oracle.encode(fam, m, " pipeline")
        parts = oracle.encode(fam, m, " pipe") + oracle.encode(fam, m, "line")
        assert whole == [toks[b" pipeline"]]
        assert parts == [toks[b" pipe"], toks[b"line"]]
        assert whole != parts


def _v1():
    # a small vocabulary trained by the oracle on a seeded corpus
    return oracle.train("gpt2", textgen.english_code(101, 300_000).encode(), 800)


@pytest.mark.parametrize("family,gen", [("gpt2", "english_code"), ("cl100k", "agent_transcript"),
                                        ("o200k", "multilingual")])
def test_invariants_on_trained_vocab(family, gen):
    text = getattr(textgen, gen)(21, 50_000)
    merges = oracle.train(family, getattr(textgen, gen)(22, 200_000).encode(), 1500)
    m = oracle.Merges(merges)
    data = text.encode()
    starts = oracle.pretokenize(family, data)
    ids, ntok = oracle.bpe_encode(m, data, starts)
    assert oracle.decode(m, ids) == data
    assert ids.max() < 256 + m.n_merges
    rank = {(int(a), int(b)) for a, b in merges}
    k = 0
    for n in ntok.tolist():
        seq = ids[k:k + n].tolist()
        assert not any((seq[i], seq[i + 1]) in rank for i in range(n - 1))
        k += n
    # every piece encodes on its own to the same IDs (F = E* o G, pieces independent)
    for p in range(0, len(starts) - 1, 97):
        one, _ = oracle.bpe_encode(m, data[starts[p]:starts[p + 1]], [0, int(starts[p + 1] - starts[p])])
        lo = int(ntok[:p].sum())
        assert one.tolist() == ids[lo:lo + ntok[p]].tolist()


def brute_train(fam, corpus, n, maxb=128):
    st = oracle.pretokenize(fam, corpus)
    cnt = collections.Counter(bytes(corpus[st[k]:st[k + 1]]) for k in range(len(st) - 1))
    words = {w: list(w) for w in cnt}
    tlen = {i: 1 for i in range(256)}
    merges, forbidden = [], set()
    while len(merges) < n:
        pc = collections.Counter()
        for w, c in cnt.items():
            s = words[w]
            for i in range(len(s) - 1):
                pc[(s[i], s[i + 1])] += c
        cands = sorted((-c, a, b) for (a, b), c in pc.items() if c >= 2 and (a, b) not in forbidden)
        pick = None
        for _, a, b in cands:
            if tlen[a] + tlen[b] > maxb:
                forbidden.add((a, b))
                continue
            pick = (a, b)
            break
        if pick is None:
            break
        a, b = pick
        z = 256 + len(merges)
        merges.append(pick)
        tlen[z] = tlen[a] + tlen[b]
        for w in words:
            s, out, i = words[w], [], 0
            while i < len(s):
                if i + 1 < len(s) and s[i] == a and s[i + 1] == b:
                    out.append(z)
                    i += 2
                else:
                    out.append(s[i])
                    i += 1
            words[w] = out
    return np.array(merges, dtype=np.uint32).reshape(-1, 2)


@pytest.mark.parametrize("family", ["gpt2", "cl100k", "o200k"])
@pytest.mark.parametrize("maxb", [128, 4])
def test_trainer_matches_brute_force(family, maxb):
    c = (textgen.multilingual(50, 6000) if family == "o200k" else textgen.english_code(50, 15000)).encode()
    a = oracle.train(family, c, 300, maxb)
    b = brute_train(family, c, 300, maxb)
    assert a.shape == b.shape and (a == b).all()


def test_trainer_deterministic_and_consistent():
    c = textgen.agent_transcript(60, 200_000).encode()
    a = oracle.train("cl100k", c, 2000)
    b = oracle.train("cl100k", c, 2000)
    assert (a == b).all()
    r = np.arange(a.shape[0])
    assert (a[:, 0] < 256 + r).all() and (a[:, 1] < 256 + r).all()
    assert len({tuple(x) for x in a.tolist()}) == a.shape[0]
    tb = oracle.Merges(a).token_bytes()
    assert max(len(t) for t in tb) <= 128


def _seam_safe(rank, tb_index, text, j, lmax):
    """No pair (x, y) of tokens with x's bytes ending at j and y's bytes starting at j has a rank."""
    xs = [t for l in range(1, min(lmax, j) + 1) for t in tb_index.get(text[j - l:j], [])]
    ys = [t for l in range(1, min(lmax, len(text) - j) + 1) for t in tb_index.get(text[j:j + l], [])]
    return not any((x, y) in rank for x in xs for y in ys)


def test_seam_criterion_splits_exactly():
    """The criterion used to cut giant pieces: where no token ending at j and token starting at j form
    a merge pair, BPE of the whole string is BPE of its two sides concatenated.  Checked on random
    strings with dense random merge lists; the unsafe positions must include real counterexamples,
    so the check is not vacuous."""
    rng = np.random.default_rng(77)
    safe_seen = unsafe_broken = 0
    for trial in range(30):
        alpha = [ord(c) for c in "abcd"[: 2 + trial % 3]]
        merges = random_consistent_merges(rng, 60, alpha)
        m = oracle.Merges(merges)
        tb = m.token_bytes()
        index = collections.defaultdict(list)
        for t, b in enumerate(tb):
            index[b].append(t)
        rank = {(int(a), int(b)): r for r, (a, b) in enumerate(merges)}
        lmax = max(len(b) for b in tb)
        text = bytes(int(c) for c in rng.choice(alpha, 120))
        whole = oracle.textbook_bpe(merges, text)
        for j in range(1, len(text)):
            split = oracle.textbook_bpe(merges, text[:j]) + oracle.textbook_bpe(merges, text[j:])
            if _seam_safe(rank, index, text, j, lmax):
                safe_seen += 1
                assert split == whole, (trial, j)
            elif split != whole:
                unsafe_broken += 1
    assert safe_seen > 50 and unsafe_broken > 50
