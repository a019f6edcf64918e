"""Pins of the oracle's added-token pass and ignore_merges rule.

Independent pin: the HuggingFace `tokenizers` library (a byte-level BPE model with the family's
pattern as a Split pre-tokenizer, special tokens matched leftmost-longest, and its own
ignore_merges switch), on ASCII text where its regex engine and ours agree on every class.  Plus
hand-worked cases (overlapping literals, literals at document ends, a piece whose merge order and
whole-piece lookup differ) and the invariant that decoding returns the text.
"""
import numpy as np
import pytest

import oracle
from family_regex import PATTERNS
from workloads import textgen


def _byte_chars():
    """The byte-to-character map of byte-level BPE: printable Latin-1 bytes stand for themselves,
    the other 68 bytes for the code points 256, 257, ... in byte order."""
    keep = set(range(ord("!"), ord("~") + 1)) | set(range(0xA1, 0xAD)) | set(range(0xAE, 0x100))
    out, extra = {}, 0
    for b in range(256):
        if b in keep:
            out[b] = chr(b)
        else:
            out[b] = chr(256 + extra)
            extra += 1
    return out


def _hf(family, merges, literals=(), ignore_merges=False):
    from tokenizers import AddedToken, Regex, Tokenizer, pre_tokenizers
    from tokenizers.models import BPE
    bc = _byte_chars()
    tb = oracle.Merges(merges).token_bytes()
    strs = ["".join(bc[x] for x in t) for t in tb]
    assert len(set(strs)) == len(strs), "HF needs one ID per byte string"
    vocab = {s: i for i, s in enumerate(strs)}
    mlist = [(strs[a], strs[b]) for a, b in np.asarray(merges).tolist()]
    tok = Tokenizer(BPE(vocab=vocab, merges=mlist, ignore_merges=ignore_merges))
    tok.pre_tokenizer = pre_tokenizers.Sequence([
        pre_tokenizers.Split(Regex(PATTERNS[family]), behavior="isolated"),
        pre_tokenizers.ByteLevel(add_prefix_space=False, use_regex=False)])
    if literals:
        tok.add_special_tokens([AddedToken(l.decode(), special=True, normalized=False) for l in literals])
    return tok


def _unique_merges(seed, n=300):
    """A random rank-consistent merge list over a few ASCII letters whose tokens all have distinct
    byte strings (and tokens whose own string does not encode to themselves)."""
    rng = np.random.default_rng(seed)
    alpha = [ord(c) for c in "abcde "]
    ids, seen, merges = list(alpha), set(), []
    tb = {i: bytes([i]) for i in range(256)}
    strings = set(tb.values())
    while len(merges) < n:
        a, b = ids[int(rng.integers(0, len(ids)))], ids[int(rng.integers(0, len(ids)))]
        s = tb[a] + tb[b]
        if (a, b) in seen or s in strings or len(s) > 12:
            continue
        seen.add((a, b))
        t = 256 + len(merges)
        merges.append((a, b))
        ids.append(t)
        tb[t] = s
        strings.add(s)
    return np.array(merges, dtype=np.uint32)


def _text(seed, n, merges):
    """Fragments of ASCII text and whole token strings (so that pieces which are vocabulary entries,
    some of them not their own BPE, occur often)."""
    rng = np.random.default_rng(seed)
    words = [t.decode() for t in oracle.Merges(merges).token_bytes()[256:] if t.strip() and b" " not in t]
    parts = ["abc", "ab", "cde", " ", "  ", "\n", "e", "d", "12", "3456", "!", "?.", "'s", " a", "eab", "\t"]
    out = []
    for i in rng.integers(0, len(parts) + 8, n):
        out.append(parts[int(i)] if i < len(parts) else " " + words[int(rng.integers(0, len(words)))])
    return "".join(out)


LITS = [b"<|endoftext|>", b"<|end|>", b"abca", b"cab", b"ab!", b"<|end", b"abc"]


@pytest.mark.parametrize("family", ["gpt2", "cl100k", "o200k"])
@pytest.mark.parametrize("ignore_merges", [False, True])
@pytest.mark.parametrize("with_lits", [False, True])
def test_matches_hf_tokenizers(family, ignore_merges, with_lits):
    merges = _unique_merges(3)
    lits = LITS if with_lits else []
    hf = _hf(family, merges, lits, ignore_merges)
    added = [(l, hf.token_to_id(l.decode())) for l in lits]
    changed = 0
    for seed in range(12):
        t = _text(seed, 60 + 40 * seed, merges)
        if with_lits:
            rng = np.random.default_rng(100 + seed)
            for _ in range(4):
                i = int(rng.integers(0, len(t) + 1))
                t = t[:i] + LITS[int(rng.integers(0, len(LITS)))].decode() + t[i:]
        exp = hf.encode(t, add_special_tokens=False).ids
        got, oo = oracle.encode_batch_ex(family, merges, t.encode(), added=added, ignore_merges=ignore_merges)
        assert got.tolist() == exp, (seed, t)
        changed += ignore_merges and got.tolist() != oracle.encode_batch_ex(family, merges, t.encode(), added=added)[0].tolist()
    # the texts hold pieces on which the whole-piece rule and the merge loop disagree
    assert changed >= 3 or not ignore_merges


def test_ignore_merges_hand_worked():
    # ranks: b+c -> "bc" (256), a+b -> "ab" (257), ab+c -> "abc" (258).  BPE of "abc" merges b+c
    # first and stops at [a, bc]; with ignore_merges "abc" is a vocabulary entry and becomes 258.
    m = np.array([(98, 99), (97, 98), (257, 99)], dtype=np.uint32)
    ids, _ = oracle.encode_batch_ex("gpt2", m, b"abc", ignore_merges=False)
    assert ids.tolist() == [97, 256]
    ids, _ = oracle.encode_batch_ex("gpt2", m, b"abc", ignore_merges=True)
    assert ids.tolist() == [258]
    # "abcc" is no entry: the merge loop runs as usual
    ids, _ = oracle.encode_batch_ex("gpt2", m, b"abcc", ignore_merges=True)
    assert ids.tolist() == [97, 256, 99]
    # two tokens with the bytes "abc" (258 and 259): the smaller ID wins
    m2 = np.array([(98, 99), (97, 98), (257, 99), (97, 256)], dtype=np.uint32)
    ids, _ = oracle.encode_batch_ex("gpt2", m2, b"abc", ignore_merges=True)
    assert ids.tolist() == [258]


def test_added_matches_hand_worked():
    lits = [b"ab", b"abc", b"bcd", b"d"]
    # leftmost first: at 0 the longest is "abc"; "bcd" starts inside it and is skipped; then "d"
    assert oracle.added_matches(b"abcd", None, lits) == [(0, 1), (3, 3)]
    # a literal crossing a document end is no match; the shorter one that fits is
    assert oracle.added_matches(b"abcd", [0, 2, 4], lits) == [(0, 0), (3, 3)]
    assert oracle.added_matches(b"xbcdx", None, lits) == [(1, 2)]
    assert oracle.added_matches(b"", None, lits) == []
    assert oracle.added_matches(b"dddd", [0, 1, 1, 4], lits) == [(0, 3), (1, 3), (2, 3), (3, 3)]
    # overlapping copies of one literal: non-overlapping, leftmost first
    assert oracle.added_matches(b"aaaaa", None, [b"aa"]) == [(0, 0), (2, 0)]


def test_added_tokens_split_documents():
    merges, fam = textgen.load_vocab("v2")
    lit = [(b"<|endoftext|>", 900001), (b"<|im_start|>", 900002)]
    t = b"hello world<|endoftext|> again<|im_start|><|im_start|>x"
    ids, oo = oracle.encode_batch_ex(fam, merges, t, added=lit)
    # the same as encoding the text segments as documents and putting the IDs between
    segs = [b"hello world", b" again", b"", b"x"]
    data = b"".join(segs)
    offs = np.concatenate([[0], np.cumsum([len(x) for x in segs])])
    e, eo = oracle.encode_batch(fam, merges, data, offs)
    parts = [e[eo[i]:eo[i + 1]].tolist() for i in range(4)]
    assert ids.tolist() == parts[0] + [900001] + parts[1] + [900002] + parts[2] + [900002] + parts[3]
    assert oo.tolist() == [0, ids.size]


@pytest.mark.parametrize("voc", ["v1", "v2", "v3"])
def test_decode_round_trip(voc):
    merges, fam = textgen.load_vocab(voc)
    tb = oracle.Merges(merges).token_bytes()
    lits = [b"<|endoftext|>", b"```", b"\n\n\n", b"the"]
    added = [(l, 1 << 22 | k) for k, l in enumerate(lits)]
    texts = [textgen.agent_transcript(11 + i, 3000).replace("\n\n", "\n<|endoftext|>\n") for i in range(3)] + ["", "the"]
    data, offs = textgen.to_batch(texts)
    for im in (False, True):
        ids, oo = oracle.encode_batch_ex(fam, merges, data, offs, added=added, ignore_merges=im)
        back = {a: l for l, a in added}
        for d in range(len(texts)):
            dec = b"".join(back[i] if i in back else tb[i] for i in ids[oo[d]:oo[d + 1]].tolist())
            assert dec == texts[d].encode()
        if not im:
            # without literals in the text and without ignore_merges, it is F itself
            e, eo = oracle.encode_batch(fam, merges, data, offs)
            plain, po = oracle.encode_batch_ex(fam, merges, data, offs)
            assert np.array_equal(e, plain) and np.array_equal(eo, po)
