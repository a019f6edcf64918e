"""Pins for the oracle's pre-tokenizer G (CPU only).

G is pinned to things other than itself: the `regex` backtracking engine running the family patterns
(a special case that reduces to a library routine), hand-worked splits (tests/golden), and the
invariants the paper relies on (pieces concatenate to the input; documents are independent; the
pre-tokenizer seam tok(A)||tok(B) != tok(A||B)).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from family_regex import regex_split
from workloads import textgen

FAMS = ("gpt2", "cl100k", "o200k")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pretokenize_cases.json")

# stress alphabet: cased letters, contraction letters, ASCII and Arabic-Indic digits, a vulgar
# fraction (No), SP, TAB, CR, LF, NBSP, apostrophe, period, CJK (Lo), a combining mark, a titlecase
# letter (Lt) and a modifier letter (Lm)
ALPHA4 = ["a", "B", "s", "t", "r", "e", "1", "٣", " ", "\t", "\r", "\n", "\xa0", "'", ".",
          "中", "́", "ǅ", "ʰ", "\xbd"]
# wider alphabet for random strings: + S, T, L, l, v, d, m, M, D, NEL, VT, FF, U+3000, an
# information separator (not \s for `regex`), a spacing mark (Mc), an emoji, slash, digit 9
ALPHA_WIDE = ALPHA4 + ["S", "T", "L", "l", "v", "d", "m", "M", "D", "\x85", "\x0b", "\x0c", "　",
                       "\x1c", "ः", "\U0001F600", "/", "9", "E", "R", "V"]


def _batch_vs_regex(family, strings):
    enc = [s.encode("utf-8") for s in strings]
    offs = np.zeros(len(enc) + 1, dtype=np.uint64)
    offs[1:] = np.cumsum([len(e) for e in enc])
    starts = oracle.pretokenize(family, b"".join(enc), offs)
    bad = []
    for i, s in enumerate(strings):
        exp, b = [], int(offs[i])
        for piece in regex_split(family, s):
            exp.append(b)
            b += len(piece.encode("utf-8"))
        lo, hi = np.searchsorted(starts, offs[i]), np.searchsorted(starts, offs[i + 1])
        if starts[lo:hi].tolist() != exp:
            bad.append(s)
    return bad


def test_golden_cases():
    doc = json.load(open(GOLDEN, encoding="utf-8"))
    for case in doc["cases"]:
        for f in FAMS:
            assert oracle.split(f, case["text"]) == case[f], (f, case["text"])
            assert regex_split(f, case["text"]) == case[f], (f, case["text"])


@pytest.mark.parametrize("family", FAMS)
def test_exhaustive_short_strings(family):
    strings = ["".join(t) for L in range(1, 5) for t in itertools.product(ALPHA4, repeat=L)]
    bad = _batch_vs_regex(family, strings)
    assert not bad, bad[:10]


@pytest.mark.parametrize("family", FAMS)
def test_random_strings(family):
    rng = np.random.default_rng(11)
    strings = []
    for _ in range(20000):
        n = int(rng.integers(5, 25))
        strings.append("".join(ALPHA_WIDE[int(i)] for i in rng.integers(0, len(ALPHA_WIDE), n)))
    bad = _batch_vs_regex(family, strings)
    assert not bad, bad[:10]


@pytest.mark.parametrize("family,gen", [("gpt2", "english_code"), ("cl100k", "agent_transcript"),
                                        ("o200k", "multilingual"), ("cl100k", "multilingual")])
def test_generated_text(family, gen):
    text = getattr(textgen, gen)(77, 60000)
    chunks = [text[i:i + 3000] for i in range(0, len(text), 3000)]
    assert not _batch_vs_regex(family, chunks)


@pytest.mark.parametrize("family", FAMS)
def test_adversarial_slices(family):
    text = textgen.adversarial(5)
    # a slice across every segment boundary of the adversarial request
    cuts = [0, 100_000, 200_000, 300_001, 400_002, 500_003, 600_005, 700_006, 800_007, 900_008,
            1_200_000, 1_900_008, 2_300_000, 2_400_008]
    chunks = [text[max(0, c - 700):c + 700] for c in cuts]
    assert not _batch_vs_regex(family, chunks)


@pytest.mark.parametrize("family", FAMS)
def test_pieces_concatenate_and_docs_independent(family):
    texts = [textgen.multilingual(9 + i, 2000 + 37 * i) for i in range(6)] + ["", " ", "\n", "x"]
    data, offs = textgen.to_batch(texts)
    starts = oracle.pretokenize(family, data, offs)
    assert starts[0] == 0 and starts[-1] == data.size
    assert np.all(np.diff(starts.astype(np.int64)) > 0)
    for i, t in enumerate(texts):
        alone = oracle.pretokenize(family, t.encode("utf-8"))
        lo, hi = np.searchsorted(starts, offs[i]), np.searchsorted(starts, offs[i + 1])
        assert (starts[lo:hi] - offs[i]).tolist() == alone[:-1].tolist()


SEAMS = [
    # (A, B, families whose split of A||B differs from split(A)||split(B))
    ("12", "34", FAMS),                           # one digit run; grouping counts from its start
    ("x\n", "\ny", ("cl100k", "o200k")),         # \s*[\r\n]+ runs to the last newline
    (".\n", "\n", FAMS),                          # newline absorption / run-end lookahead
    (" pipe", "line", FAMS),                       # the paper's Figure 4 seam
    ("a ", "b", FAMS),                             # whitespace lookahead: the space joins "b"
    ("a ", " b", ()),                              # no seam effect
]


@pytest.mark.parametrize("family", FAMS)
def test_seams(family):
    for a, b, differ in SEAMS:
        joint = oracle.split(family, a + b)
        sep = oracle.split(family, a) + oracle.split(family, b)
        assert (joint != sep) == (family in differ), (family, a, b, joint, sep)


@pytest.mark.parametrize("bad", [b"\x80", b"a\xc0\xafb", b"\xe0\x80\x80", b"\xed\xa0\x80", b"\xf4\x90\x80\x80",
                                 b"\xf8\x88\x80\x80\x80", b"\xe4\xb8", b"\xc3", b"abc\xff", b"\xc2\x41"])
def test_invalid_utf8_rejected(bad):
    with pytest.raises(oracle.OracleError) as e:
        oracle.pretokenize("cl100k", bad)
    assert e.value.code == -1


def test_valid_edge_code_points():
    for s in ["\U0010FFFF", "", "￿", "\U00010000", "߿", "ࠀ", "\x7f\x00"]:
        assert "".join(oracle.split("o200k", s)) == s


def test_doc_split_inside_a_char_is_invalid():
    data = "中".encode()
    with pytest.raises(oracle.OracleError):
        oracle.pretokenize("cl100k", data, [0, 1, 3])


def test_empty_and_bad_offsets():
    assert oracle.pretokenize("gpt2", b"", [0, 0, 0]).tolist() == [0]
    with pytest.raises(oracle.OracleError):
        oracle.pretokenize("gpt2", b"abc", [0, 2, 1, 3])
