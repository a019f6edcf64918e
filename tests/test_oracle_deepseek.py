"""Pins for the oracle's DeepSeek-style pre-tokenizer (CPU only).

The family is three splitters applied one after the other; each re-splits every piece of the one
before it, and unmatched stretches stay pieces (TokTier, arXiv 2607.29678, derivation paragraph on
the DeepSeek family).  The oracle's serial matchers are pinned to things other than themselves:
  * the `regex` engine running the three patterns of tests/family_regex.py stage by stage
    (exhaustively on short strings over a stress alphabet, and on random strings and generated text);
  * the HuggingFace `tokenizers` library's own sequence of isolating split pre-tokenizers on the same
    patterns (its regex engine is Oniguruma, a separate implementation of the composition);
  * hand-worked splits (tests/golden/pretokenize_deepseek_cases.json) and the seams that the stage
    cuts create.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from family_regex import DS_STAGES, regex_split
from workloads import textgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pretokenize_deepseek_cases.json")

# stress alphabet: ASCII letters, a Latin letter with accent, an ideograph, a kana prolonged sound
# mark (Lm) and middle dot (Po) from the kana block, a kana combining mark, an unassigned kana-block
# code point, an ideograph just past the stage-2 range, a digit, SP, TAB, CR, LF, NBSP, ASCII
# punctuation and symbol, a non-ASCII quotation mark, a combining acute, a control
ALPHA_DS = ["a", "Z", "é", "中", "ー", "・", "゙", "぀", "龦", "1", " ", "\t",
            "\r", "\n", ".", "$", "«", "́", "\x00", "\xa0"]
# wider alphabet for random strings: + apostrophe, an Arabic-Indic digit, an emoji, a zero-width
# space (format character), kana-block symbol and dash, hiragana, more letters, the euro sign, NEL,
# the ideographic space, a CJK closing bracket outside the stage-2 range
ALPHA_DS_WIDE = ALPHA_DS + ["'", "٣", "\U0001F600", "​", "゛", "゠", "あ", "B", "x",
                            "€", "\x85", "　", "」", "9", "-", "_"]


def _batch_vs(strings, split):
    enc = [s.encode("utf-8") for s in strings]
    offs = np.zeros(len(enc) + 1, dtype=np.uint64)
    offs[1:] = np.cumsum([len(e) for e in enc])
    starts = oracle.pretokenize("deepseek", b"".join(enc), offs)
    bad = []
    for i, s in enumerate(strings):
        exp, b = [], int(offs[i])
        for piece in split(s):
            exp.append(b)
            b += len(piece.encode("utf-8"))
        lo, hi = np.searchsorted(starts, offs[i]), np.searchsorted(starts, offs[i + 1])
        if starts[lo:hi].tolist() != exp:
            bad.append(s)
    return bad


def _regex(s):
    return regex_split("deepseek", s)


def test_golden_cases():
    doc = json.load(open(GOLDEN, encoding="utf-8"))
    assert len(doc["cases"]) >= 15
    for case in doc["cases"]:
        assert oracle.split("deepseek", case["text"]) == case["deepseek"], case
        assert _regex(case["text"]) == case["deepseek"], case


def test_exhaustive_short_strings():
    strings = ["".join(t) for L in range(1, 5) for t in itertools.product(ALPHA_DS, repeat=L)]
    bad = _batch_vs(strings, _regex)
    assert not bad, bad[:10]


def test_random_strings():
    rng = np.random.default_rng(12)
    strings = []
    for _ in range(20000):
        n = int(rng.integers(5, 30))
        strings.append("".join(ALPHA_DS_WIDE[int(i)] for i in rng.integers(0, len(ALPHA_DS_WIDE), n)))
    bad = _batch_vs(strings, _regex)
    assert not bad, bad[:10]


def test_against_hf_split_sequence():
    """The HF tokenizers library composes the three patterns as a sequence of isolating splits."""
    tokenizers = pytest.importorskip("tokenizers")
    pt = tokenizers.pre_tokenizers.Sequence(
        [tokenizers.pre_tokenizers.Split(tokenizers.Regex(p), behavior="isolated") for p in DS_STAGES])

    def hf(s):
        return [x for x, _ in pt.pre_tokenize_str(s)]

    strings = ["".join(t) for L in range(1, 4) for t in itertools.product(ALPHA_DS, repeat=L)]
    text = textgen.kana_mix(31, 40000)
    strings += [text[i:i + 2000] for i in range(0, len(text), 2000)]
    bad = _batch_vs(strings, hf)
    assert not bad, bad[:10]


@pytest.mark.parametrize("gen", ["kana_mix", "multilingual", "agent_transcript", "english_code"])
def test_generated_text(gen):
    text = getattr(textgen, gen)(78, 60000)
    chunks = [text[i:i + 3000] for i in range(0, len(text), 3000)]
    assert not _batch_vs(chunks, _regex)


def test_adversarial_slices():
    text = textgen.adversarial(5)
    cuts = [0, 100_000, 200_000, 300_001, 400_002, 500_003, 600_005, 700_006, 800_007, 900_008,
            1_200_000, 1_900_008, 2_300_000, 2_400_008]
    assert not _batch_vs([text[max(0, c - 700):c + 700] for c in cuts], _regex)


def test_pieces_concatenate_and_docs_independent():
    texts = [textgen.kana_mix(9 + i, 2000 + 37 * i) for i in range(6)] + ["", " ", "\n", "x", "1"]
    data, offs = textgen.to_batch(texts)
    starts = oracle.pretokenize("deepseek", data, offs)
    assert starts[0] == 0 and starts[-1] == data.size
    assert np.all(np.diff(starts.astype(np.int64)) > 0)
    for i, t in enumerate(texts):
        alone = oracle.pretokenize("deepseek", t.encode("utf-8"))
        lo, hi = np.searchsorted(starts, offs[i]), np.searchsorted(starts, offs[i + 1])
        assert (starts[lo:hi] - offs[i]).tolist() == alone[:-1].tolist()


# (A, B): the split of A||B differs from split(A)||split(B) ...
SEAMS_DIFFER = [("12", "34"), ("x ", "y"), (".", "abc"), ("x.", "\n"), ("あ", "い")]
# ... and cuts that the stages force: these splits concatenate
SEAMS_SAME = [("abc", "123"), ("x ", "中"), ("中", "x"), ("123", "4"), ("ab", "\x00")]


def test_stage_seams():
    for a, b in SEAMS_DIFFER:
        assert oracle.split("deepseek", a + b) != oracle.split("deepseek", a) + oracle.split("deepseek", b), (a, b)
    for a, b in SEAMS_SAME:
        assert oracle.split("deepseek", a + b) == oracle.split("deepseek", a) + oracle.split("deepseek", b), (a, b)
