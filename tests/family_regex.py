"""The three rule families written as `regex` patterns, used only to pin the oracle's matchers.

These are this project's own wording of the GPT-2-, cl100k- and o200k-style pre-tokenizer patterns
that the TokTier paper evaluates (arXiv 2607.29678, pre-tokenization paragraph: a leftmost-first
alternation regex with backtracking).  Readings taken where the paper is silent:
  * contractions are ASCII-only; the cl100k and o200k families accept either case ([sS] ...), the
    GPT-2 family lowercase only;
  * the o200k "other" alternative absorbs trailing CR/LF only;
  * digits are grouped 1-3 code points, greedy from the run start.
`regex` is a backtracking engine, so matching these patterns with findall is a special case of the
pre-tokenizer that reduces to a library routine.
"""
import regex

_C_LOWER = r"'s|'t|'re|'ve|'m|'ll|'d"
_C_ANY = r"'[sS]|'[tT]|'[rR][eE]|'[vV][eE]|'[mM]|'[lL][lL]|'[dD]"
_A = r"[\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}]"
_B = r"[\p{Ll}\p{Lm}\p{Lo}\p{M}]"
_X = r"[^\r\n\p{L}\p{N}]"

PATTERNS = {
    "gpt2": "|".join([
        _C_LOWER,
        r" ?\p{L}+",
        r" ?\p{N}+",
        r" ?[^\s\p{L}\p{N}]+",
        r"\s+(?!\S)",
        r"\s+",
    ]),
    "cl100k": "|".join([
        _C_ANY,
        _X + r"?\p{L}+",
        r"\p{N}{1,3}",
        r" ?[^\s\p{L}\p{N}]+[\r\n]*",
        r"\s*[\r\n]+",
        r"\s+(?!\S)",
        r"\s+",
    ]),
    "o200k": "|".join([
        _X + "?" + _A + "*" + _B + "+(?:" + _C_ANY + ")?",
        _X + "?" + _A + "+" + _B + "*(?:" + _C_ANY + ")?",
        r"\p{N}{1,3}",
        r" ?[^\s\p{L}\p{N}]+[\r\n]*",
        r"\s*[\r\n]+",
        r"\s+(?!\S)",
        r"\s+",
    ]),
}

COMPILED = {k: regex.compile(v) for k, v in PATTERNS.items()}


def regex_split(family, text):
    pieces = COMPILED[family].findall(text)
    assert "".join(pieces) == text, "pattern left a gap"
    return pieces
