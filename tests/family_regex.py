"""The rule families written as `regex` patterns, used only to pin the oracle's matchers.

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

# DeepSeek style: three splitters applied one after the other (paper, derivation paragraph on the
# DeepSeek family).  Each re-splits every piece of the one before it, and the text between two
# matches of a splitter stays a piece of its own.  Our wording: digit groups; runs of CJK
# ideographs (U+4E00-U+9FA5) and kana (U+3040-U+30FF); then the body alternatives.
DS_STAGES = [
    r"\p{N}{1,3}",
    r"[\u4E00-\u9FA5\u3040-\u30FF]+",
    "|".join([
        r"[!-/:-@\[-`{-~][A-Za-z]+",
        r"[^\r\n\p{L}\p{P}\p{S}]?[\p{L}\p{M}]+",
        r" ?[\p{P}\p{S}]+[\r\n]*",
        r"\s*[\r\n]+",
        r"\s+(?!\S)",
        r"\s+",
    ]),
]
DS_COMPILED = [regex.compile(p) for p in DS_STAGES]


def split_isolated(pattern, text):
    """One splitter: its matches and the unmatched stretches between them, in order."""
    out, last = [], 0
    for m in pattern.finditer(text):
        if m.start() > last:
            out.append(text[last:m.start()])
        out.append(m.group())
        last = m.end()
    if last < len(text):
        out.append(text[last:])
    return out


def regex_split(family, text):
    if family == "deepseek":
        pieces = [text] if text else []
        for pat in DS_COMPILED:
            pieces = [q for p in pieces for q in split_isolated(pat, p)]
        return pieces
    pieces = COMPILED[family].findall(text)
    assert "".join(pieces) == text, "pattern left a gap"
    return pieces
