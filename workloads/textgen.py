"""Seeded synthetic text generators for the tokenization workloads.

This module holds no tokenizer arithmetic: it only produces text.  It is shared by the tests, the
benchmark and the vocabulary-training script.  Everything is driven by numpy's PCG64 generator, so a
(seed, size) pair always yields the same bytes; every workload logs its SHA-256.

The paper (TokTier, arXiv 2607.29678) measures on real agent sessions, Nemotron-CC text and Qwen3
session samples, none of which is available here; these generators stand in for them with the same
shapes: English-like prose mixed with code (EC), agent transcripts with tool calls, listings, diffs,
hashes, timestamps and mixed LF/CRLF line ends (AT), a multilingual mix with CJK, emoji and
combining marks, and an adversarial request built from long single-class runs.
"""
import hashlib
import os

import numpy as np

LEXICON_SEED = 7
LEXICON_SIZE = 50_000

_ONSETS = ["", "", "b", "c", "d", "f", "g", "h", "j", "k", "l", "m", "n", "p", "qu", "r", "s", "t",
           "v", "w", "x", "y", "z", "bl", "br", "ch", "cl", "cr", "dr", "fl", "fr", "gl", "gr", "pl",
           "pr", "sc", "sh", "sk", "sl", "sm", "sn", "sp", "st", "str", "sw", "th", "tr", "tw", "wh"]
_VOWELS = ["a", "e", "i", "o", "u", "a", "e", "i", "o", "y", "ai", "au", "ea", "ee", "ie", "io",
           "oa", "oo", "ou"]
_CODAS = ["", "", "", "", "b", "ck", "d", "ft", "g", "k", "l", "ld", "ll", "lt", "m", "mp", "n",
          "nd", "ng", "nk", "nt", "p", "r", "rd", "rk", "rn", "rt", "s", "sh", "ss", "st", "t", "th",
          "x", "z"]


def sha256(data: bytes) -> str:
    return hashlib.sha256(data).hexdigest()


class Lexicon:
    """50K pseudo-words with a Zipf(1.1) rank distribution."""

    def __init__(self, seed=LEXICON_SEED, size=LEXICON_SIZE):
        rng = np.random.default_rng(seed)
        words, seen = [], set()
        while len(words) < size:
            nsyl = rng.choice([1, 2, 3, 4], size=4096, p=[0.28, 0.42, 0.22, 0.08])
            on = rng.integers(0, len(_ONSETS), size=(4096, 4))
            vo = rng.integers(0, len(_VOWELS), size=(4096, 4))
            co = rng.integers(0, len(_CODAS), size=(4096, 4))
            for i in range(4096):
                w = "".join(_ONSETS[on[i, k]] + _VOWELS[vo[i, k]] + _CODAS[co[i, k]]
                            for k in range(nsyl[i]))
                if w not in seen:
                    seen.add(w)
                    words.append(w)
                    if len(words) == size:
                        break
        # the most frequent ranks get the shortest words, as in natural language
        words.sort(key=lambda w: (len(w), w))
        head = words[:2000]
        rng.shuffle(head)
        self.words = np.array(head + words[2000:], dtype=object)
        ranks = np.arange(1, size + 1, dtype=np.float64)
        cdf = np.cumsum(ranks ** -1.1)
        self.cdf = cdf / cdf[-1]

    def sample(self, rng, n):
        return self.words[np.searchsorted(self.cdf, rng.random(n), side="right")]


_LEX = None


def lexicon():
    global _LEX
    if _LEX is None:
        _LEX = Lexicon()
    return _LEX


_CONTRACTIONS = ["'s", "'t", "'re", "'ve", "'ll", "'d", "'m"]


def _number(rng):
    k = rng.integers(1, 8)
    s = str(rng.integers(10 ** (k - 1), 10 ** k))
    if rng.random() < 0.25:
        s += "." + str(rng.integers(0, 100))
    return s


def _sentence(rng, lex):
    n = int(rng.integers(5, 21))
    ws = list(lex.sample(rng, n))
    r = rng.random(n)
    for i in range(n):
        if r[i] < 0.02:
            ws[i] = ws[i] + _CONTRACTIONS[int(rng.integers(0, len(_CONTRACTIONS)))]
        elif r[i] < 0.05:
            ws[i] = _number(rng)
        elif r[i] < 0.12:
            ws[i] = ws[i] + ","
        elif r[i] < 0.14:
            ws[i] = "(" + ws[i] + ")"
        elif r[i] < 0.16:
            ws[i] = '"' + ws[i] + '"'
    ws[0] = ws[0][:1].upper() + ws[0][1:]
    end = rng.choice([".", ".", ".", ".", "?", "!", ":", ";"])
    return " ".join(ws) + end


def _ident(rng, lex):
    k = rng.random()
    parts = list(lex.sample(rng, int(rng.integers(1, 4))))
    if k < 0.45:
        return "_".join(parts)
    if k < 0.75:
        return parts[0] + "".join(p[:1].upper() + p[1:] for p in parts[1:])
    if k < 0.85:
        return "_".join(parts).upper()
    return "".join(p[:1].upper() + p[1:] for p in parts)


_OPS = [" = ", " += ", " == ", " != ", " -> ", " + ", " - ", " * ", " / ", " < ", " >= ", " && ",
        " || ", ": ", "::"]


def _code_line(rng, lex):
    t = rng.integers(0, 10)
    a, b, c = _ident(rng, lex), _ident(rng, lex), _ident(rng, lex)
    if t == 0:
        return f"def {a}({b}, {c}):"
    if t == 1:
        return f"{a}{_OPS[int(rng.integers(0, len(_OPS)))]}{b}({c}, {_number(rng)})"
    if t == 2:
        return f"if {a} == {_number(rng)}:"
    if t == 3:
        return f"return {a}.{b}({c})"
    if t == 4:
        return "# " + " ".join(lex.sample(rng, int(rng.integers(3, 10))))
    if t == 5:
        return "// " + " ".join(lex.sample(rng, int(rng.integers(3, 10))))
    if t == 6:
        words = " ".join(lex.sample(rng, int(rng.integers(1, 6))))
        return f'{a}.{b}("{words}")'
    if t == 7:
        return f"for {a} in range({_number(rng)}):"
    if t == 8:
        return f"{a}[{b}] = {{'{c}': {_number(rng)}, '{a}': [{b}]}}"
    return f"const {a} = new {b[:1].upper() + b[1:]}({c});"


def _indent(rng, level):
    return "\t" * level if rng.random() < 0.2 else "    " * level


def _code_block(rng, lex):
    lines, level = [], 0
    for _ in range(int(rng.integers(3, 16))):
        line = _code_line(rng, lex)
        lines.append(_indent(rng, level) + line)
        if line.endswith(":"):
            level = min(level + 1, 4)
        elif rng.random() < 0.3:
            level = max(level - 1, 0)
    return "\n".join(lines) + "\n\n"


def _prose_block(rng, lex):
    return " ".join(_sentence(rng, lex) for _ in range(int(rng.integers(2, 7)))) + "\n\n"


def _cut(text, n_chars):
    if len(text) < n_chars:
        raise AssertionError("generator produced too little text")
    return text[:n_chars]


def english_code(seed, n_chars):
    """EC: prose paragraphs (sentence case, punctuation, 2% contractions, 3% numbers) mixed with
    ~30% code lines (4-space or tab indents, snake/camel/UPPER identifiers, operators, literals,
    comments); LF line ends.  Returns exactly n_chars code points (all ASCII)."""
    rng = np.random.default_rng(seed)
    lex = lexicon()
    parts, total = [], 0
    while total < n_chars:
        blk = _code_block(rng, lex) if rng.random() < 0.3 else _prose_block(rng, lex)
        parts.append(blk)
        total += len(blk)
    return _cut("".join(parts), n_chars)


_TOOLS = ["read_file", "write_file", "run_command", "search_code", "list_dir", "apply_patch", "grep"]
_MONTHS = ["Jan", "Feb", "Mar", "Apr", "May", "Jun", "Jul", "Aug", "Sep", "Oct", "Nov", "Dec"]
_EXT = [".py", ".rs", ".ts", ".go", ".cc", ".h", ".md", ".json", ".toml", ".yaml"]


def _path(rng, lex):
    parts = ["_".join(lex.sample(rng, int(rng.integers(1, 3)))) for _ in range(int(rng.integers(1, 4)))]
    return "src/" + "/".join(parts) + _EXT[int(rng.integers(0, len(_EXT)))]


def _hex(rng, n):
    return "".join("0123456789abcdef"[int(x)] for x in rng.integers(0, 16, n))


def _stamp(rng):
    return "2025-%02d-%02dT%02d:%02d:%02dZ" % (int(rng.integers(1, 13)), int(rng.integers(1, 29)),
                                               int(rng.integers(0, 24)), int(rng.integers(0, 60)),
                                               int(rng.integers(0, 60)))


def _at_block(rng, lex):
    t = int(rng.integers(0, 9))
    if t == 0:
        return "User: " + _prose_block(rng, lex)
    if t == 1:
        return "Assistant: " + _prose_block(rng, lex)
    if t == 2:
        name = _TOOLS[int(rng.integers(0, len(_TOOLS)))]
        return ('{"type": "tool_use", "id": "toolu_%s", "name": "%s", "input": {"path": "%s", '
                '"offset": %d, "limit": %d}}\n' % (_hex(rng, 24), name, _path(rng, lex),
                                                   int(rng.integers(0, 2000)), int(rng.integers(1, 400))))
    if t == 3:
        start = int(rng.integers(1, 3000))
        lines = [_code_line(rng, lex) for _ in range(int(rng.integers(3, 20)))]
        return "".join("%6d\t%s%s\n" % (start + i, _indent(rng, int(rng.integers(0, 3))), ln)
                       for i, ln in enumerate(lines)) + "\n"
    if t == 4:
        rows = []
        for _ in range(int(rng.integers(3, 12))):
            rows.append("-rw-r--r--  1 agent staff %8d %s %2d %02d:%02d %s" % (
                int(rng.integers(10, 10 ** 6)), _MONTHS[int(rng.integers(0, 12))],
                int(rng.integers(1, 29)), int(rng.integers(0, 24)), int(rng.integers(0, 60)),
                _path(rng, lex)))
        return "\n".join(rows) + "\n\n"
    if t == 5:
        p = _path(rng, lex)
        a = int(rng.integers(1, 900))
        out = ["diff --git a/%s b/%s" % (p, p), "index %s..%s 100644" % (_hex(rng, 7), _hex(rng, 7)),
               "--- a/" + p, "+++ b/" + p, "@@ -%d,%d +%d,%d @@ def %s():" % (
                   a, int(rng.integers(3, 12)), a, int(rng.integers(3, 12)), _ident(rng, lex))]
        for _ in range(int(rng.integers(3, 14))):
            out.append(rng.choice(["+", "-", " "]) + "    " + _code_line(rng, lex))
        return "\n".join(out) + "\n\n"
    if t == 6:
        return "commit %s\nAuthor: %s <%s@example.com>\nDate:   %s\n\n    %s\n\n" % (
            _hex(rng, 40), _ident(rng, lex), lex.sample(rng, 1)[0], _stamp(rng), _sentence(rng, lex))
    if t == 7:
        frames = []
        for _ in range(int(rng.integers(2, 6))):
            frames.append('  File "/usr/lib/python3.10/%s", line %d, in %s\n    %s' % (
                _path(rng, lex)[4:], int(rng.integers(1, 3000)), _ident(rng, lex), _code_line(rng, lex)))
        return ("Traceback (most recent call last):\n" + "\n".join(frames) +
                "\nValueError: %s\n\n" % _sentence(rng, lex))
    return "[%s] %s\n" % (_stamp(rng), _sentence(rng, lex))


def agent_transcript(seed, n_chars):
    """AT: user/assistant turns, JSON tool calls, line-numbered code excerpts, file listings, diffs,
    commit hashes, timestamps and stack traces; space and tab indentation; each block ends its
    lines with LF (70%) or CRLF (30%).  Returns exactly n_chars code points (all ASCII)."""
    rng = np.random.default_rng(seed)
    lex = lexicon()
    parts, total = [], 0
    while total < n_chars:
        blk = _at_block(rng, lex)
        if rng.random() < 0.3:
            blk = blk.replace("\n", "\r\n")
        parts.append(blk)
        total += len(blk)
    return _cut("".join(parts), n_chars)


_EMOJI = np.concatenate([np.arange(0x1F300, 0x1F650), np.arange(0x1F680, 0x1F700),
                         np.arange(0x1F900, 0x1FA00)])


def multilingual(seed, n_chars):
    """EC text plus, by code-point count, ~10% CJK (runs of 2-8 ideographs, Zipf over 3,000 of
    U+4E00-U+9FFF), ~2% emoji, ~1% combining marks U+0300-U+036F (80% after a letter, 20% after
    punctuation, a space or a digit) and ~1% camelCase / mixed-case words.  Exactly n_chars code
    points."""
    rng = np.random.default_rng(seed)
    base = english_code(seed + 1_000_003, int(n_chars * 0.9) + 64)
    words = base.split(" ")
    nw = len(words)
    ideo = 0x4E00 + rng.permutation(0x9FFF - 0x4E00 + 1)[:3000]
    ranks = np.arange(1, 3001, dtype=np.float64)
    icdf = np.cumsum(ranks ** -1.0)
    icdf /= icdf[-1]
    # CJK runs
    cjk_target = int(0.10 * n_chars)
    got = 0
    while got < cjk_target:
        k = int(rng.integers(2, 9))
        run = "".join(chr(int(ideo[j])) for j in np.searchsorted(icdf, rng.random(k), side="right"))
        i = int(rng.integers(0, nw))
        words[i] = run + words[i] if rng.random() < 0.5 else words[i] + run
        got += k
    # emoji
    for _ in range(int(0.02 * n_chars)):
        i = int(rng.integers(0, nw))
        e = chr(int(_EMOJI[int(rng.integers(0, len(_EMOJI)))]))
        words[i] = words[i] + e if rng.random() < 0.7 else e + words[i]
    # case boosts
    for _ in range(int(0.01 * n_chars / 6)):
        i = int(rng.integers(0, nw))
        w = words[i]
        if w.isalpha() and len(w) > 3:
            j = int(rng.integers(1, len(w)))
            words[i] = w[:j] + w[j:].upper() if rng.random() < 0.5 else w[:j] + w[j:].capitalize()
    # combining marks
    n_marks = int(0.01 * n_chars)
    for _ in range(n_marks):
        i = int(rng.integers(0, nw))
        w = words[i]
        m = chr(0x300 + int(rng.integers(0, 0x70)))
        if rng.random() < 0.8:
            pos = [k for k, ch in enumerate(w) if ch.isalpha()]
            if pos:
                k = pos[int(rng.integers(0, len(pos)))]
                words[i] = w[:k + 1] + m + w[k + 1:]
                continue
        pos = [k for k, ch in enumerate(w) if not ch.isalpha()]
        if pos:
            k = pos[int(rng.integers(0, len(pos)))]
            words[i] = w[:k + 1] + m + w[k + 1:]
        else:
            words[i] = m + w if rng.random() < 0.5 else w + m
    return _cut(" ".join(words), n_chars)


def kana_mix(seed, n_chars):
    """Multilingual text (above) with, by code-point count, ~6% kana runs (hiragana U+3041-U+3096,
    katakana U+30A1-U+30FA, with the prolonged sound mark U+30FC and the middle dot U+30FB inside),
    ~2% CJK punctuation (U+3001, U+3002, U+300C, U+300D, U+FF08, U+FF09), ~1% digits glued to the
    ends of words, and a few kana-block characters that are marks, symbols, dashes or unassigned
    (U+3099, U+309B, U+30A0, U+3040).  Exactly n_chars code points."""
    rng = np.random.default_rng(seed)
    words = multilingual(seed + 2_000_003, int(n_chars * 0.92) + 64).split(" ")
    nw = len(words)
    hira = [chr(c) for c in range(0x3041, 0x3097)]
    kata = [chr(c) for c in range(0x30A1, 0x30FB)]
    punct = ["\u3001", "\u3002", "\u300c", "\u300d", "\uff08", "\uff09"]
    odd = ["\u3099", "\u309b", "\u30a0", "\u3040"]
    got = 0
    while got < int(0.06 * n_chars):
        k = int(rng.integers(2, 10))
        src = hira if rng.random() < 0.5 else kata
        run = [src[int(j)] for j in rng.integers(0, len(src), k)]
        if rng.random() < 0.3:
            run[int(rng.integers(0, k))] = "\u30fc" if rng.random() < 0.6 else "\u30fb"
        i = int(rng.integers(0, nw))
        words[i] = "".join(run) + words[i] if rng.random() < 0.5 else words[i] + "".join(run)
        got += k
    for _ in range(int(0.02 * n_chars)):
        i = int(rng.integers(0, nw))
        c = punct[int(rng.integers(0, len(punct)))]
        words[i] = words[i] + c if rng.random() < 0.7 else c + words[i]
    for _ in range(int(0.01 * n_chars / 2)):
        i = int(rng.integers(0, nw))
        d = str(int(rng.integers(0, 10 ** int(rng.integers(1, 5)))))
        words[i] = words[i] + d if rng.random() < 0.5 else d + words[i]
    for _ in range(max(1, n_chars // 2000)):
        i = int(rng.integers(0, nw))
        words[i] = words[i] + odd[int(rng.integers(0, len(odd)))]
    return _cut(" ".join(words), n_chars)


def _alternating(rng, n):
    letters = "abcdefghijklmnopqrstuvwxyzABCDEFGHIJKLMNOPQRSTUVWXYZé中"
    digits = "0123456789٣"
    spaces = " \t\n\r "
    other = ".,;:!?'\"()[]{}-+*/=<>@#$%^&|~"
    classes = [letters, digits, spaces, other]
    idx = rng.integers(0, 1 << 30, n)
    return "".join(classes[i % 4][int(idx[i]) % len(classes[i % 4])] for i in range(n))


def adversarial(seed, n_chars=4_400_000):
    """The adversarial request: a 200,000-char letter run (100,000 'a' then 100,000 random a-z),
    3 runs of 100,000 random digits, 100,000 spaces, 100,000 tabs, 100,000 CRLF pairs, 100,000
    random {SP, TAB, CR, LF} (each whitespace run followed by a letter), 1,000,000 chars cycling
    letter/number/whitespace/other with random members, 500,000 chars of letters each followed by
    1-3 combining marks, then agent-transcript text up to exactly n_chars code points."""
    rng = np.random.default_rng(seed)
    az = np.frombuffer(b"abcdefghijklmnopqrstuvwxyz", dtype=np.uint8)
    seg = []
    seg.append("a" * 100_000 + az[rng.integers(0, 26, 100_000)].tobytes().decode())
    for _ in range(3):
        seg.append(" " + (np.frombuffer(b"0123456789", np.uint8)[rng.integers(0, 10, 100_000)]).tobytes().decode())
    seg.append("x" + " " * 100_000 + "x")
    seg.append("\t" * 100_000 + "x")
    seg.append("\r\n" * 50_000 + "x")
    seg.append(np.frombuffer(b" \t\r\n", np.uint8)[rng.integers(0, 4, 100_000)].tobytes().decode() + "x")
    seg.append(_alternating(rng, 1_000_000))
    marks = []
    total = 0
    while total < 500_000:
        k = int(rng.integers(1, 4))
        marks.append(chr(int(az[int(rng.integers(0, 26))])) +
                     "".join(chr(0x300 + int(x)) for x in rng.integers(0, 0x70, k)))
        total += 1 + k
    seg.append("".join(marks)[:500_000])
    head = "".join(seg)
    rest = n_chars - len(head)
    if rest < 0:
        raise AssertionError("adversarial segments exceed the request size")
    return head + agent_transcript(seed + 17, rest)


def batch_lengths(seed, n_docs=64, lo=4.0, hi=6.0):
    rng = np.random.default_rng(seed)
    return np.floor(10.0 ** rng.uniform(lo, hi, n_docs)).astype(np.int64)


def to_batch(texts):
    """Concatenate UTF-8 documents: returns (bytes as uint8 array, uint64 offsets[D+1])."""
    enc = [t.encode("utf-8") for t in texts]
    offs = np.zeros(len(enc) + 1, dtype=np.uint64)
    if enc:
        offs[1:] = np.cumsum([len(e) for e in enc])
    data = np.frombuffer(b"".join(enc), dtype=np.uint8).copy() if enc else np.zeros(0, np.uint8)
    return data, offs


# ---------------------------------------------------------------------------------------------
# the five workloads and the four vocabularies

WORKLOADS = {
    # name: (family, vocab, description)
    "c1_ec4k": ("gpt2", "v1", "single 4 KB ASCII English+code request"),
    "c2_at100k": ("cl100k", "v2", "single 100K-char agent transcript"),
    "c3_mix1m": ("o200k", "v3", "single 1M-char multilingual request"),
    "c4_batch64": ("cl100k", "v4", "batch of 64 agent transcripts, lengths log-uniform 1e4-1e6"),
    "c5_adv4m4": ("cl100k", "v2", "adversarial 4.4M-char request"),
}

VOCABS = {
    # name: (family, n_merges, corpus generator, corpus size in chars, corpus seed)
    "v1": ("gpt2", 1_000, "english_code", 1_000_000, 101),
    "v2": ("cl100k", 32_768, "agent_transcript", 32_000_000, 102),
    "v3": ("o200k", 131_072, "multilingual", 64_000_000, 103),
    "v4": ("cl100k", 131_072, "agent_transcript", 64_000_000, 104),
}


def workload(name, scale=1.0):
    """Return (family, vocab name, data uint8[n], offsets uint64[D+1]) for one workload.
    `scale` < 1 shrinks the request sizes (for quick tests); 1.0 is the full size."""
    fam, voc, _ = WORKLOADS[name]
    if name == "c1_ec4k":
        texts = [english_code(1, max(1, int(4096 * scale)))]
    elif name == "c2_at100k":
        texts = [agent_transcript(2, max(1, int(100_000 * scale)))]
    elif name == "c3_mix1m":
        texts = [multilingual(3, max(1, int(1_000_000 * scale)))]
    elif name == "c4_batch64":
        lens = batch_lengths(4)
        texts = [agent_transcript(4_000 + i, max(1, int(l * scale))) for i, l in enumerate(lens)]
    elif name == "c5_adv4m4":
        if scale >= 1.0:
            texts = [adversarial(5)]
        else:
            full = adversarial(5)
            # keep the structure: take an evenly spaced set of slices of the full request
            n = max(1, int(len(full) * scale))
            k = 16
            step = len(full) // k
            texts = ["".join(full[i * step:i * step + n // k] for i in range(k))]
    else:
        raise KeyError(name)
    data, offs = to_batch(texts)
    return fam, voc, data, offs


def corpus(vocab_name):
    fam, n_merges, gen, size, seed = VOCABS[vocab_name]
    text = globals()[gen](seed, size)
    return text.encode("utf-8")


_VOCAB_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "vocabs")


def load_vocab(name):
    """Merge list (uint32[n, 2]) and family of a stored vocabulary (written by oracle/train_vocabs.py)."""
    with np.load(os.path.join(_VOCAB_DIR, name + ".npz"), allow_pickle=False) as z:
        return z["merges"].astype(np.uint32), str(z["family"])
