"""GPU checks of incremental repair (toktier_repair_append) against the oracle, bit for bit.

The repaired records of A || B must equal the oracle's full encoding of A || B (IDs and each token's
source byte offset), whatever the certificate decides: a splice or a full re-encode.  Cached records
of A come from the oracle.  Cases: appends to generated sessions of all four families at many cut
points, multi-step sessions that feed each repaired result back as the next cache, and the
boundary effects the pages name (a piece merged across the seam, digit grouping, whitespace
lookahead, newline absorption, case runs) placed at the seam and stretched past the first windows,
and sessions repaired in place (RepairSession).
"""
import numpy as np
import pytest

import oracle
from workloads import textgen

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module")
def tt():
    import torch
    import exact_bpe_tokenization_amd as tt
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tt.lib()
    return tt


_TOK = {}


class _Orc:
    """The oracle's encoder for one merge list, with its token byte lengths."""

    def __init__(self, merges):
        self.m = oracle.Merges(merges)
        self.len = oracle.token_lengths(merges)


def tok(tt, voc, fam):
    key = (voc, fam)
    if key not in _TOK:
        merges, _ = textgen.load_vocab(voc)
        _TOK[key] = (tt.Tokenizer(merges, fam), _Orc(merges))
    return _TOK[key]


def records(fam, m, raw):
    """The oracle's records of raw as one document: IDs and each token's source byte offset."""
    ids, _ = oracle.encode_batch(fam, m.m, np.frombuffer(raw, np.uint8) if raw else np.zeros(0, np.uint8),
                                 [0, len(raw)])
    spans = np.concatenate([[0], np.cumsum(m.len[ids.astype(np.int64)])[:-1]]) if ids.size else np.zeros(0)
    return ids.astype(np.uint32), spans.astype(np.uint32)


def check(t, fam, m, a: bytes, b: bytes, label):
    ca, cs = records(fam, m, a)
    ids, spans, info = t.repair_append(a + b, len(a), ca, cs)
    eids, espans = records(fam, m, a + b)
    assert np.array_equal(ids, eids), (label, info)
    assert np.array_equal(spans, espans), (label, info)
    return info


CASES = [("v1", "gpt2", "english_code"), ("v2", "cl100k", "agent_transcript"), ("v3", "o200k", "multilingual"),
         ("v3", "deepseek", "kana_mix")]


@pytest.mark.parametrize("voc,fam,gen", CASES)
def test_appends_to_generated_sessions(tt, voc, fam, gen):
    t, m = tok(tt, voc, fam)
    text = getattr(textgen, gen)(700, 40_000)
    rng = np.random.default_rng(7)
    spliced = 0
    n = 40
    for k in range(n):
        cut = int(rng.integers(600, 30_000))
        add = int(rng.integers(1, 3000))
        a, b = text[:cut].encode(), text[cut:cut + add].encode()
        info = check(t, fam, m, a, b, f"{fam} cut {cut} add {add}")
        spliced += info["spliced"]
    _say("appends", fam, spliced, "of", n, "spliced")
    assert spliced >= n * 3 // 4


@pytest.mark.parametrize("voc,fam,gen", CASES)
def test_multi_step_session(tt, voc, fam, gen):
    t, m = tok(tt, voc, fam)
    text = getattr(textgen, gen)(701, 60_000).encode()
    rng = np.random.default_rng(8)
    cut = 2000
    while text[cut] & 0xC0 == 0x80:
        cut += 1
    ids, spans = records(fam, m, text[:cut])
    steps = 0
    while cut < len(text):
        nxt = min(len(text), cut + int(rng.integers(50, 4000)))
        while nxt < len(text) and text[nxt] & 0xC0 == 0x80:
            nxt += 1
        ids, spans, info = t.repair_append(text[:nxt], cut, ids, spans)
        cut = nxt
        steps += 1
    eids, espans = records(fam, m, text)
    _say("multi-step", fam, steps)
    assert np.array_equal(ids, eids) and np.array_equal(spans, espans)


SEAMS = [
    ("prose " * 200 + "the pipe", "line runs"),                     # one piece across the seam
    ("x" * 700 + " 1234", "5678 y"),                                   # digit grouping from the run start
    ("word " * 150 + "1" * 3000, "23 z"),                              # a digit run longer than the windows
    ("word " * 150 + "a" + " " * 2000, "b"),                           # trailing spaces: lookahead
    ("word " * 150 + "x." + "\n" * 700, "\n y"),                        # newline absorption
    ("word " * 150 + "x" + " \t" * 1500, "\r\n z"),                    # whitespace up to the last CR/LF
    ("Word " * 150 + "get" + "HTTP" * 400, "Response ok"),             # an uppercase run (case rule)
    ("word " * 150 + "'", "s and 're"),                                # contraction across the seam
    ("a" * 5000, "a" * 10),                                            # one letter run
    ("中" * 800 + "x", "1 あい"),                                        # CJK, digits, kana
    ("text " * 200, ""),                                               # empty append
]


@pytest.mark.parametrize("voc,fam", [("v1", "gpt2"), ("v2", "cl100k"), ("v3", "o200k"), ("v3", "deepseek")])
def test_seam_effects(tt, voc, fam):
    t, m = tok(tt, voc, fam)
    for a, b in SEAMS:
        info = check(t, fam, m, a.encode(), b.encode(), (fam, a[-12:], b[:12]))
        _say("seam", fam, repr(a[-8:]), repr(b[:8]), info)


def test_short_and_empty(tt):
    t, m = tok(tt, "v2", "cl100k")
    for a, b in [("", ""), ("", "hello"), ("hi", " there"), ("x" * 511, "y"), ("x" * 513, "y")]:
        info = check(t, "cl100k", m, a.encode(), b.encode(), (a[:5], b))
        if len(a) <= 512:
            assert info["spliced"] == 0 and info["attempts"] == 0


def test_rejects_bad_records(tt):
    t, m = tok(tt, "v2", "cl100k")
    a = ("word " * 200).encode()
    ca, cs = records("cl100k", m, a)
    bad_spans = cs.copy()
    bad_spans[0] = 1
    with pytest.raises(tt.ToktierError) as e:
        t.repair_append(a + b"x", len(a), ca, bad_spans)
    assert e.value.status == 1
    with pytest.raises(tt.ToktierError) as e:
        t.repair_append("é".encode() + a, 1, ca[:1], cs[:1])   # A ends inside a character
    assert e.value.status == 4


@pytest.mark.parametrize("voc,fam,gen", CASES)
def test_in_place_session(tt, voc, fam, gen):
    """RepairSession repairs its records in place (output arrays = cached arrays), growing its
    buffers past their first capacity; after every append the records equal the oracle's full
    encoding of the session text, and the first append of each case is checked on its own."""
    t, m = tok(tt, voc, fam)
    text = getattr(textgen, gen)(702, 30_000).encode()
    rng = np.random.default_rng(9)
    cut = 3000
    while text[cut] & 0xC0 == 0x80:
        cut += 1
    s = tt.RepairSession(t, text[:cut])
    ids, spans = records(fam, m, text[:cut])
    assert np.array_equal(s.ids, ids) and np.array_equal(s.spans, spans)
    steps = spliced = 0
    while cut < len(text):
        nxt = min(len(text), cut + int(rng.integers(20, 6000)))
        while nxt < len(text) and text[nxt] & 0xC0 == 0x80:
            nxt += 1
        info = s.append(text[cut:nxt])
        cut = nxt
        steps += 1
        spliced += info["spliced"]
        if steps in (1, 2) or cut == len(text):
            eids, espans = records(fam, m, text[:cut])
            assert np.array_equal(s.ids, eids) and np.array_equal(s.spans, espans), (fam, steps, info)
    assert bytes(s.text) == text
    _say("in-place session", fam, steps, "appends,", spliced, "spliced")
    assert spliced >= steps // 2


def test_rejects_overlap_and_bad_append(tt):
    t, m = tok(tt, "v2", "cl100k")
    a = ("word " * 300).encode()
    ca, cs = records("cl100k", m, a)
    vocab = t.vocab
    import torch
    scratch = torch.empty(tt.toktier_repair_scratch_bytes(vocab, len(a) + 8), dtype=torch.uint8, device="cuda:0")
    from exact_bpe_tokenization_amd import binding
    text = np.frombuffer(a + b" more", np.uint8)
    buf = np.empty(2 * text.size + ca.size, np.uint32)   # ids and spans overlapping the cached records
    buf[:ca.size] = ca
    with pytest.raises(tt.ToktierError) as e:
        binding._repair(vocab, text, len(a), buf[:ca.size], cs, ca.size, buf[1:1 + text.size],
                        buf[1 + text.size:1 + 2 * text.size], scratch, None)
    assert e.value.status == 1
    with pytest.raises(tt.ToktierError) as e:        # invalid UTF-8 in the append
        t.repair_append(a + b"ok \xff", len(a), ca, cs)
    assert e.value.status == 4
