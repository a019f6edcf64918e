"""Pins of the oracle's token spans (the source byte offset of every token).

The spans follow from the IDs: a document's tokens spell its bytes in order.  They are checked
against what that fixes -- every token's bytes appear in the text at its span, spans are strictly
increasing inside a document, the first starts at the document's offset and the last ends at the
next one -- and against spans built independently, piece by piece, from the serial pre-tokenizer
and the pure-Python textbook BPE; plus a hand-worked case.
"""
import numpy as np
import pytest

import oracle
from workloads import textgen


def _merges_from(pairs_bytes):
    """A merge list from byte-string pairs (left, right), each side a byte or an earlier merge."""
    ids = {bytes([i]): i for i in range(256)}
    out = []
    for a, b in pairs_bytes:
        out.append((ids[a], ids[b]))
        ids[a + b] = 255 + len(out)
    return np.asarray(out, dtype=np.uint32)


def test_hand_worked_spans():
    # merges "pi", "pe", "pipe", "li", "ne", "line".  The gpt2 pattern keeps a leading space with the
    # letters, so " pipeline" is one piece; with no merge taking the space its BPE is
    # [" ", "pipe", "line"] at spans 0, 1, 5, and the second document's "line" starts at byte 9
    m = _merges_from([(b"p", b"i"), (b"p", b"e"), (b"pi", b"pe"), (b"l", b"i"), (b"n", b"e"), (b"li", b"ne")])
    data, offs = textgen.to_batch([" pipeline", "line"])
    ids, oo = oracle.encode_batch("gpt2", m, data, offs)
    tb = oracle.Merges(m).token_bytes()
    assert [tb[i] for i in ids] == [b" ", b"pipe", b"line", b"line"]
    assert oracle.token_spans(m, ids, oo, offs).tolist() == [0, 1, 5, 9]


@pytest.mark.parametrize("voc,gen", [("v1", textgen.english_code), ("v2", textgen.agent_transcript),
                                     ("v3", textgen.multilingual)])
def test_spans_spell_the_text(voc, gen):
    merges, fam = textgen.load_vocab(voc)
    texts = [gen(50 + i, 300 + 97 * i) for i in range(6)] + ["", "x", ""]
    data, offs = textgen.to_batch(texts)
    ids, oo = oracle.encode_batch(fam, merges, data, offs)
    sp = oracle.token_spans(merges, ids, oo, offs)
    tb = oracle.Merges(merges).token_bytes()
    raw = data.tobytes()
    for d in range(len(offs) - 1):
        a, b = int(oo[d]), int(oo[d + 1])
        if a == b:
            assert offs[d] == offs[d + 1]
            continue
        assert int(sp[a]) == int(offs[d])
        assert np.all(np.diff(sp[a:b].astype(np.int64)) > 0)
        last = int(ids[b - 1])
        assert int(sp[b - 1]) + len(tb[last]) == int(offs[d + 1])
    for i in range(ids.size):
        t = tb[int(ids[i])]
        assert raw[int(sp[i]):int(sp[i]) + len(t)] == t


@pytest.mark.parametrize("fam,voc", [("gpt2", "v1"), ("cl100k", "v2"), ("o200k", "v3")])
def test_spans_match_piecewise_textbook(fam, voc):
    merges, _ = textgen.load_vocab(voc)
    rng = np.random.default_rng(5)
    texts = [textgen.multilingual(int(rng.integers(0, 1000)), 150) for _ in range(3)]
    data, offs = textgen.to_batch(texts)
    ids, oo = oracle.encode_batch(fam, merges, data, offs)
    sp = oracle.token_spans(merges, ids, oo, offs)
    # independently: pieces from G, each piece's tokens from the textbook loop, spans inside the piece
    starts = oracle.pretokenize(fam, data, offs).astype(np.int64)
    tb = oracle.Merges(merges).token_bytes()
    raw = data.tobytes()
    exp = []
    for k in range(starts.size - 1):
        pos = int(starts[k])
        for t in oracle.textbook_bpe(merges, raw[starts[k]:starts[k + 1]]):
            exp.append(pos)
            pos += len(tb[t])
    assert sp.tolist() == exp
