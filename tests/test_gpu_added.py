"""GPU parity of the added-token pass and the ignore_merges rule against the oracle, bit for bit.

Added tokens: literals inserted into the workloads (special-token markers, a code fence, a one-byte
literal), literals at document ends, adjacent and overlapping literals (clusters that the
leftmost-longest scan walks), a literal that crosses a document boundary (no match), documents
that are exactly a literal, dense literals, a vocabulary with literals but a text without any, and
token spans through the literal path.  ignore_merges: the workloads, every token's own string as a
document (each must come back as the smallest ID with that string, including tokens longer than the
whole-piece tables' 32 bytes), and random merge lists with tokens that are not their own BPE.
"""
import numpy as np
import pytest

import oracle
from parity import compare_ids
from workloads import textgen

pytestmark = pytest.mark.gpu

LIT_BASE = 1 << 22   # literal IDs outside every merge list's range


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


def tok_for(tt, voc, lits=(), ignore_merges=False):
    key = (voc, tuple(lits), ignore_merges)
    if key not in _TOK:
        merges, fam = textgen.load_vocab(voc)
        added = [(l, LIT_BASE + k) for k, l in enumerate(lits)]
        _TOK[key] = (tt.Tokenizer(merges, fam, added=added, ignore_merges=ignore_merges), merges, fam, added)
    return _TOK[key]


def _check(tok, merges, fam, added, data, offs, ignore_merges, label, spans=False):
    _say(label, data.size if hasattr(data, "size") else len(data))
    raw = data.tobytes() if hasattr(data, "tobytes") else bytes(data)
    if spans:
        ids, oo, sp = tok.encode(raw, offs, spans=True)
    else:
        ids, oo = tok.encode(raw, offs)
    eids, eoo = oracle.encode_batch_ex(fam, merges, raw, offs, added=added, ignore_merges=ignore_merges)
    compare_ids(eids, eoo, ids, oo)
    if spans:
        # a token's span: its document's offset plus the lengths of the tokens before it
        tb = oracle.Merges(merges).token_bytes()
        litlen = {i: len(l) for l, i in added}
        offs_ = [0, len(raw)] if offs is None else list(offs)
        exp = np.zeros(eids.size, dtype=np.uint64)
        for d in range(len(offs_) - 1):
            pos = int(offs_[d])
            for t in range(int(eoo[d]), int(eoo[d + 1])):
                exp[t] = pos
                i = int(eids[t])
                pos += litlen[i] if i in litlen else len(tb[i])
        bad = np.flatnonzero(exp != sp.astype(np.uint64))
        assert bad.size == 0, f"{bad.size} spans differ, first at {bad[0]}"


LITS = [b"<|endoftext|>", b"<|im_start|>", b"<|im_end|>", b"```", b"\xc2\xa7"]


def _insert_literals(texts, seed, per_doc=6):
    rng = np.random.default_rng(seed)
    out = []
    for t in texts:
        for _ in range(per_doc):
            i = int(rng.integers(0, len(t) + 1))
            t = t[:i] + LITS[int(rng.integers(0, len(LITS)))].decode() + t[i:]
        out.append(t)
    return out


@pytest.mark.parametrize("name", ["c1_ec4k", "c2_at100k", "c3_mix1m", "c4_batch64"])
def test_added_workloads(tt, name):
    fam, voc, data, offs = textgen.workload(name, 0.1 if name == "c4_batch64" else 1.0)
    tok, merges, fam, added = tok_for(tt, voc, LITS)
    texts = [data[int(offs[d]):int(offs[d + 1])].tobytes().decode() for d in range(len(offs) - 1)]
    texts = _insert_literals(texts, 7, per_doc=40)
    d2, o2 = textgen.to_batch(texts)
    _check(tok, merges, fam, added, d2, o2, False, f"added {name}")


def test_added_spans(tt):
    tok, merges, fam, added = tok_for(tt, "v2", LITS)
    texts = _insert_literals([textgen.agent_transcript(40 + i, 5000 + 300 * i) for i in range(6)], 9, per_doc=25)
    texts += ["<|endoftext|>", "", "§§§", "x<|im_end|>"]
    d2, o2 = textgen.to_batch(texts)
    _check(tok, merges, fam, added, d2, o2, False, "added spans", spans=True)


def test_added_edge_cases(tt):
    lits = [b"ab", b"abc", b"bcd", b"d", b"<|eot|>", b"aa"]
    tok, merges, fam, added = tok_for(tt, "v2", lits)
    cases = [
        ["abcd"], ["ab", "cd"], ["abcd", "", "d"], ["", ""], ["<|eot|>"], ["<|eot|><|eot|>", "<|eot|>x"],
        ["<|eo", "t|>"],                                  # crosses a document boundary: no literal
        ["a" * 9], ["a" * 4097 + "bcd"], ["xbcdx", "dd d"], ["hello world" * 500 + "abcd" * 300],
        ["d" * 5000], ["aab" * 3000, "ab" * 2000 + "c"],  # dense literals and long overlap clusters
        ["no literal here at all, only text"],            # one-byte literal "d" absent too
        ["z" * 8191 + "abc", "q" * 8192 + "<|eot|>"],     # literals at tile edges
    ]
    for strings in cases:
        data, offs = textgen.to_batch(strings)
        _check(tok, merges, fam, added, data, offs, False, ["edge"] + [s[:12] for s in strings], spans=True)


def test_added_without_matches_and_errors(tt):
    tok, merges, fam, added = tok_for(tt, "v2", [b"<|never|>"])
    data, offs = textgen.workload("c2_at100k", 1.0)[2:]
    _check(tok, merges, fam, added, data, offs, False, "added no matches")
    with pytest.raises(tt.ToktierError) as e:
        tok.encode(b"abc<|never|>def", [0, 5, 2, 15])
    assert e.value.status == 1
    with pytest.raises(tt.ToktierError) as e:
        tok.encode(b"abc<|never|>d\xffef")
    assert e.value.status == 4
    # still exact afterwards
    _check(tok, merges, fam, added, b"x<|never|>y", None, False, "after errors")


def test_bad_added_tokens_rejected(tt):
    merges, fam = textgen.load_vocab("v1")
    for bad in ([(b"", 5)], [(b"\xff", 5)], [(b"ab", 5), (b"ab", 6)], [(b"x" * 257, 5)]):
        with pytest.raises(tt.ToktierError) as e:
            tt.toktier_load_vocab_ex(merges, fam, 0, bad)
        assert e.value.status == 1


@pytest.mark.parametrize("name", list(textgen.WORKLOADS))
def test_ignore_merges_workloads(tt, name):
    fam, voc, data, offs = textgen.workload(name, 0.05 if name in ("c4_batch64", "c5_adv4m4") else 1.0)
    tok, merges, fam, added = tok_for(tt, voc, (), True)
    _check(tok, merges, fam, added, data, offs, True, f"ignore_merges {name}")


@pytest.mark.parametrize("voc", ["v1", "v2", "v3", "v4"])
def test_ignore_merges_every_token_string(tt, voc):
    tok, merges, fam, added = tok_for(tt, voc, (), True)
    tb = oracle.Merges(merges).token_bytes()
    texts = []
    for t in range(256, len(tb)):
        try:
            texts.append(tb[t].decode("utf-8"))
        except UnicodeDecodeError:
            pass
    data, offs = textgen.to_batch(texts)
    long_ = sum(len(t.encode()) > 32 for t in texts)
    _check(tok, merges, fam, added, data, offs, True, f"ignore_merges token strings {voc} (>32 B: {long_})")


@pytest.mark.parametrize("seed", [0, 1])
def test_ignore_merges_random_lists(tt, seed):
    rng = np.random.default_rng(seed)
    alpha = [ord(c) for c in "abcd"]
    ids, seen, merges = list(alpha), set(), []
    ln = {i: 1 for i in alpha}
    while len(merges) < 400:   # tokens of at most 80 bytes (ignore_merges takes tokens up to 256)
        a, b = ids[int(rng.integers(0, len(ids)))], ids[int(rng.integers(0, len(ids)))]
        if (a, b) in seen or ln[a] + ln[b] > 80:
            continue
        seen.add((a, b))
        merges.append((a, b))
        ids.append(255 + len(merges))
        ln[ids[-1]] = ln[a] + ln[b]
    merges = np.array(merges, dtype=np.uint32)
    tb = oracle.Merges(merges).token_bytes()
    words = ["".join(chr(int(c)) for c in rng.choice(alpha, int(rng.integers(1, 90)))) for _ in range(2000)]
    words += [tb[t].decode() for t in range(256, len(tb))]
    lits = [b"abca", b"<|x|>"]
    added = [(l, LIT_BASE + k) for k, l in enumerate(lits)]
    for fam in ("gpt2", "cl100k", "o200k"):
        tok = tt.Tokenizer(merges, fam, added=added, ignore_merges=True)
        data, offs = textgen.to_batch([" ".join(words[i:i + 5]) for i in range(0, len(words), 5)])
        _check(tok, merges, fam, added, data, offs, True, f"ignore_merges random {seed} {fam}", spans=True)
