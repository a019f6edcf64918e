"""GPU parity of the DeepSeek-style family (three splitters in sequence) against the oracle, bit for bit.

Split level on every string of up to three characters over the family's stress alphabet, on random
stress strings with long single-kind runs across 8 KiB tiles (digits, kana, ideographs, punctuation,
controls that no alternative matches), on generated text of several kinds; ID level (131,072-merge
vocabulary) on the same text, on multi-document batches with empty and one-character documents, with
token spans, and through the added-token pass.
"""
import itertools

import numpy as np
import pytest

import oracle
from parity import compare_ids, compare_starts
from test_oracle_deepseek import ALPHA_DS, ALPHA_DS_WIDE
from workloads import textgen

pytestmark = pytest.mark.gpu

FAM = "deepseek"


def _say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module")
def tt():
    import torch
    import exact_bpe_tokenization_amd as tt
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tt.lib()
    return tt


@pytest.fixture(scope="module")
def bare(tt):
    return tt.Tokenizer(np.zeros((0, 2), np.uint32), FAM)


@pytest.fixture(scope="module")
def v3(tt):
    merges, _ = textgen.load_vocab("v3")
    return tt.Tokenizer(merges, FAM), merges


def test_split_exhaustive_short(bare):
    strings = ["".join(t) for L in range(1, 4) for t in itertools.product(ALPHA_DS, repeat=L)]
    data, offs = textgen.to_batch(strings)
    _say("ds split exhaustive", data.size, len(strings))
    compare_starts(oracle.pretokenize(FAM, data, offs), bare.pretokenize(data.tobytes(), offs), data)


@pytest.mark.parametrize("seed", [1, 2])
def test_split_random_stress(bare, seed):
    rng = np.random.default_rng(100 + seed)
    strings = ["".join(ALPHA_DS_WIDE[int(i)] for i in rng.integers(0, len(ALPHA_DS_WIDE), int(rng.integers(1, 40))))
               for _ in range(30000)]
    strings += ["1" * 10001 + "a", "あ" * 3000 + "x", "中" * 3000 + "1" * 7, "." * 9000 + "abc",
                "\x00" * 9000 + "a", "a" * 8190 + "1" * 5 + "中" * 5, " " * 8193 + "1", "a1" * 5000,
                "・" * 3000, "$" + "a" * 9000, "ー" * 2000 + "ア" * 2000]
    data, offs = textgen.to_batch(strings)
    _say("ds split random", seed, data.size)
    compare_starts(oracle.pretokenize(FAM, data, offs), bare.pretokenize(data.tobytes(), offs), data)


@pytest.mark.parametrize("gen,n", [("kana_mix", 1_000_000), ("multilingual", 300_000),
                                   ("agent_transcript", 300_000), ("english_code", 100_000)])
def test_ids_generated(v3, gen, n):
    tok, merges = v3
    texts = [getattr(textgen, gen)(500 + i, n // 4 + 1237 * i) for i in range(4)] + ["", "1", "中"]
    data, offs = textgen.to_batch(texts)
    _say("ds ids", gen, data.size)
    st = tok.pretokenize(data.tobytes(), offs)
    compare_starts(oracle.pretokenize(FAM, data, offs), st, data)
    ids, oo = tok.encode(data.tobytes(), offs)
    eids, eoo = oracle.encode_batch(FAM, merges, data, offs)
    compare_ids(eids, eoo, ids, oo)


def test_ids_adversarial_slices(v3):
    tok, merges = v3
    text = textgen.adversarial(5)
    cuts = [0, 100_000, 200_000, 300_001, 400_002, 500_003, 600_005, 700_006, 800_007, 900_008,
            1_200_000, 1_900_008, 2_300_000, 2_400_008]
    texts = [text[max(0, c - 20000):c + 20000] for c in cuts]
    data, offs = textgen.to_batch(texts)
    _say("ds adversarial slices", data.size)
    ids, oo = tok.encode(data.tobytes(), offs)
    eids, eoo = oracle.encode_batch(FAM, merges, data, offs)
    compare_ids(eids, eoo, ids, oo)


def test_spans_and_added(tt, v3):
    _, merges = v3
    text = textgen.kana_mix(611, 200_000)
    data, offs = textgen.to_batch([text[:90_000], text[90_000:]])
    tok = tt.Tokenizer(merges, FAM)
    _say("ds spans", data.size)
    ids, oo, spans = tok.encode(data.tobytes(), offs, spans=True)
    eids, eoo = oracle.encode_batch(FAM, merges, data, offs)
    compare_ids(eids, eoo, ids, oo)
    assert np.array_equal(spans, oracle.token_spans(merges, eids, eoo, offs))
    lits = [("<|user|>".encode(), 1 << 22), ("。".encode(), (1 << 22) + 1)]
    lt = tt.Tokenizer(merges, FAM, added=lits)
    t2 = "<|user|>" + text[:50_000] + "<|user|>x"
    data2, offs2 = textgen.to_batch([t2, "。。<|user|>"])
    _say("ds added", data2.size)
    ids2, oo2 = lt.encode(data2.tobytes(), offs2)
    eids2, eoo2 = oracle.encode_batch_ex(FAM, merges, data2, offs2, added=lits)
    compare_ids(eids2, eoo2, ids2, oo2)
