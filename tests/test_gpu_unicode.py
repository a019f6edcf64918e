"""GPU split parity over every Unicode scalar value.

Each family's pre-tokenizer classifies characters with the device's two-stage Unicode table (decoded
from UTF-8 on the GPU).  Here every scalar value U+0000..U+10FFFF except the surrogates appears in the
input, in a seeded random order, cut into documents of random lengths that straddle the 8 KiB tiles;
a second batch puts each scalar value after a random character of a small mixed alphabet (letters,
digits, spaces, CR/LF, punctuation, an apostrophe) so that every value is also seen next to each
class.  Piece boundaries must equal the oracle's exactly.
"""
import numpy as np
import pytest

import oracle
from parity import compare_starts
from workloads import textgen

pytestmark = pytest.mark.gpu

FAMS = ("gpt2", "cl100k", "o200k", "deepseek")
CONTEXT = list("aZ9 \t\r\n.'s") + ["é", "中", "٣"]


def _say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module")
def tt():
    import torch
    import exact_bpe_tokenization_amd as tt
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tt.lib()
    return tt


def _all_scalars(seed):
    cps = np.concatenate([np.arange(0, 0xD800), np.arange(0xE000, 0x110000)])
    return np.random.default_rng(seed).permutation(cps)


def _documents(chars, seed):
    rng = np.random.default_rng(seed)
    docs, i = [], 0
    while i < len(chars):
        k = int(10 ** rng.uniform(0, 4.3))
        docs.append("".join(chars[i:i + k]))
        i += k
    return docs


@pytest.mark.parametrize("family", FAMS)
def test_split_every_scalar(tt, family):
    cps = _all_scalars(11)
    chars = [chr(int(c)) for c in cps]
    data, offs = textgen.to_batch(_documents(chars, 12))
    _say("split every scalar", family, data.size, offs.size - 1)
    tok = tt.Tokenizer(np.zeros((0, 2), np.uint32), family)
    compare_starts(oracle.pretokenize(family, data, offs), tok.pretokenize(data.tobytes(), offs), data)


@pytest.mark.parametrize("family", FAMS)
def test_split_every_scalar_in_context(tt, family):
    cps = _all_scalars(13)
    rng = np.random.default_rng(14)
    ctx = rng.integers(0, len(CONTEXT), cps.size)
    chars = [CONTEXT[int(k)] + chr(int(c)) for k, c in zip(ctx, cps)]
    data, offs = textgen.to_batch(_documents(chars, 15))
    _say("split every scalar in context", family, data.size, offs.size - 1)
    tok = tt.Tokenizer(np.zeros((0, 2), np.uint32), family)
    compare_starts(oracle.pretokenize(family, data, offs), tok.pretokenize(data.tobytes(), offs), data)
