"""C ABI checks that need no GPU: the library loads and exports every symbol include/toktier.h
declares; host-side validation rejects bad inputs with the documented status codes before any device
call; without a GPU a device call fails loudly; the frozen Unicode table matches a fresh probe of the
`regex` engine and agrees with the oracle's independently probed classes."""
import os
import re

import numpy as np
import pytest

import exact_bpe_tokenization_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "toktier.h")).read()
    return sorted(set(re.findall(r"\b(toktier_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    lib = tt.lib()
    decl = declared_symbols()
    assert decl == sorted(tt.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = tt.lib()
    for s in range(8):
        assert lib.toktier_status_string(s) not in (b"", b"unknown status")


@pytest.mark.parametrize("merges,family,status", [
    ([(300, 1)], "gpt2", 3),                     # operand created by a later merge
    ([(97, 98), (97, 98)], "cl100k", 3),         # duplicate byte pair
    ([(97, 98), (256, 99), (256, 99)], "o200k", 3),  # duplicate general pair
    ([(97, 98), (257, 97)], "gpt2", 3),          # rank 1 refers to its own token
    ([(97, 98)], 9, 2),                          # unknown family
])
def test_load_vocab_rejects(merges, family, status):
    with pytest.raises(tt.ToktierError) as e:
        tt.toktier_load_vocab(merges, family)
    assert e.value.status == status


def test_workspace_bytes():
    a = tt.toktier_workspace_bytes(0, 1)
    b = tt.toktier_workspace_bytes(4096, 1)
    c = tt.toktier_workspace_bytes(18_448_209, 64)
    assert 0 < a < b < c
    with pytest.raises(tt.ToktierError):
        tt.toktier_workspace_bytes(1 << 32, 1)


def test_device_call_fails_loudly_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(tt.ToktierError) as e:
        tt.toktier_load_vocab([(97, 98)], "gpt2")
    assert e.value.status == 6


def test_unicode_table_frozen_and_independent():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "gen", os.path.join(ROOT, "exact_bpe_tokenization_amd", "csrc", "gen_unicode_table.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    text, digest = gen.build()
    assert digest == tt.toktier_unicode_table_sha256()
    assert text == open(os.path.join(ROOT, "exact_bpe_tokenization_amd", "csrc", "unicode_table.inc")).read()
    # the oracle probes the same engine with different code; the two must agree everywhere
    from oracle import unicode_classes as uc
    orc = uc.class_table()
    cats = np.frombuffer(gen.categories(), dtype=np.uint8)
    mapping = {0: uc.LU, 1: uc.LL, 2: uc.LO, 3: uc.N, 4: uc.W, 5: uc.M, 6: uc.O, 6 | 16: uc.PS}
    mapped = np.vectorize(mapping.get, otypes=[np.uint8])(cats)
    assert np.array_equal(mapped, orc)
