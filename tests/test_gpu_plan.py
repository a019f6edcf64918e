"""HIP-graph plans (toktier_plan_*): the captured kernel chain replayed on fixed buffers.

Every replay must equal the eager encode and the oracle bit for bit.  The graph is replayed several
times with the program's own eager work and synchronizations between replays (an eager encode of
another text on another workspace), with and without spans, and after new text of the same size is
written into the input buffer (a replay recomputes everything; nothing is cached).
"""
import numpy as np
import pytest

import oracle
from parity import compare_ids
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


def _dev(tt, data, offs):
    import torch
    n, d = data.size, len(offs) - 1
    bufs = dict(
        data=torch.from_numpy(data.copy()).cuda(),
        offs=torch.from_numpy(np.asarray(offs, dtype=np.int64)).cuda(),
        ids=torch.empty(max(n, 1), dtype=torch.int32, device="cuda"),
        oo=torch.empty(d + 1, dtype=torch.int64, device="cuda"),
        spans=torch.empty(max(n, 1), dtype=torch.int32, device="cuda"),
    )
    return bufs


@pytest.mark.parametrize("name,scale", [("c1_ec4k", 1.0), ("c2_at100k", 1.0), ("c3_mix1m", 0.3),
                                        ("c4_batch64", 0.05), ("c5_adv4m4", 0.1)])
@pytest.mark.parametrize("spans", [False, True])
def test_plan_replays_match_eager_and_oracle(tt, name, scale, spans):
    import torch
    fam, voc, data, offs = textgen.workload(name, scale)
    merges, _ = textgen.load_vocab(voc)
    tok = tt.Tokenizer(merges, fam)
    eids, eoo = oracle.encode_batch(fam, merges, data, offs)
    espans = oracle.token_spans(merges, eids, eoo, offs) if spans else None
    b = _dev(tt, data, offs)
    ws = torch.empty(tt.toktier_workspace_bytes_ex(tok.vocab, data.size, len(offs) - 1), dtype=torch.uint8,
                     device="cuda")
    plan = tt.Plan(tok.vocab, b["data"], b["offs"], b["ids"], b["oo"], ws, out_spans=b["spans"] if spans else None)
    other = textgen.agent_transcript(55, 30000).encode()
    for rep in range(3):
        _say("plan", name, scale, "spans" if spans else "ids", "replay", rep, data.size)
        nt = plan.launch()
        ids = b["ids"][:nt].cpu().numpy().view(np.uint32)
        oo = b["oo"].cpu().numpy().astype(np.uint64)
        compare_ids(eids, eoo, ids, oo)
        if spans:
            assert np.array_equal(b["spans"][:nt].cpu().numpy().view(np.uint32), espans.astype(np.uint32))
        tok.encode(other)                 # eager work on the tokenizer's own buffers between replays
        torch.cuda.synchronize()


def test_plan_sees_new_input(tt):
    import torch
    merges, fam = textgen.load_vocab("v2")
    tok = tt.Tokenizer(merges, fam)
    t1 = textgen.agent_transcript(61, 50000).encode()
    t2 = textgen.agent_transcript(62, 80000).encode()[:len(t1)]
    while t2 and (t2[-1] & 0xC0) == 0x80:       # keep it valid UTF-8 at the same length
        t2 = t2[:-1] + b" "
    offs = [0, 20000, len(t1)]
    b = _dev(tt, np.frombuffer(t1, np.uint8), offs)
    ws = torch.empty(tt.toktier_workspace_bytes(len(t1), 2), dtype=torch.uint8, device="cuda")
    plan = tt.Plan(tok.vocab, b["data"], b["offs"], b["ids"], b["oo"], ws)
    for t in (t1, t2, t1):
        b["data"].copy_(torch.from_numpy(np.frombuffer(t, np.uint8).copy()).cuda())
        nt = plan.launch()
        eids, eoo = oracle.encode_batch(fam, merges, np.frombuffer(t, np.uint8), offs)
        compare_ids(eids, eoo, b["ids"][:nt].cpu().numpy().view(np.uint32), b["oo"].cpu().numpy().astype(np.uint64))


def test_plan_rejects_added_tokens(tt):
    import torch
    merges, fam = textgen.load_vocab("v2")
    tok = tt.Tokenizer(merges, fam, added=[(b"<|x|>", 1 << 22)])
    data = np.frombuffer(b"hello <|x|> world", np.uint8)
    b = _dev(tt, data, [0, data.size])
    ws = torch.empty(tt.toktier_workspace_bytes_ex(tok.vocab, data.size, 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(tt.ToktierError) as e:
        tt.Plan(tok.vocab, b["data"], b["offs"], b["ids"], b["oo"], ws)
    assert e.value.status == 1


def test_bucket_plan_serves_three_request_sizes(tt):
    """One plan captured for a size bucket (toktier_plan_create_bucket), replayed on three requests of
    different sizes and document counts written into its buffers (sizes in device memory), each
    against the oracle; replays are repeated with eager work of another workspace in between; an
    oversized request encodes nothing and is reported."""
    import torch
    merges, fam = textgen.load_vocab("v2")
    tok = tt.Tokenizer(merges, fam)
    max_bytes, max_docs = 400_000, 16
    data_b = torch.zeros(max_bytes, dtype=torch.uint8, device="cuda")
    offs_b = torch.zeros(max_docs + 1, dtype=torch.int64, device="cuda")
    sizes = torch.zeros(2, dtype=torch.int64, device="cuda")
    ids_b = torch.empty(max_bytes, dtype=torch.int32, device="cuda")
    oo_b = torch.empty(max_docs + 1, dtype=torch.int64, device="cuda")
    ws = torch.empty(tt.toktier_workspace_bytes_ex(tok.vocab, max_bytes, max_docs), dtype=torch.uint8, device="cuda")
    plan = tt.BucketPlan(tok.vocab, data_b, offs_b, sizes, ids_b, oo_b, ws)
    requests = [
        [textgen.agent_transcript(71, 100_000)],                                            # one 100K-char document
        [textgen.english_code(72, k) for k in (5000, 1, 60_000, 0, 120_000, 33)],          # six, with empty ones
        ["x = 1\n"],                                                                        # a few bytes
    ]
    other = textgen.agent_transcript(73, 50_000).encode()
    for rep in range(2):
        for k, texts in enumerate(requests):
            data, offs = textgen.to_batch(texts)
            _say("bucket plan request", k, "replay", rep, data.size, len(offs) - 1)
            data_b[: data.size].copy_(torch.from_numpy(data))
            offs_b[: offs.size].copy_(torch.from_numpy(offs.astype(np.int64)))
            sizes.copy_(torch.tensor([data.size, offs.size - 1], dtype=torch.int64))
            nt = plan.launch()
            eids, eoo = oracle.encode_batch(fam, merges, data, offs)
            compare_ids(eids, eoo, ids_b[:nt].cpu().numpy().view(np.uint32), oo_b[: offs.size].cpu().numpy())
            tok.encode(other)   # eager work on another workspace between replays
    # a request larger than the bucket: nothing encoded, reported as an invalid argument
    sizes.copy_(torch.tensor([max_bytes + 1, 1], dtype=torch.int64))
    with pytest.raises(tt.ToktierError):
        plan.launch()
    sizes.copy_(torch.tensor([10, max_docs + 1], dtype=torch.int64))
    with pytest.raises(tt.ToktierError):
        plan.launch()
