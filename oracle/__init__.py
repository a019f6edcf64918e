"""CPU oracle for exact byte-level BPE tokenization (TEST INFRASTRUCTURE ONLY).

Plain, serial reference implementations of what the GPU path computes (TokTier, arXiv 2607.29678:
F = E* o G -- a leftmost-first pre-tokenizer G, then byte-level BPE E on every piece independently):

* ``pretokenize``  -- G, a hand-written leftmost-first matcher per regex alternative (oracle.c)
* ``bpe_encode``   -- E, priority-queue BPE over a linked list (oracle.c)
* ``encode_batch`` -- F over a batch of documents, with per-document ID offsets
* ``token_spans``  -- the source byte offset of every token of such a batch
* ``added_matches`` / ``encode_batch_ex`` -- the leftmost-longest added-token pass in front of F,
  and the ignore_merges whole-piece rule
* ``train``        -- the byte-level BPE trainer that produces the merge lists used as inputs
* ``textbook_bpe`` -- the exhaustive textbook merge loop in pure Python, for pinning E on tiny inputs

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package; the
GPU library never does, and the two share no code.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import unicode_classes

FAMILIES = {"gpt2": 1, "cl100k": 2, "o200k": 3, "deepseek": 4}

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_SANITIZE=1: a separate build with AddressSanitizer and UndefinedBehaviorSanitizer (the
# process must preload their runtimes; see tests/test_oracle_sanitized.py)
SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_SO = os.path.join(_BUILD, "liboracle_san.so" if SANITIZE else "liboracle.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

_ERRORS = {
    -1: "invalid UTF-8",
    -2: "output capacity exceeded",
    -3: "unknown family",
    -4: "bad document offsets",
    -5: "out of memory",
    -6: "no alternative matched",
}


class OracleError(RuntimeError):
    def __init__(self, code):
        self.code = code
        super().__init__(_ERRORS.get(code, f"oracle error {code}"))


def build(force=True):
    """Compile oracle.c with gcc into oracle/_build/liboracle.so (liboracle_san.so when sanitized)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        opt = SAN_FLAGS if SANITIZE else ["-O2"]
        subprocess.check_call(["gcc"] + opt + ["-std=c99", "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build(force=True)
    L = ctypes.CDLL(_SO)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.orc_set_classes.argtypes = [u8p, ctypes.c_uint64]
    L.orc_set_classes.restype = ctypes.c_int
    L.orc_pretokenize.argtypes = [ctypes.c_int, u8p, ctypes.c_uint64, u64p, ctypes.c_uint32, u64p,
                                  ctypes.c_uint64]
    L.orc_pretokenize.restype = ctypes.c_int64
    L.orc_bpe_new.argtypes = [u32p, ctypes.c_uint32]
    L.orc_bpe_new.restype = ctypes.c_void_p
    L.orc_bpe_free.argtypes = [ctypes.c_void_p]
    L.orc_bpe_free.restype = None
    L.orc_bpe_encode.argtypes = [ctypes.c_void_p, u8p, u64p, ctypes.c_uint64, u32p, ctypes.c_uint64,
                                 u32p]
    L.orc_bpe_encode.restype = ctypes.c_int64
    L.orc_train.argtypes = [ctypes.c_int, u8p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                            u32p]
    L.orc_train.restype = ctypes.c_int64
    L.orc_encode_batch.argtypes = [ctypes.c_int, ctypes.c_void_p, u8p, ctypes.c_uint64, u64p,
                                   ctypes.c_uint32, u32p, ctypes.c_uint64, u64p]
    L.orc_encode_batch.restype = ctypes.c_int64
    tab = np.ascontiguousarray(unicode_classes.class_table())
    rc = L.orc_set_classes(tab.ctypes.data_as(u8p), tab.size)
    if rc:
        raise RuntimeError(f"orc_set_classes failed: {rc}")
    _lib = L
    return L


def _p(a, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def _family(f):
    return FAMILIES[f] if isinstance(f, str) else int(f)


def _as_u8(data):
    if isinstance(data, np.ndarray):
        return np.ascontiguousarray(data, dtype=np.uint8)
    return np.frombuffer(bytes(data), dtype=np.uint8) if len(data) else np.zeros(0, np.uint8)


def _offsets(data_len, offsets):
    if offsets is None:
        offsets = [0, data_len]
    return np.ascontiguousarray(offsets, dtype=np.uint64)


def pretokenize(family, data, offsets=None):
    """G over a batch: returns uint64 piece start byte offsets (document order), followed by the
    batch end, so that piece k is [out[k], out[k+1])."""
    L = lib()
    buf = _as_u8(data)
    offs = _offsets(buf.size, offsets)
    out = np.zeros(buf.size + 2, dtype=np.uint64)
    n = L.orc_pretokenize(_family(family), _p(buf, ctypes.c_uint8), buf.size, _p(offs, ctypes.c_uint64),
                          offs.size - 1, _p(out, ctypes.c_uint64), buf.size + 1)
    if n < 0:
        raise OracleError(n)
    out[n] = buf.size
    return out[: n + 1].copy()


def split(family, text):
    """G on one string: the list of piece strings (for hand-worked cases)."""
    data = text.encode("utf-8")
    st = pretokenize(family, data)
    return [data[st[k]:st[k + 1]].decode("utf-8") for k in range(len(st) - 1)]


class Merges:
    """A merge list in the oracle's own rank map.  merges[r] = (left_id, right_id) creates 256 + r."""

    def __init__(self, merges):
        m = np.ascontiguousarray(np.asarray(merges, dtype=np.uint32).reshape(-1, 2))
        self.merges = m
        self._h = lib().orc_bpe_new(_p(m, ctypes.c_uint32), m.shape[0])
        if not self._h:
            raise MemoryError

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.orc_bpe_free(self._h)
            self._h = None

    @property
    def n_merges(self):
        return self.merges.shape[0]

    def token_bytes(self):
        """Byte string of every token ID (for decode)."""
        tb = [bytes([b]) for b in range(256)]
        for a, b in self.merges:
            tb.append(tb[a] + tb[b])
        return tb


def bpe_encode(merges, data, piece_starts):
    """E on every piece [piece_starts[k], piece_starts[k+1]): returns (ids uint32, ntok uint32)."""
    L = lib()
    m = merges if isinstance(merges, Merges) else Merges(merges)
    buf = _as_u8(data)
    ps = np.ascontiguousarray(piece_starts, dtype=np.uint64)
    npieces = ps.size - 1
    out = np.zeros(max(buf.size, 1), dtype=np.uint32)
    ntok = np.zeros(max(npieces, 1), dtype=np.uint32)
    n = L.orc_bpe_encode(m._h, _p(buf, ctypes.c_uint8), _p(ps, ctypes.c_uint64), npieces,
                         _p(out, ctypes.c_uint32), out.size, _p(ntok, ctypes.c_uint32))
    if n < 0:
        raise OracleError(n)
    return out[:n].copy(), ntok[:npieces].copy()


def encode_batch(family, merges, data, offsets=None):
    """F = E* o G over a batch: returns (ids uint32[T], out_offsets uint64[D+1])."""
    L = lib()
    m = merges if isinstance(merges, Merges) else Merges(merges)
    buf = _as_u8(data)
    offs = _offsets(buf.size, offsets)
    out = np.zeros(max(buf.size, 1), dtype=np.uint32)
    oo = np.zeros(offs.size, dtype=np.uint64)
    n = L.orc_encode_batch(_family(family), m._h, _p(buf, ctypes.c_uint8), buf.size,
                           _p(offs, ctypes.c_uint64), offs.size - 1, _p(out, ctypes.c_uint32), out.size,
                           _p(oo, ctypes.c_uint64))
    if n < 0:
        raise OracleError(n)
    return out[:n].copy(), oo


def encode(family, merges, text):
    """F on one string: list of IDs."""
    ids, _ = encode_batch(family, merges, text.encode("utf-8"))
    return ids.tolist()


def train(family, corpus, n_merges, max_token_bytes=128):
    """Train a byte-level BPE merge list (uint32[n, 2]) on `corpus` (bytes).  Each step merges the
    most frequent adjacent pair (counted over the pre-tokenized pieces, at least twice), ties to the
    smallest (left, right); merges whose token would exceed max_token_bytes are skipped."""
    L = lib()
    buf = _as_u8(corpus)
    out = np.zeros(2 * max(n_merges, 1), dtype=np.uint32)
    n = L.orc_train(_family(family), _p(buf, ctypes.c_uint8), buf.size, n_merges, max_token_bytes,
                    _p(out, ctypes.c_uint32))
    if n < 0:
        raise OracleError(n)
    return out[: 2 * n].reshape(-1, 2).copy()


def textbook_bpe(merges, piece: bytes):
    """The textbook loop, written out: while some adjacent pair has a rank, merge the leftmost
    occurrence of the lowest-ranked pair.  Quadratic; for tiny inputs only."""
    rank = {}
    for r, (a, b) in enumerate(np.asarray(merges).reshape(-1, 2).tolist()):
        rank.setdefault((a, b), r)
    seq = list(piece)
    while True:
        best = None
        for i in range(len(seq) - 1):
            r = rank.get((seq[i], seq[i + 1]))
            if r is not None and (best is None or r < best[0]):
                best = (r, i)
        if best is None:
            return seq
        r, i = best
        seq[i:i + 2] = [256 + r]


def token_lengths(merges):
    """Byte length of every token ID: 1 for the 256 byte tokens, len(left) + len(right) for the token
    that merge r creates (ID 256 + r)."""
    m = np.asarray(merges, dtype=np.int64).reshape(-1, 2)
    ln = np.ones(256 + m.shape[0], dtype=np.int64)
    for r, (a, b) in enumerate(m.tolist()):
        ln[256 + r] = ln[a] + ln[b]
    return ln


def token_spans(merges, ids, out_offsets, offsets):
    """Source byte offset of every token.  Document d's tokens, ids[out_offsets[d]:out_offsets[d+1]],
    spell its bytes [offsets[d], offsets[d+1]) in order (F = E* o G only regroups the text), so token
    i starts where the tokens before it in its document end.  (TokTier's session store keeps these
    byte spans beside the IDs; its GPU path does not produce them.)"""
    ln = token_lengths(merges)[np.asarray(ids, dtype=np.int64)]
    out = np.zeros(len(ids), dtype=np.uint64)
    for d in range(len(offsets) - 1):
        a, b = int(out_offsets[d]), int(out_offsets[d + 1])
        if a < b:
            out[a:b] = int(offsets[d]) + np.concatenate([[0], np.cumsum(ln[a:b - 1])])
    return out


def added_matches(data, offsets, literals):
    """The added-token pass: literals (special and added tokens) that the model reserves as single
    IDs are taken out of the text before the family's pre-tokenizer runs (paper, implementation
    paragraph on added and special tokens: a leftmost-longest literal pass).  Within each document,
    scanning left to right: where some literal starts and ends inside the document, the longest
    such literal is taken and the scan resumes after it; elsewhere the scan moves one byte on.
    Returns a list of (start byte, literal index) in text order."""
    raw = bytes(_as_u8(data))
    offs = [int(x) for x in _offsets(len(raw), offsets)]
    lits = [bytes(l) for l in literals]
    if any(len(l) == 0 for l in lits):
        raise ValueError("empty literal")
    starts = {}                                  # position -> indices of the literals found there
    for k, l in enumerate(lits):
        i = raw.find(l)
        while i >= 0:
            starts.setdefault(i, []).append(k)
            i = raw.find(l, i + 1)
    out, d, resume = [], 0, 0
    for p in sorted(starts):
        if p < resume:
            continue
        while offs[d + 1] <= p:                  # the document holding byte p
            d += 1
        fit = [k for k in starts[p] if p + len(lits[k]) <= offs[d + 1]]
        if not fit:
            continue
        k = max(fit, key=lambda k: (len(lits[k]), -k))
        out.append((p, k))
        resume = p + len(lits[k])
    return out


def encode_batch_ex(family, merges, data, offsets=None, added=(), ignore_merges=False):
    """F with the added-token pass in front of it and, optionally, the ignore_merges rule in E.

    added: (literal bytes, ID) pairs; every literal taken by ``added_matches`` becomes its one ID, and
    the text between literals (and between a literal and its document's ends) is tokenized as a
    document of its own.  ignore_merges (paper, GPU BPE paragraph: the Llama 3 / gpt-oss encoder
    emits one ID when the whole piece is a vocabulary entry): a piece whose bytes are some token's
    bytes becomes that token -- the smallest such ID when several tokens share the bytes -- and
    only the other pieces go through the merge loop.  Returns (ids uint32[T], out_offsets
    uint64[D+1])."""
    m = merges if isinstance(merges, Merges) else Merges(merges)
    raw = bytes(_as_u8(data))
    offs = [int(x) for x in _offsets(len(raw), offsets)]
    lits = [bytes(b) for b, _ in added]
    lid = [int(i) for _, i in added]
    found = added_matches(raw, offs, lits) if lits else []
    # documents cut at the literals: items are ("seg", a, b) or ("lit", k), per document in order
    items, fi = [], 0
    for d in range(len(offs) - 1):
        doc, cur = [], offs[d]
        while fi < len(found) and found[fi][0] < offs[d + 1]:
            p, k = found[fi]
            doc.append(("seg", cur, p))
            doc.append(("lit", k))
            cur = p + len(lits[k])
            fi += 1
        doc.append(("seg", cur, offs[d + 1]))
        items.append(doc)
    segs = [(it[1], it[2]) for doc in items for it in doc if it[0] == "seg"]
    seg_offs = np.array([0] + [b for _, b in segs], dtype=np.uint64) if segs else np.zeros(1, np.uint64)
    # G on the text segments (segment i spans [segs[i][0], segs[i][1]) of raw, cut out and
    # concatenated; each is a document of its own)
    text = b"".join(raw[a:b] for a, b in segs)
    cut = np.concatenate([[0], np.cumsum([b - a for a, b in segs])]).astype(np.uint64)
    if not ignore_merges:   # F on the segments as documents
        e, eo = encode_batch(family, m, text, cut)
        seg_ids = [e[int(eo[i]):int(eo[i + 1])].tolist() for i in range(len(segs))]
        return _join_items(items, seg_ids, lid)
    starts = pretokenize(family, text, cut)
    pieces = [text[int(starts[k]):int(starts[k + 1])] for k in range(len(starts) - 1)]
    whole = {}
    if ignore_merges:
        for t, b in enumerate(m.token_bytes()):
            whole.setdefault(b, t)
    # E on every piece that the whole-piece rule does not settle
    todo = [i for i, pc in enumerate(pieces) if pc not in whole]
    ids_of = [[whole[pc]] if pc in whole else None for pc in pieces]
    if todo:
        buf = b"".join(pieces[i] for i in todo)
        ps = np.concatenate([[0], np.cumsum([len(pieces[i]) for i in todo])]).astype(np.uint64)
        e, nt = bpe_encode(m, buf, ps)
        pos = 0
        for i, c in zip(todo, nt.tolist()):
            ids_of[i] = e[pos:pos + c].tolist()
            pos += c
    piece_seg = np.searchsorted(cut, starts[:-1], side="right") - 1
    seg_ids = [[] for _ in segs]
    for i, sidx in enumerate(piece_seg.tolist()):
        seg_ids[sidx].extend(ids_of[i])
    return _join_items(items, seg_ids, lid)


def _join_items(items, seg_ids, lid):
    """Per document, the text segments' IDs with the literals' IDs between them."""
    out, oo, si = [], [0], 0
    for doc in items:
        for it in doc:
            if it[0] == "lit":
                out.append(lid[it[1]])
            else:
                out.extend(seg_ids[si])
                si += 1
        oo.append(len(out))
    return np.array(out, dtype=np.uint32), np.array(oo, dtype=np.uint64)


def decode(merges, ids):
    tb = (merges if isinstance(merges, Merges) else Merges(merges)).token_bytes()
    return b"".join(tb[i] for i in ids)
