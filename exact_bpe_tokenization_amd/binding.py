"""Thin Python binding of libtoktier (include/toktier.h): argument marshalling only.

Every step of the tokenization runs in the library's HIP kernels.  torch is used for device memory
and streams; it is imported first so that the library binds to the HIP runtime torch has loaded.
There is no fallback: if the library is missing or a call fails, a ToktierError is raised.
"""
import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# TOKTIER_LIBRARY may name another build of the same library (same exports), e.g. an instrumented one
LIB_PATH = os.environ.get("TOKTIER_LIBRARY") or os.path.join(HERE, "libtoktier.so")

TOKTIER_GPT2, TOKTIER_CL100K, TOKTIER_O200K, TOKTIER_DEEPSEEK = 1, 2, 3, 4
TOKTIER_IGNORE_MERGES = 1
FAMILIES = {"gpt2": TOKTIER_GPT2, "cl100k": TOKTIER_CL100K, "o200k": TOKTIER_O200K,
            "deepseek": TOKTIER_DEEPSEEK}
STATUS = {0: "TOKTIER_OK", 1: "TOKTIER_E_INVALID_ARG", 2: "TOKTIER_E_BAD_FAMILY", 3: "TOKTIER_E_BAD_MERGES",
          4: "TOKTIER_E_INVALID_UTF8", 5: "TOKTIER_E_CAPACITY", 6: "TOKTIER_E_HIP", 7: "TOKTIER_E_OOM"}

# every symbol declared in include/toktier.h
EXPORTS = ("toktier_load_vocab", "toktier_load_vocab_ex", "toktier_free_vocab", "toktier_vocab_info",
           "toktier_workspace_bytes", "toktier_workspace_bytes_ex",
           "toktier_encode_batch", "toktier_encode_batch_spans", "toktier_encode_batch_timed",
           "toktier_encode_batch_static",
           "toktier_pretokenize_batch", "toktier_repair_scratch_bytes", "toktier_repair_append",
           "toktier_plan_create", "toktier_plan_create_bucket", "toktier_plan_launch", "toktier_plan_free",
           "toktier_last_status", "toktier_status_string", "toktier_last_hip_error",
           "toktier_unicode_table_sha256")

# kernel launches of one encode call, in stream order (TOKTIER_K_* in toktier.h)
KERNELS = ("summary", "pieces", "tiles", "giant_seams", "bpe", "bpe_giant", "emit")


class RepairInfo(ctypes.Structure):
    """toktier_repair_info"""
    _fields_ = [("attempts", ctypes.c_uint32), ("window_chars", ctypes.c_uint32), ("spliced", ctypes.c_uint32),
                ("pad", ctypes.c_uint32), ("splice_byte", ctypes.c_uint64), ("fresh_tokens", ctypes.c_uint64)]


class ToktierError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        lib_ = _lib
        msg = STATUS.get(status, str(status))
        if lib_ is not None:
            msg += ": " + lib_.toktier_status_string(status).decode()
            if status == 6:
                msg += " (" + lib_.toktier_last_hip_error().decode() + ")"
        super().__init__(f"{what}: {msg}" if what else msg)


_lib = None


def lib():
    """Load libtoktier.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ToktierError(6, f"{LIB_PATH} is missing; run exact_bpe_tokenization_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.toktier_load_vocab.argtypes = [vp, u32, i32, ctypes.POINTER(vp)]
    L.toktier_load_vocab_ex.argtypes = [vp, u32, i32, u32, vp, vp, vp, u32, ctypes.POINTER(vp)]
    L.toktier_workspace_bytes_ex.argtypes = [vp, u64, u32, u64p]
    L.toktier_free_vocab.argtypes = [vp]
    L.toktier_vocab_info.argtypes = [vp, ctypes.POINTER(u32), ctypes.POINTER(i32)]
    L.toktier_workspace_bytes.argtypes = [u64, u32, u64p]
    L.toktier_encode_batch.argtypes = [vp, vp, vp, u32, u64, vp, u64, vp, vp, u64, vp, u64p]
    L.toktier_encode_batch_spans.argtypes = [vp, vp, vp, u32, u64, vp, vp, u64, vp, vp, u64, vp, u64p]
    L.toktier_encode_batch_timed.argtypes = [vp, vp, vp, u32, u64, vp, u64, vp, vp, u64, vp, u64p, vp, vp]
    L.toktier_encode_batch_static.argtypes = [vp, vp, vp, u32, u64, vp, u64, vp, vp, u64p]
    L.toktier_pretokenize_batch.argtypes = [vp, vp, vp, u32, u64, vp, u64, vp, u64, vp, u64p]
    L.toktier_last_status.argtypes = [vp, vp, u64p]
    L.toktier_plan_create.argtypes = [vp, vp, vp, u32, u64, vp, u64, vp, vp, vp, u64, vp, ctypes.POINTER(vp)]
    L.toktier_plan_create_bucket.argtypes = [vp, vp, vp, u32, u64, vp, vp, u64, vp, vp, vp, u64, vp,
                                             ctypes.POINTER(vp)]
    L.toktier_plan_launch.argtypes = [vp, vp, u64p]
    L.toktier_plan_free.argtypes = [vp]
    L.toktier_repair_scratch_bytes.argtypes = [vp, u64, u64p]
    L.toktier_repair_append.argtypes = [vp, vp, u64, u64, vp, vp, u64, vp, vp, u64, u64p, vp, u64, vp,
                                        ctypes.POINTER(RepairInfo)]
    for f in ("toktier_status_string",):
        getattr(L, f).argtypes = [i32]
        getattr(L, f).restype = ctypes.c_char_p
    for f in ("toktier_last_hip_error", "toktier_unicode_table_sha256"):
        getattr(L, f).argtypes = []
        getattr(L, f).restype = ctypes.c_char_p
    for f in EXPORTS:
        if getattr(L, f).restype is ctypes.c_int:
            getattr(L, f).restype = i32
    _lib = L
    return L


def _check(rc, what):
    if rc != 0:
        raise ToktierError(rc, what)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() else 0)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


class Vocab:
    """An immutable vocabulary handle (merge list + rule family) on the current device."""

    def __init__(self, handle, n_merges, family):
        self._h = handle
        self.n_merges = n_merges
        self.family = family

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            _check(lib().toktier_free_vocab(self._h), "toktier_free_vocab")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def toktier_load_vocab(merges, family):
    """merges: uint32 array-like of shape (n, 2), rank r joins (left, right) into 256 + r."""
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.uint32).reshape(-1, 2))
    fam = FAMILIES.get(family, family) if isinstance(family, str) else int(family)
    h = ctypes.c_void_p()
    rc = lib().toktier_load_vocab(m.ctypes.data_as(ctypes.c_void_p) if m.size else None, m.shape[0], fam,
                                  ctypes.byref(h))
    _check(rc, "toktier_load_vocab")
    return Vocab(h, m.shape[0], fam)


def toktier_load_vocab_ex(merges, family, flags=0, added=()):
    """toktier_load_vocab with vocabulary flags (TOKTIER_IGNORE_MERGES) and added tokens: `added` is a
    sequence of (literal bytes, ID) pairs."""
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.uint32).reshape(-1, 2))
    fam = FAMILIES.get(family, family) if isinstance(family, str) else int(family)
    lits = [bytes(b) for b, _ in added]
    blob = np.frombuffer(b"".join(lits) or b"\0", dtype=np.uint8).copy()
    offs = np.zeros(len(lits) + 1, dtype=np.uint32)
    offs[1:] = np.cumsum([len(b) for b in lits]) if lits else []
    ids = np.asarray([int(i) for _, i in added] or [0], dtype=np.uint32)
    h = ctypes.c_void_p()
    rc = lib().toktier_load_vocab_ex(m.ctypes.data_as(ctypes.c_void_p) if m.size else None, m.shape[0], fam,
                                     int(flags), blob.ctypes.data_as(ctypes.c_void_p),
                                     offs.ctypes.data_as(ctypes.c_void_p), ids.ctypes.data_as(ctypes.c_void_p),
                                     len(lits), ctypes.byref(h))
    _check(rc, "toktier_load_vocab_ex")
    return Vocab(h, m.shape[0], fam)


def toktier_free_vocab(vocab):
    vocab.close()


def toktier_vocab_info(vocab):
    n, f = ctypes.c_uint32(), ctypes.c_int()
    _check(lib().toktier_vocab_info(vocab.handle, ctypes.byref(n), ctypes.byref(f)), "toktier_vocab_info")
    return n.value, f.value


def toktier_workspace_bytes(total_bytes, n_docs):
    out = ctypes.c_uint64()
    _check(lib().toktier_workspace_bytes(int(total_bytes), int(n_docs), ctypes.byref(out)),
           "toktier_workspace_bytes")
    return out.value


def toktier_workspace_bytes_ex(vocab, total_bytes, n_docs):
    out = ctypes.c_uint64()
    _check(lib().toktier_workspace_bytes_ex(vocab.handle, int(total_bytes), int(n_docs), ctypes.byref(out)),
           "toktier_workspace_bytes_ex")
    return out.value


def toktier_encode_batch(vocab, data, offsets, out_ids, out_offsets, workspace, stream=None, sync=True):
    """data: uint8 device tensor; offsets: int64 device tensor [D+1] (read as uint64);
    out_ids: int32 device tensor (read as uint32) with >= len(data) elements; out_offsets: int64
    device tensor [D+1]; workspace: uint8 device tensor of toktier_workspace_bytes bytes.
    Returns the token count when sync is True, else None (the call is then fully asynchronous)."""
    n_tok = ctypes.c_uint64()
    rc = lib().toktier_encode_batch(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1, data.numel(),
                                    _ptr(out_ids), out_ids.numel(), _ptr(out_offsets), _ptr(workspace),
                                    workspace.numel(), _stream(stream), ctypes.byref(n_tok) if sync else None)
    _check(rc, "toktier_encode_batch")
    return n_tok.value if sync else None


def toktier_encode_batch_static(vocab, data, offsets, out_ids, out_offsets, stream=None, sync=True):
    """toktier_encode_batch on the library-owned scratch of the device (no workspace argument, no
    allocation in the call).  Returns the token count when sync is True, else None."""
    n_tok = ctypes.c_uint64()
    rc = lib().toktier_encode_batch_static(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1,
                                           data.numel(), _ptr(out_ids), out_ids.numel(), _ptr(out_offsets),
                                           _stream(stream), ctypes.byref(n_tok) if sync else None)
    _check(rc, "toktier_encode_batch_static")
    return n_tok.value if sync else None


def toktier_encode_batch_spans(vocab, data, offsets, out_ids, out_spans, out_offsets, workspace, stream=None,
                               sync=True):
    """toktier_encode_batch that also writes each token's source byte offset to out_spans (int32
    device tensor, read as uint32, >= len(data) elements)."""
    n_tok = ctypes.c_uint64()
    rc = lib().toktier_encode_batch_spans(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1,
                                          data.numel(), _ptr(out_ids), _ptr(out_spans), out_ids.numel(),
                                          _ptr(out_offsets), _ptr(workspace), workspace.numel(), _stream(stream),
                                          ctypes.byref(n_tok) if sync else None)
    _check(rc, "toktier_encode_batch_spans")
    return n_tok.value if sync else None


def toktier_encode_batch_timed(vocab, data, offsets, out_ids, out_offsets, workspace, events_before,
                               events_after, stream=None, sync=True):
    """toktier_encode_batch plus HIP events recorded around each kernel launch.  events_before /
    events_after: sequences of len(KERNELS) raw hipEvent_t handles (ints) or None."""
    arr_t = ctypes.c_void_p * len(KERNELS)
    eb = arr_t(*[e or None for e in events_before]) if events_before is not None else None
    ea = arr_t(*[e or None for e in events_after]) if events_after is not None else None
    n_tok = ctypes.c_uint64()
    rc = lib().toktier_encode_batch_timed(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1,
                                          data.numel(), _ptr(out_ids), out_ids.numel(), _ptr(out_offsets),
                                          _ptr(workspace), workspace.numel(), _stream(stream),
                                          ctypes.byref(n_tok) if sync else None, eb, ea)
    _check(rc, "toktier_encode_batch_timed")
    return n_tok.value if sync else None


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded (for per-kernel timing)."""

    def __init__(self, count):
        torch.cuda.init()
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(count):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise ToktierError(6, "hipEventCreate")
            self.handles.append(h.value)

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        if self._hip.hipEventSynchronize(ctypes.c_void_p(b)) != 0:
            raise ToktierError(6, "hipEventSynchronize")
        if self._hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise ToktierError(6, "hipEventElapsedTime")
        return out.value

    def __del__(self):
        for h in getattr(self, "handles", []):
            self._hip.hipEventDestroy(ctypes.c_void_p(h))


def toktier_pretokenize_batch(vocab, data, offsets, out_starts, workspace, stream=None):
    """Stage 1 only: writes piece start byte offsets (+ sentinel) to out_starts (int32 device
    tensor, >= len(data) + 1 elements) and returns the number of pieces."""
    n = ctypes.c_uint64()
    rc = lib().toktier_pretokenize_batch(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1,
                                         data.numel(), _ptr(out_starts), out_starts.numel(), _ptr(workspace),
                                         workspace.numel(), _stream(stream), ctypes.byref(n))
    _check(rc, "toktier_pretokenize_batch")
    return n.value


class Plan:
    """A captured encode (toktier_plan_create) bound to fixed device buffers; launch() replays it."""

    def __init__(self, vocab, data, offsets, out_ids, out_offsets, workspace, out_spans=None, stream=None):
        self.vocab = vocab
        self._keep = (data, offsets, out_ids, out_offsets, workspace, out_spans)
        h = ctypes.c_void_p()
        rc = lib().toktier_plan_create(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1, data.numel(),
                                       _ptr(out_ids), out_ids.numel(), _ptr(out_offsets), _ptr(out_spans),
                                       _ptr(workspace), workspace.numel(), _stream(stream), ctypes.byref(h))
        _check(rc, "toktier_plan_create")
        self.handle = h

    def launch(self, stream=None, sync=True):
        """Replay; returns the token count when sync is True (else None)."""
        n = ctypes.c_uint64()
        _check(lib().toktier_plan_launch(self.handle, _stream(stream), ctypes.byref(n) if sync else None),
               "toktier_plan_launch")
        return n.value if sync else None

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.toktier_plan_free(self.handle)
            self.handle = None


class BucketPlan(Plan):
    """A captured encode for a size bucket (toktier_plan_create_bucket): buffers sized for max_bytes /
    max_docs (data, offsets of max_docs + 1 entries), and a device tensor `sizes` (2 x int64: total
    bytes, documents) that every launch() reads to find the request it encodes."""

    def __init__(self, vocab, data, offsets, sizes, out_ids, out_offsets, workspace, out_spans=None, stream=None):
        self.vocab = vocab
        self._keep = (data, offsets, sizes, out_ids, out_offsets, workspace, out_spans)
        h = ctypes.c_void_p()
        rc = lib().toktier_plan_create_bucket(vocab.handle, _ptr(data), _ptr(offsets), offsets.numel() - 1,
                                              data.numel(), _ptr(sizes), _ptr(out_ids), out_ids.numel(),
                                              _ptr(out_offsets), _ptr(out_spans), _ptr(workspace), workspace.numel(),
                                              _stream(stream), ctypes.byref(h))
        _check(rc, "toktier_plan_create_bucket")
        self.handle = h


def toktier_repair_scratch_bytes(vocab, total_bytes):
    n = ctypes.c_uint64()
    _check(lib().toktier_repair_scratch_bytes(vocab.handle, total_bytes, ctypes.byref(n)),
           "toktier_repair_scratch_bytes")
    return n.value


def toktier_repair_append(vocab, text, len_a, cached_ids, cached_spans, scratch, stream=None):
    """Incremental repair of an append: text = A || B (host bytes), len_a = bytes of A, cached records
    of A (uint32 arrays).  Returns (ids uint32[T], spans uint32[T], info dict) for A || B."""
    tb = np.frombuffer(bytes(text), dtype=np.uint8)
    ci = np.ascontiguousarray(cached_ids, dtype=np.uint32)
    cs = np.ascontiguousarray(cached_spans, dtype=np.uint32)
    cap = max(tb.size, 1)
    out_ids = np.empty(cap, dtype=np.uint32)
    out_spans = np.empty(cap, dtype=np.uint32)
    k, info = _repair(vocab, tb, len_a, ci, cs, ci.size, out_ids, out_spans, scratch, stream)
    return out_ids[:k].copy(), out_spans[:k].copy(), info


def _repair(vocab, text, len_a, ci, cs, n_cached, out_ids, out_spans, scratch, stream):
    """One toktier_repair_append call on host numpy buffers (text uint8, records uint32)."""
    n = ctypes.c_uint64()
    info = RepairInfo()
    vp = ctypes.c_void_p
    rc = lib().toktier_repair_append(vocab.handle, vp(text.ctypes.data if text.size else None), len_a, text.size,
                                     vp(ci.ctypes.data), vp(cs.ctypes.data), n_cached,
                                     vp(out_ids.ctypes.data), vp(out_spans.ctypes.data), out_ids.size,
                                     ctypes.byref(n), _ptr(scratch), scratch.numel(), _stream(stream),
                                     ctypes.byref(info))
    _check(rc, "toktier_repair_append")
    return n.value, {f: getattr(info, f) for f, _ in RepairInfo._fields_ if f != "pad"}


class RepairSession:
    """A session's text and token records in host buffers that grow by doubling.  append(B) repairs
    the records of A into those of A || B in place (toktier_repair_append with the output arrays the
    cached ones), so a splice touches only the window's records and the bytes of B and of the window."""

    def __init__(self, tok, text=b""):
        raw = bytes(text)
        self.tok = tok
        self.n_bytes = len(raw)
        self._text = np.empty(max(2 * len(raw), 4096), dtype=np.uint8)
        self._text[:len(raw)] = np.frombuffer(raw, dtype=np.uint8)
        self._ids = np.empty(self._text.size, dtype=np.uint32)
        self._spans = np.empty(self._text.size, dtype=np.uint32)
        if raw:
            ids, _, spans = tok.encode(raw, spans=True)
        else:
            ids = spans = np.zeros(0, dtype=np.uint32)
        self.n_tokens = ids.size
        self._ids[:ids.size] = ids
        self._spans[:spans.size] = spans
        self._scratch = None
        self.last_info = None

    @property
    def text(self):
        return self._text[:self.n_bytes]

    @property
    def ids(self):
        return self._ids[:self.n_tokens]

    @property
    def spans(self):
        return self._spans[:self.n_tokens]

    def append(self, b):
        """Append the bytes b (A || B must be valid UTF-8); returns the repair's info dict."""
        add = np.frombuffer(bytes(b), dtype=np.uint8)
        total = self.n_bytes + add.size
        if total > self._text.size:
            cap = max(2 * self._text.size, total)
            for name in ("_text", "_ids", "_spans"):
                old = getattr(self, name)
                new = np.empty(cap, dtype=old.dtype)
                new[:old.size] = old
                setattr(self, name, new)
        self._text[self.n_bytes:total] = add
        vocab = self.tok.vocab
        with torch.cuda.device(self.tok.device):
            need = toktier_repair_scratch_bytes(vocab, total)
            if self._scratch is None or self._scratch.numel() < need:
                grow = need if self._scratch is None else max(need, 2 * self._scratch.numel())
                self._scratch = torch.empty(grow, dtype=torch.uint8, device=self.tok.device)
            k, info = _repair(vocab, self._text[:total], self.n_bytes, self._ids, self._spans, self.n_tokens,
                              self._ids, self._spans, self._scratch, None)
        self.n_bytes, self.n_tokens, self.last_info = total, k, info
        return info


def toktier_last_status(workspace, stream=None):
    n = ctypes.c_uint64()
    _check(lib().toktier_last_status(_ptr(workspace), _stream(stream), ctypes.byref(n)), "toktier_last_status")
    return n.value


def toktier_unicode_table_sha256():
    return lib().toktier_unicode_table_sha256().decode()


class Tokenizer:
    """Convenience wrapper: a vocabulary plus device buffers sized for the largest batch seen."""

    def __init__(self, merges, family, device="cuda:0", added=(), ignore_merges=False):
        self.device = torch.device(device)
        with torch.cuda.device(self.device):
            if added or ignore_merges:
                self.vocab = toktier_load_vocab_ex(merges, family, TOKTIER_IGNORE_MERGES if ignore_merges else 0,
                                                   added)
            else:
                self.vocab = toktier_load_vocab(merges, family)
        self._cap = -1
        self._docs = -1

    def _buffers(self, n, d):
        if n > self._cap or d > self._docs:
            self._cap, self._docs = max(n, self._cap), max(d, self._docs)
            ws = toktier_workspace_bytes_ex(self.vocab, self._cap, self._docs)
            self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
            self.out_ids = torch.empty(max(self._cap, 1), dtype=torch.int32, device=self.device)
            self.out_offsets = torch.empty(self._docs + 1, dtype=torch.int64, device=self.device)
            self.out_starts = torch.empty(self._cap + 1, dtype=torch.int32, device=self.device)

    def encode_device(self, data, offsets, stream=None, sync=True):
        """data/offsets already on the device.  Returns (ids view, offsets view, n_tokens)."""
        n, d = data.numel(), offsets.numel() - 1
        self._buffers(n, d)
        ws = self.workspace[: toktier_workspace_bytes_ex(self.vocab, n, d)]
        nt = toktier_encode_batch(self.vocab, data, offsets, self.out_ids[: max(n, 1)],
                                  self.out_offsets[: d + 1], ws, stream=stream, sync=sync)
        return self.out_ids, self.out_offsets[: d + 1], nt

    def encode(self, data: bytes, offsets=None, spans=False):
        """Host bytes in, host numpy arrays out: (ids uint32[T], out_offsets uint64[D+1]), plus the
        tokens' source byte offsets (uint32[T]) as a third array when spans is True."""
        arr = np.frombuffer(bytes(data), dtype=np.uint8) if len(data) else np.zeros(0, np.uint8)
        offs = np.asarray([0, arr.size] if offsets is None else offsets, dtype=np.int64)
        dd = torch.from_numpy(arr.copy()).to(self.device)
        do = torch.from_numpy(offs).to(self.device)
        if not spans:
            ids, oo, nt = self.encode_device(dd, do)
            return (ids[:nt].cpu().numpy().view(np.uint32).copy(), oo.cpu().numpy().astype(np.uint64))
        n, d = arr.size, offs.size - 1
        self._buffers(n, d)
        ws = self.workspace[: toktier_workspace_bytes_ex(self.vocab, n, d)]
        out_spans = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)
        nt = toktier_encode_batch_spans(self.vocab, dd, do, self.out_ids[: max(n, 1)], out_spans,
                                        self.out_offsets[: d + 1], ws)
        return (self.out_ids[:nt].cpu().numpy().view(np.uint32).copy(),
                self.out_offsets[: d + 1].cpu().numpy().astype(np.uint64),
                out_spans[:nt].cpu().numpy().view(np.uint32).copy())

    def repair_append(self, text: bytes, len_a, cached_ids, cached_spans):
        """Records of text = A || B from the cached records of A (toktier_repair_append)."""
        with torch.cuda.device(self.device):
            need = toktier_repair_scratch_bytes(self.vocab, len(text))
            if getattr(self, "_repair_scratch", None) is None or self._repair_scratch.numel() < need:
                self._repair_scratch = torch.empty(need, dtype=torch.uint8, device=self.device)
            return toktier_repair_append(self.vocab, text, len_a, cached_ids, cached_spans, self._repair_scratch)

    def pretokenize(self, data: bytes, offsets=None):
        arr = np.frombuffer(bytes(data), dtype=np.uint8) if len(data) else np.zeros(0, np.uint8)
        offs = np.asarray([0, arr.size] if offsets is None else offsets, dtype=np.int64)
        n, d = arr.size, offs.size - 1
        self._buffers(n, d)
        dd = torch.from_numpy(arr.copy()).to(self.device)
        do = torch.from_numpy(offs).to(self.device)
        ws = self.workspace[: toktier_workspace_bytes_ex(self.vocab, n, d)]
        np_ = toktier_pretokenize_batch(self.vocab, dd, do, self.out_starts[: n + 1], ws)
        return self.out_starts[: np_ + 1].cpu().numpy().view(np.uint32).astype(np.uint64)
