/*
 * toktier.h -- C ABI of the MI355X (gfx950) exact full-request tokenizer.
 *
 * The library tokenizes whole requests on one GPU the way a serial GPT-family tokenizer does, bit
 * for bit (TokTier: Exact Stateful CPU+GPU Tokenization for Agentic LLM Serving, arXiv 2607.29678;
 * GPU full-tokenization section and Figure 6):
 *   stage 1  regex-exact run decomposition of the pre-tokenizer: UTF-8 decode, character classes,
 *            maximal same-class runs and a per-character piece-start rule, all by parallel scans;
 *   stage 2  byte-level BPE of every piece independently, length-binned, merge ranks looked up in
 *            a hash table resident in device memory; then compaction of the IDs.
 * The concatenated IDs equal F = E* o G of the serial tokenizer (summary page, §2.2).
 *
 * Conventions shared by every entry point
 *   - Every function returns an int status: TOKTIER_OK (0) or one of the TOKTIER_E_* codes below;
 *     toktier_status_string() names it.  A failing call leaves no sticky HIP error behind.
 *   - "device" pointers are HIP device memory of the device that was current when the vocabulary
 *     was loaded; "host" pointers are ordinary process memory.
 *   - All device buffers passed in (input bytes, offsets, outputs, workspace) are owned by the
 *     caller.  The library owns only the vocabulary handle and the device tables behind it.
 *   - The encode and pretokenize calls allocate nothing: every scratch byte lives
 *     in the caller's workspace, and all their work is enqueued on the caller's stream.
 *   - Calls on different streams are independent when they use different workspaces; a workspace
 *     must not be shared by two calls in flight.  Results never depend on earlier calls.
 */
#ifndef TOKTIER_H
#define TOKTIER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct toktier_vocab toktier_vocab;   /* opaque; immutable after load */

/* Pre-tokenizer rule families (paper: the GPT-2, cl100k and o200k pattern lineages and the DeepSeek
 * family's three splitters in sequence; the exact alternatives are implemented by the oracle and
 * summarized below). */
enum {
    TOKTIER_GPT2 = 1,     /* contractions ('s 't 're 've 'm 'll 'd, lowercase), ' ?' + letters,
                             ' ?' + numbers, ' ?' + other, whitespace with lookahead */
    TOKTIER_CL100K = 2,   /* case-insensitive contractions, one non-letter prefix + letters, digits
                             grouped 1-3, other + trailing CR/LF, whitespace up to the last CR/LF */
    TOKTIER_O200K = 3,    /* cl100k plus a case-boundary letter rule (upper* lower+ | upper+ lower*),
                             marks inside words, contractions as word suffixes */
    TOKTIER_DEEPSEEK = 4  /* three splitters, each re-splitting every piece of the one before and
                             keeping unmatched stretches as pieces: digit groups of 1-3; runs of CJK
                             ideographs U+4E00-U+9FA5 and kana U+3040-U+30FF; then ASCII punctuation
                             + ASCII letters, an optional non-letter/punctuation/symbol/CR/LF
                             character + letters and marks, ' ?' + punctuation/symbols + trailing
                             CR/LF, and the cl100k whitespace rules */
};

enum {
    TOKTIER_OK = 0,
    TOKTIER_E_INVALID_ARG = 1,   /* null pointer, bad size, bad offsets, wrong device */
    TOKTIER_E_BAD_FAMILY = 2,    /* family not one of the enum values above */
    TOKTIER_E_BAD_MERGES = 3,    /* merge list rank-inconsistent, duplicated or too large */
    TOKTIER_E_INVALID_UTF8 = 4,  /* input bytes are not valid UTF-8 (detected on the device) */
    TOKTIER_E_CAPACITY = 5,      /* an output or the workspace is smaller than required */
    TOKTIER_E_HIP = 6,           /* a HIP runtime call failed (see toktier_last_hip_error) */
    TOKTIER_E_OOM = 7            /* host or device allocation failed while loading a vocabulary */
};

/* Largest merge count accepted: ranks stay below 2^20 (and IDs below 2^21). */
#define TOKTIER_MAX_MERGES ((1u << 20) - 1u)

/*
 * Load a merge list and its rule family; build the device tables on the current HIP device.
 *   merges    host, uint32[2 * n_merges]: merges[2r], merges[2r+1] are the (left, right) token IDs
 *             joined by merge rank r, which creates token ID 256 + r (byte-level BPE: IDs 0..255
 *             are the byte values).  Ranks are the list order; lower rank merges first.
 *   n_merges  0 .. TOKTIER_MAX_MERGES.
 *   family    TOKTIER_GPT2 / TOKTIER_CL100K / TOKTIER_O200K / TOKTIER_DEEPSEEK.
 *   out       receives the handle; unchanged on failure.
 * The list must be rank-consistent: left, right < 256 + r for every rank r, and no (left, right)
 * pair may appear twice.  The GPU merges every leftmost non-overlapping occurrence of the minimum
 * rank pair in one round (paper, GPU BPE paragraph); that schedule equals the serial textbook loop
 * exactly when the list is rank-consistent, so other lists are rejected with TOKTIER_E_BAD_MERGES.
 * Errors: E_INVALID_ARG, E_BAD_FAMILY, E_BAD_MERGES, E_OOM, E_HIP.  Synchronous.
 */
int toktier_load_vocab(const uint32_t *merges, uint32_t n_merges, int family, toktier_vocab **out);

/* Vocabulary flags of toktier_load_vocab_ex. */
enum {
    /* A piece whose bytes are some token's bytes becomes that token (the smallest such ID), without
     * the merge loop; other pieces merge as usual (paper, GPU BPE paragraph: the encoders configured
     * with ignore_merges, Llama 3 and gpt-oss, emit one ID for a piece that is a vocabulary entry). */
    TOKTIER_IGNORE_MERGES = 1
};

/* Limits on added tokens. */
#define TOKTIER_MAX_ADDED 65536u
#define TOKTIER_MAX_ADDED_BYTES 256u

/*
 * toktier_load_vocab with vocabulary flags and added tokens.
 *   flags          0 or TOKTIER_IGNORE_MERGES.  TOKTIER_IGNORE_MERGES needs every token to be at
 *                  most 256 bytes long (else E_INVALID_ARG).
 *   added_bytes    host, the added tokens' byte strings concatenated (may be NULL when n_added = 0).
 *   added_offsets  host, uint32[n_added + 1]: token k is added_bytes[added_offsets[k] ..
 *                  added_offsets[k+1]); added_offsets[0] = 0.
 *   added_ids      host, uint32[n_added]: the ID that token k is encoded as (any value; typically
 *                  256 + n_merges + k, or a model's reserved ID).
 *   n_added        0 .. TOKTIER_MAX_ADDED.
 * Added tokens (special tokens such as <|endoftext|>) are literals that the model reserves as single
 * IDs.  Before the family's pre-tokenizer runs, each document is scanned left to right for them,
 * leftmost-longest: where one or more literals start and end inside the document, the longest is
 * taken and the scan resumes after it (paper, implementation paragraph on added and special
 * tokens).  Each taken literal becomes its one ID; the text between literals is tokenized as if it
 * were a document of its own.  Every literal must be 1 .. TOKTIER_MAX_ADDED_BYTES bytes of valid
 * UTF-8, and no two may be equal (else E_INVALID_ARG).
 * Encoding with added tokens costs one host read of the literal count inside the encode call (that
 * call then synchronizes its stream even when out_n_tokens is NULL) and a larger workspace
 * (toktier_workspace_bytes_ex).  toktier_pretokenize_batch ignores added tokens.
 * Errors: as toktier_load_vocab.  Synchronous.
 */
int toktier_load_vocab_ex(const uint32_t *merges, uint32_t n_merges, int family, uint32_t flags,
                          const uint8_t *added_bytes, const uint32_t *added_offsets, const uint32_t *added_ids,
                          uint32_t n_added, toktier_vocab **out);

/* Release a handle and its device tables (synchronizes the device).  NULL is accepted. */
int toktier_free_vocab(toktier_vocab *v);

/* Vocabulary facts: number of merges and family (either pointer may be NULL). */
int toktier_vocab_info(const toktier_vocab *v, uint32_t *n_merges, int *family);

/*
 * Workspace size (bytes) that toktier_encode_batch / toktier_pretokenize_batch need for a batch of
 * total_bytes input bytes in n_docs documents.  Pure host arithmetic; no device call.
 * Errors: E_INVALID_ARG (total_bytes >= 2^32 - 1 or n_docs == 0xFFFFFFFF).
 */
int toktier_workspace_bytes(uint64_t total_bytes, uint32_t n_docs, uint64_t *out_bytes);

/*
 * Workspace size for encoding with vocabulary v: equal to toktier_workspace_bytes for a vocabulary
 * without added tokens; with added tokens it also holds the literal matches and the intermediate
 * output of the documents cut at the literals (up to about 80 bytes per input byte more when the
 * shortest literal is one byte long, less for longer ones).  Pure host arithmetic.
 * Errors: E_INVALID_ARG.
 */
int toktier_workspace_bytes_ex(const toktier_vocab *v, uint64_t total_bytes, uint32_t n_docs,
                               uint64_t *out_bytes);

/*
 * Tokenize a batch of documents (paper: multi-document batches are concatenated and runs are cut
 * at document boundaries).
 *   v            vocabulary handle (its device must be the current device).
 *   bytes        device, uint8[total_bytes]: the documents' UTF-8 text, concatenated.
 *   offsets      device, uint64[n_docs + 1]: document d is bytes[offsets[d], offsets[d+1]);
 *                offsets[0] = 0, non-decreasing, offsets[n_docs] = total_bytes.  Empty documents
 *                are allowed.  Every document is tokenized on its own (its first and last
 *                characters see the start and end of text).
 *   n_docs       number of documents (>= 1).
 *   total_bytes  < 2^32 - 1.
 *   out_ids      device, uint32[ids_capacity]: receives the token IDs of all documents in order.
 *   ids_capacity must be >= total_bytes (a token is never shorter than one byte, so this always
 *                suffices); otherwise TOKTIER_E_CAPACITY before any device work.
 *   out_offsets  device, uint64[n_docs + 1]: out_offsets[d] is the index in out_ids of document
 *                d's first token; out_offsets[n_docs] is the total token count.
 *   workspace    device scratch of at least toktier_workspace_bytes_ex(v, total_bytes, n_docs) bytes
 *                (= toktier_workspace_bytes(total_bytes, n_docs) for a vocabulary without added tokens),
 *                256-byte aligned; contents on entry do not matter.
 *   stream       hipStream_t (passed as void*); NULL means the default stream.
 *   out_n_tokens host; if non-NULL the call waits for the stream and stores the token count
 *                there (one device-to-host read).  If NULL the call returns right after enqueueing
 *                and the result (and any device-detected error) is only visible through
 *                out_offsets[n_docs] and a later call to toktier_last_status on the workspace.
 * Errors: E_INVALID_ARG, E_CAPACITY, E_HIP, and (only when out_n_tokens is non-NULL)
 *         E_INVALID_UTF8 / E_INVALID_ARG for bad bytes or offsets found on the device; the output
 *         contents are then unspecified.
 */
int toktier_encode_batch(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                         uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                         uint64_t ids_capacity, uint64_t *out_offsets, void *workspace,
                         uint64_t workspace_bytes, void *stream, uint64_t *out_n_tokens);

/*
 * toktier_encode_batch plus source byte spans of the tokens (paper: the session store keeps token
 * IDs with their source byte spans, session-state paragraph and Figure 14a; the GPU path it
 * describes returns IDs only, and its closing follow-ups list GPU span export).  A span is stored as
 * its start; the end is the next token's start.  Same kernels, same IDs and out_offsets; in addition
 *   out_spans    device, uint32[ids_capacity]: out_spans[i] is the batch byte offset of the first
 *                byte of token i.  Token i covers bytes [out_spans[i], out_spans[i + 1]), the last
 *                token of document d ending at offsets[d + 1]: the tokens of a document tile it, and
 *                each token's bytes are its vocabulary string.
 * Other arguments, ownership and errors as in toktier_encode_batch; out_spans may be NULL only when
 * total_bytes == 0 (E_INVALID_ARG otherwise).
 */
int toktier_encode_batch_spans(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                               uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                               uint32_t *out_spans, uint64_t ids_capacity, uint64_t *out_offsets,
                               void *workspace, uint64_t workspace_bytes, void *stream,
                               uint64_t *out_n_tokens);

/* Size of the library-owned scratch that toktier_encode_batch_static uses on each device. */
#define TOKTIER_STATIC_SCRATCH_BYTES (128ull << 20)

/*
 * toktier_encode_batch for callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace: the same
 * kernels run on a scratch array of TOKTIER_STATIC_SCRATCH_BYTES bytes that the library holds on
 * each device from the moment a vocabulary is first loaded there until the process ends.  The call
 * itself allocates nothing (no hipMalloc, hipFree, pinned host memory or other allocating routine).
 *   Arguments v, bytes, offsets, n_docs, total_bytes, out_ids, ids_capacity, out_offsets and
 *   stream as in toktier_encode_batch; the caller still owns the input and output buffers.
 *   out_n_tokens  host, may be NULL: if non-NULL, one blocking device-to-host copy of the control
 *                 block, then the token count is stored there and device-detected errors
 *                 (E_INVALID_UTF8, bad offsets) are returned; if NULL, the call only enqueues and the
 *                 count is out_offsets[n_docs].
 * Limits: toktier_workspace_bytes(total_bytes, n_docs) must not exceed TOKTIER_STATIC_SCRATCH_BYTES
 * (else E_CAPACITY before any device work; about 4.7 MB of input); vocabularies with added tokens are
 * rejected (E_INVALID_ARG).  Every call on one device shares that device's scratch, and each call
 * clears what it needs at its start: calls that overlap on one device (other streams, other host
 * threads) race and must be serialized by the caller.
 * Errors: E_INVALID_ARG, E_CAPACITY, E_HIP, and (with out_n_tokens) E_INVALID_UTF8.
 */
int toktier_encode_batch_static(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids, uint64_t ids_capacity,
                                uint64_t *out_offsets, void *stream, uint64_t *out_n_tokens);

/*
 * Stage 1 alone, for split-level checks (paper, exactness section: boundaries are compared apart
 * from IDs because an ID comparison can hide a wrong split).  Runs exactly the pre-tokenization
 * kernels that toktier_encode_batch runs and copies the piece starts out.
 *   out_piece_starts  device, uint32[starts_capacity]: byte offset of every piece start in input
 *                     order, followed by total_bytes as a sentinel.
 *   starts_capacity   must be >= total_bytes + 1.
 *   out_n_pieces      host, required: receives the number of pieces (synchronizes the stream).
 * Other arguments as in toktier_encode_batch.  Errors as in toktier_encode_batch.
 */
int toktier_pretokenize_batch(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                              uint32_t n_docs, uint64_t total_bytes, uint32_t *out_piece_starts,
                              uint64_t starts_capacity, void *workspace, uint64_t workspace_bytes,
                              void *stream, uint64_t *out_n_pieces);

/*
 * Status that the device recorded in a workspace during the last call that used it (waits for the
 * stream).  Lets callers of the asynchronous form (out_n_tokens == NULL) check for invalid input.
 *   out_n_tokens  host, may be NULL: token count of that call.
 */
int toktier_last_status(void *workspace, void *stream, uint64_t *out_n_tokens);

/* Kernel launches of one toktier_encode_batch call, in stream order (indices for the timed form).
 * An index may cover several launches of one step. */
enum {
    TOKTIER_K_SUMMARY = 0,    /* clear the control block and look-back flags; per tile: the        */
                              /* characters that decide the backward flags, the documents near it  */
    TOKTIER_K_PIECES,         /* UTF-8 decode + validation, automaton scan, piece starts per tile   */
    TOKTIER_K_TILES,          /* per 8 KiB tile: the starts' global places; single bytes and        */
                              /* whole-piece table lookups; the other pieces listed by length       */
    TOKTIER_K_GIANT_SEAMS,    /* pieces > 4096 bytes: seams no merge crosses, then chunks           */
    TOKTIER_K_BPE,            /* BPE of the listed pieces and chunks of <= 4096 bytes: lane per     */
                              /* piece (<= 32), a wavefront (<= 64), two elements per lane (<= 128),*/
                              /* a workgroup per piece (<= 4096)                                    */
    TOKTIER_K_BPE_GIANT,      /* BPE, one workgroup per longer chunk, sequence in device memory;    */
                              /* then (last workgroup) each giant piece's token count and its       */
                              /* chunks' output places                                              */
    TOKTIER_K_EMIT,           /* per tile: IDs placed by a scan of token counts, document offsets,  */
                              /* token spans                                                        */
    TOKTIER_K_COUNT
};

/*
 * Benchmark hook: exactly toktier_encode_batch, and in addition records caller-created HIP events
 * (hipEvent_t passed as void*) on the stream immediately before and after each kernel launch:
 * events_before[k] / events_after[k] for launch k in the enum above.  Either array, and any entry,
 * may be NULL (not recorded).  Launches that a batch does not need (e.g. every kernel after
 * TOKTIER_K_SUMMARY when total_bytes == 0) record nothing.  Errors as in toktier_encode_batch.
 */
int toktier_encode_batch_timed(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                               uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                               uint64_t ids_capacity, uint64_t *out_offsets, void *workspace,
                               uint64_t workspace_bytes, void *stream, uint64_t *out_n_tokens,
                               void *const *events_before, void *const *events_after);

/*
 * Incremental repair of an append (paper, incremental repair section and Figure 5).  A session
 * holds the records of its text A -- the token IDs of A and each token's source byte offset, as
 * toktier_encode_batch_spans returns them for A as one document -- and the next request is A || B.
 * The last w characters of A (w = 512, doubled at most five times) and B are encoded on the GPU as
 * a window; in the longest run of records where the cached and the window's records agree in
 * position and ID (at least two tokens, more bytes than the longest token) a splice point is
 * accepted when the pre-tokenizer automaton is synchronized before it inside the window (the
 * composition of its characters' transition maps sends every state to one state), the contexts up
 * to it are the same for A alone and for A || B, and a piece starts there.  The output is then A's
 * records before the splice point followed by the window's records from it; if every window
 * misses, the whole text is encoded.  Either way the output equals the encoding of A || B as one
 * document, records in the same form as the cached ones.
 *   v             vocabulary handle without added tokens (E_INVALID_ARG otherwise).
 * A splice reads only the window: B, A's last w characters and the cached records from the window's
 * start on (work of the order of the append plus the window, whatever the length of A); the rest of
 * A is read only by the full-text encode.
 *   text          host, uint8[len_total]: A || B, valid UTF-8; A ends on a character boundary.
 *                 Invalid bytes in B or in a window are reported; earlier bytes of A only when the
 *                 whole text is encoded.
 *   len_a         bytes of A (<= len_total < 2^32 - 1).
 *   cached_ids, cached_spans   host, uint32[n_cached]: the records of A (spans start at 0, strictly
 *                 increasing, below len_a; n_cached = 0 only when len_a = 0).  Not checked to be
 *                 the encoding of A (the caller keeps them from an earlier encode); the order is
 *                 checked from the window's start on.
 *   out_ids, out_spans   host, uint32[capacity]: the records of A || B; capacity >= len_total.  Either
 *                 exactly the cached arrays (then the records are repaired in place: those before
 *                 the splice point are not copied) or arrays that overlap neither them nor each
 *                 other (E_INVALID_ARG otherwise).
 *   out_n         host: number of records written.
 *   scratch       device, toktier_repair_scratch_bytes(v, len_total) bytes (text staging, records
 *                 and the encoder's workspace), 256-byte aligned.
 *   stream        hipStream_t (void*), NULL = default; the call synchronizes it.
 *   info          host, may be NULL: windows tried, last window size, whether it spliced and where.
 * Errors: E_INVALID_ARG, E_CAPACITY, E_INVALID_UTF8, E_HIP, and the encoder's errors.
 */
typedef struct {
    uint32_t attempts;       /* windows encoded (0: A is no longer than the first window) */
    uint32_t window_chars;   /* characters of A in the last window encoded */
    uint32_t spliced;        /* 1: cached records up to splice_byte + window records; 0: full encode */
    uint32_t pad;
    uint64_t splice_byte;    /* byte offset of the splice point when spliced */
    uint64_t fresh_tokens;   /* records taken from the GPU encode (window or full text) */
} toktier_repair_info;

int toktier_repair_scratch_bytes(const toktier_vocab *v, uint64_t total_bytes, uint64_t *out_bytes);

int toktier_repair_append(const toktier_vocab *v, const uint8_t *text, uint64_t len_a, uint64_t len_total,
                          const uint32_t *cached_ids, const uint32_t *cached_spans, uint64_t n_cached,
                          uint32_t *out_ids, uint32_t *out_spans, uint64_t capacity, uint64_t *out_n,
                          void *scratch, uint64_t scratch_bytes, void *stream, toktier_repair_info *info);

/*
 * Plans: the kernel chain of toktier_encode_batch (or of the span form when out_spans is non-NULL)
 * captured once as a HIP graph for fixed device buffers and sizes, then replayed (paper, latency
 * paragraph: counts stay on the device and a CUDA graph removes the host from the chain).  A replay
 * encodes whatever the bytes and offsets buffers hold at that time (same total_bytes and n_docs);
 * nothing is cached between replays.  Arguments as in toktier_encode_batch(_spans); the buffers, and
 * the vocabulary (its device tables are bound into the graph), must outlive the plan: free every
 * plan before its vocabulary.  Vocabularies with added tokens are rejected (E_INVALID_ARG): their
 * literal pass reads a count on the host.  Plans sharing a workspace must not run at the same time.
 *   toktier_plan_create  captures and uploads the graph (on `stream`; no kernel runs).
 *   toktier_plan_launch  replays it on `stream`; out_n_tokens as in toktier_encode_batch (NULL: no
 *                        wait; the count and device-detected errors then come from
 *                        toktier_last_status on the workspace).
 *   toktier_plan_free    releases the graph (NULL is a no-op).
 * Errors: those of toktier_encode_batch, E_HIP for graph failures, E_OOM.
 */
typedef struct toktier_plan toktier_plan;
int toktier_plan_create(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets, uint32_t n_docs,
                        uint64_t total_bytes, uint32_t *out_ids, uint64_t ids_capacity, uint64_t *out_offsets,
                        uint32_t *out_spans, void *workspace, uint64_t workspace_bytes, void *stream,
                        toktier_plan **out);
/*
 * A plan over a size bucket (paper, latency paragraph: the chain is captured as a graph for a small
 * set of input-size buckets).  The graph is captured once for at most max_bytes input bytes and
 * max_docs documents; every replay encodes the request whose sizes the device buffer `sizes` holds at
 * that time -- sizes[0] total bytes, sizes[1] documents (1 .. max_docs) -- from bytes[0 .. sizes[0]) and
 * offsets[0 .. sizes[1]], writing out_offsets[0 .. sizes[1]] and the IDs (spans).  So one plan serves
 * any request up to its bucket, and the sizes can be written by the host or by earlier device work.
 *   bytes, offsets, out_*, workspace  as in toktier_plan_create, sized for the bucket (the workspace:
 *                 toktier_workspace_bytes(max_bytes, max_docs)); ids_capacity >= max_bytes.
 *   sizes         device, 2 x uint64; read by every replay, not at creation.
 * A replay whose sizes exceed the bucket, or name no document, encodes nothing and reports
 * E_INVALID_ARG (through toktier_plan_launch's count, or toktier_last_status).  Replay with
 * toktier_plan_launch, release with toktier_plan_free.  Errors at creation: those of
 * toktier_plan_create, E_INVALID_ARG for a NULL sizes pointer or max_bytes == 0.
 */
int toktier_plan_create_bucket(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                               uint32_t max_docs, uint64_t max_bytes, const uint64_t *sizes, uint32_t *out_ids,
                               uint64_t ids_capacity, uint64_t *out_offsets, uint32_t *out_spans, void *workspace,
                               uint64_t workspace_bytes, void *stream, toktier_plan **out);
int toktier_plan_launch(toktier_plan *p, void *stream, uint64_t *out_n_tokens);
int toktier_plan_free(toktier_plan *p);

/* Static English text for a status code. */
const char *toktier_status_string(int status);

/* Text of the last HIP error seen by this thread inside the library (empty if none). */
const char *toktier_last_hip_error(void);

/* SHA-256 (hex) of the library's frozen Unicode category table. */
const char *toktier_unicode_table_sha256(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKTIER_H */
