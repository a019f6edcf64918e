// internal.h -- shared definitions of the gfx950 tokenizer library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

// ---------------------------------------------------------------------------------------------
// stage-1 geometry: one workgroup per 8 KiB tile, 16 input bytes per thread
constexpr int PRE_THREADS = 512;
constexpr int PRE_CHUNK = 16;
constexpr int TILE = PRE_THREADS * PRE_CHUNK;  // 8192
constexpr int HALO = 16;                       // character codes computed past a tile
constexpr int RAW_LEAD = 4, RAW_TAIL = 24;     // raw bytes kept before / after a tile

// token-offset scan: one workgroup per 4096 pieces

// giant pieces are cut at seams that no merge can cross: about every GCH bytes where such seams are
// common, and at both ends of stretches longer than GCH without one
constexpr uint32_t GCH = 48;
// BPE list entries: a piece index, or CHUNK_ITEM | index into the chunk table
constexpr uint32_t CHUNK_ITEM = 1u << 31;

// BPE length bins (piece bytes): lane <= LANE_MAX < wave <= WAVE_MAX < block <= BLOCK_MAX < giant
constexpr int LANE_MAX = 64;      // lane kernels: <= 16 (by 8, 12, 16), 17..32 and 33..64 bytes
constexpr int SEG2_MAX = 128;     // one wavefront, two elements per lane: 65..128 bytes
constexpr int TABLE_MAX = 32;     // whole-piece tables hold pieces of 2..32 bytes
constexpr int WAVE_MAX = 1024;
constexpr int BLOCK_MAX = 4096;
constexpr int BLOCK_THREADS = 256;
// pieces of up to SHORT_MAX bytes are encoded by the tile encoder (their bytes lie in its window);
// longer ones are listed by the pieces kernel and encoded before it
constexpr int SHORT_MAX = SEG2_MAX;
constexpr int GIANT_THREADS = 1024;

// ---------------------------------------------------------------------------------------------
// per-byte character code written by the classify kernel
//   bits 0-2 category; bit 3 CR or LF; bit 4 U+0020 (whitespace) or punctuation / symbol (other
//   characters); bits 5-6 contraction length code at an apostrophe (0 none, 1 two chars "'x", 2
//   three chars "'xy"), in the DeepSeek-style family instead bit 5 ASCII letter or ASCII
//   punctuation / symbol and bit 6 a code point of the CJK ranges of its second splitter; bit 7
//   first char of a document
enum : uint8_t { CAT_LU = 0, CAT_LL = 1, CAT_LO = 2, CAT_N = 3, CAT_W = 4, CAT_M = 5, CAT_O = 6,
                 CAT_CONT = 7 };
constexpr uint8_t CC_CRLF = 8, CC_SP = 16, CC_PS = 16, CC_CONTR_SHIFT = 5, CC_DOC = 128;
constexpr uint8_t CC_DS_ASCII = 32, CC_DS_CJK = 64;
constexpr uint8_t CC_EOF = 0xFF;   // placed past the end of the batch

// ---------------------------------------------------------------------------------------------
// character codes -> automaton context parts (the pieces kernel and the host-side repair check)

// DeepSeek-style bits of a character's code (code = its category bits, with CC_PS): ASCII letter or
// ASCII punctuation / symbol (the first character of that family's punctuation-word alternative),
// and a code point of its second splitter's CJK ranges (ideographs U+4E00..U+9FA5, hiragana and
// katakana U+3040..U+30FF)
__host__ __device__ __forceinline__ uint32_t ds_bits(uint32_t cp, uint32_t code)
{
    const uint32_t cat = code & 7u;
    const bool ascii = cp < 0x80u && (cat <= CAT_LO || (cat == CAT_O && (code & CC_PS)));
    const bool cjk = cp - 0x4E00u <= 0x9FA5u - 0x4E00u || cp - 0x3040u <= 0x30FFu - 0x3040u;
    return (ascii ? CC_DS_ASCII : 0u) | (cjk ? CC_DS_CJK : 0u);
}

// self code of a character (13 values) from its byte code and its NA flag, without branches:
// LU 0, LL 1, LO 2, N 3, M 4, other 5 (6, 7 with a one- or two-letter contraction after an
// apostrophe), whitespace 8 + 2 (space) + 1 (NA), CR/LF 12
__host__ __device__ __forceinline__ uint32_t self_code(uint32_t code, bool na)
{
    const uint32_t cat = code & 7u;
    const uint32_t base = (0x05483210u >> (4u * cat)) & 15u;
    const uint32_t other = base + ((code >> CC_CONTR_SHIFT) & 3u);
    const uint32_t ws = (code & CC_CRLF) ? 12u : 8u + ((code & CC_SP) ? 2u : 0u) + (na ? 1u : 0u);
    return cat == CAT_W ? ws : (cat == CAT_O ? other : base);
}

// next-character code: letter 0, N 1, W 2, M 3, other 4, end of document or batch 5
__host__ __device__ __forceinline__ uint32_t next_code(uint32_t code)
{
    return (code & CC_DOC) ? 5u : (0x44321000u >> (4u * (code & 7u))) & 15u;   // CC_EOF has CC_DOC set
}

// DeepSeek style (16 self codes): ASCII letter 0, other letter 1, CJK-range letter 2, mark 3,
// CJK-range mark 4, ASCII punctuation / symbol 5, other punctuation / symbol 6, CJK-range one 7,
// other character 8, CJK-range other 9, number 10, whitespace 11 + 2 (space) + 1 (NA), CR/LF 15
__host__ __device__ __forceinline__ uint32_t self_code_ds(uint32_t code)
{
    const uint32_t cat = code & 7u;
    const bool cjk = code & CC_DS_CJK, asc = code & CC_DS_ASCII, ps = code & CC_PS;
    if (cat <= CAT_LO) return asc ? 0u : (cjk ? 2u : 1u);
    if (cat == CAT_M) return cjk ? 4u : 3u;
    if (cat == CAT_O) return ps ? (asc ? 5u : (cjk ? 7u : 6u)) : (cjk ? 9u : 8u);
    if (cat == CAT_N) return 10u;
    return (code & CC_CRLF) ? 15u : ((code & CC_SP) ? 13u : 11u);
}

// DeepSeek style next-character code: ASCII letter 0, letter or mark 1, CJK-range letter or mark 2,
// punctuation / symbol 3, CJK-range one 4, whitespace 5, other 6, CJK-range other 7, number 8, end
// of document or batch 9
__host__ __device__ __forceinline__ uint32_t next_code_ds(uint32_t code)
{
    const uint32_t cat = code & 7u;
    const bool cjk = code & CC_DS_CJK;
    if ((code & CC_DOC) || cat == CAT_CONT) return 9u;
    if (cat <= CAT_LO || cat == CAT_M) return (code & CC_DS_ASCII) ? 0u : (cjk ? 2u : 1u);
    if (cat == CAT_O) return (code & CC_PS) ? (cjk ? 4u : 3u) : (cjk ? 7u : 6u);
    return cat == CAT_W ? 5u : 8u;
}

// ---------------------------------------------------------------------------------------------
// pre-tokenizer automaton: the state before a character says what the running match expects
enum : int { S_ST = 0, S_LRUN, S_NALL, S_N1, S_N2, S_ORUN, S_ORNL, S_ONL, S_WNL, S_WNS, S_C1,
             S_C2, S_LA, S_LB, S_LEND, NSTATES };
static_assert(NSTATES == 15, "a transition map holds one byte per state in 16 bytes, byte 15 free");

// character context: self code (13) x first-of-document (2) x next-char code (6) x flag (2);
// DeepSeek style: self code (16) x first-of-document (2) x next-char code (10), no flag
constexpr int NSELF = 13, NNEXT = 6, NCTX = NSELF * 2 * NNEXT * 2;
constexpr int DS_NSELF = 16, DS_NNEXT = 10, DS_NCTX = DS_NSELF * 2 * DS_NNEXT;
constexpr int NCTX_MAX = NCTX > DS_NCTX ? NCTX : DS_NCTX;

// ---------------------------------------------------------------------------------------------
// merge tables.  A merge's rank word (rkx) is rank << 2 | L << 1 | R, where L (R) is set when the
// token the merge creates is the left (right) operand of some merge: a pair (x, y) can only have a
// rank when x is some merge's left operand and y some merge's right operand, so the BPE kernels skip
// the lookups of the pairs that fail this test.  Pair hash slot: bits 63..22 = (left << 21 | right),
// bits 21..0 = rkx.  Ranks stay below 2^20, token IDs below 2^21.
constexpr uint32_t NO_RANK = 0xFFFFFFFFu;
constexpr uint32_t NO_PIECE = 0xFFFFFFFFu;
constexpr uint64_t EMPTY_SLOT = ~0ull;
constexpr uint32_t RKX_MASK = 0x3FFFFFu;
__host__ __device__ __forceinline__ uint32_t rkx_rank(uint32_t x) { return x == NO_RANK ? NO_RANK : x >> 2; }
// a sequence element of the short BPE units: token ID | L << 31 | R << 30 (bytes carry both)
constexpr uint32_t ID_MASK = 0x3FFFFFFFu, EL_L = 1u << 31, EL_R = 1u << 30, EL_BYTE = EL_L | EL_R;
// the element a merge of rank word x creates
__device__ __forceinline__ uint32_t merged_element(uint32_t x) { return (256u + (x >> 2)) | ((x & 3u) << 30); }
// can the pair of elements (a, b) have a rank?
__device__ __forceinline__ bool may_merge(uint32_t a, uint32_t b) { return (a & EL_L) && (b & EL_R); }

constexpr int FAMILY_GPT2 = 1, FAMILY_O200K = 3, FAMILY_DEEPSEEK = 4;   // the family codes of the public header

struct DevVocab {
    const uint32_t *r2;       // 65536 byte-pair rank words (rkx), NO_RANK for no merge
    const uint64_t *slots;    // pair table: 8-byte slots (left << 21 | right) << 22 | rkx, two-choice cuckoo
    const uint32_t *merges;   // 2 * n_merges (left, right)
    const uint4 *fmap16;      // NCTX (DeepSeek style: DS_NCTX) transition maps, one byte per state s (bytes 0..14):
                              //   bits 0-3 the next state, bit 4 set when a piece starts here in s
    // whole-piece tables: pieces whose BPE result is one token (NULL while they are being built)
    // (two-choice cuckoo tables: every key is in one of its two candidate slots, both read at once)
    const uint4 *wa;          // 2..7 bytes: {key lo, key hi, id, 0}, key = bytes | len << 56; key 0 = empty
    const uint4 *wb;          // 8..32 bytes: 3 x uint4 = {k0, k1}, {k2, k3}, {len, id, 0, 0}; len 0 = empty
    const uint4 *hot;         // HOT_SLOTS entries of the short table, the lowest IDs: 2-way sets, copied to LDS
    // every token's byte string: bytes, offsets, and a hash from (string) to token ID, used to find
    // seams no merge can cross in giant pieces (NULL when the longest token exceeds STR_LMAX bytes)
    const uint8_t *tok_bytes;
    const uint32_t *tok_off;  // 256 + n_merges + 1 offsets into tok_bytes
    const uint32_t *tok_len;  // byte length of every token (for token spans; always present)
    const uint4 *str;         // {key lo, key hi, id, len}; len 0 = empty slot
    uint64_t pseed, wseed, bseed;   // seeds of the candidate-slot hashes (pairs, wa, wb)
    uint32_t slot_cap, wa_cap, wb_cap;
    uint32_t str_mask, str_shift, lmax;
    uint32_t n_merges;
    int family;
    uint32_t flags;           // VF_* below
};

// vocabulary flags: VF_IGNORE_MERGES -- the whole-piece tables hold every token's byte string (the
// smallest ID of each), and pieces longer than TABLE_MAX are looked up in the token string hash
constexpr uint32_t VF_IGNORE_MERGES = 1u;

// token string hash: H(s) = sum s_i P^(len-1-i) mod 2^64, so H(s c) = H(s) P + c and
// H(c s) = c P^len + H(s); the key mixes in the length
constexpr uint64_t STR_P = 0x100000001B3ull;
constexpr uint32_t STR_LMAX = 256;
__host__ __device__ __forceinline__ uint64_t str_key(uint64_t h, uint32_t len)
{
    return h ^ ((uint64_t)len * 0x9E3779B97F4A7C15ull);
}
__host__ __device__ __forceinline__ uint64_t str_slot(uint64_t key, uint32_t shift)
{
    return (key * 0xD6E8FEB86659FD93ull) >> shift;
}

// whole-piece keys
constexpr uint32_t WA_MAX = 7;

// The hot part of the short whole-piece table: the 2..7-byte entries with the lowest token IDs (the
// first merges are the most frequent pairs of the training text, and their tokens dominate real
// text) in HOT_SLOTS / 2 sets of two, small enough for every tile workgroup to keep in LDS.
constexpr uint32_t HOT_SLOTS = 1024;
__host__ __device__ __forceinline__ uint32_t hot_set(uint64_t key)
{
    return (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> 55);   // HOT_SLOTS / 2 = 512 sets
}

// Two-choice cuckoo hashing: a 64-bit digest of the key, mixed with the table's seed, gives two
// candidate slots in [0, cap) (its two 32-bit halves scaled to cap).  A lookup reads both slots at
// once, so it always costs one round trip, and the tables stay small (under half full).
__host__ __device__ __forceinline__ uint64_t ck_mix(uint64_t x)
{
    x ^= x >> 33;
    x *= 0xFF51AFD7ED558CCDull;
    x ^= x >> 33;
    x *= 0xC4CEB9FE1A85EC53ull;
    x ^= x >> 33;
    return x;
}
__host__ __device__ __forceinline__ void ck_slots(uint64_t digest, uint64_t seed, uint32_t cap, uint32_t &i1,
                                                  uint32_t &i2)
{
    const uint64_t h = ck_mix(digest ^ seed);
    i1 = (uint32_t)(((h & 0xFFFFFFFFull) * cap) >> 32);
    i2 = (uint32_t)(((h >> 32) * cap) >> 32);
}
// digest of an 8..32-byte key (its four words and length)
__host__ __device__ __forceinline__ uint64_t wb_digest(uint64_t k0, uint64_t k1, uint64_t k2, uint64_t k3,
                                                      uint32_t len)
{
    uint64_t h = k0 * 0x9E3779B97F4A7C15ull;
    h ^= (k1 + 0x632BE59BD9B4E019ull) * 0xC2B2AE3D27D4EB4Full;
    h ^= (k2 + 0x85EBCA77C2B2AE63ull) * 0x165667B19E3779F9ull;
    h ^= (k3 + len) * 0x27D4EB2F165667C5ull;
    return h;
}

// ---------------------------------------------------------------------------------------------
// wavefront primitives on DPP moves

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves (no LDS round trips): a
// Hillis-Steele scan inside each row of 16 lanes (row_shr 1, 2, 4, 8), then row 0's total added to
// row 1 and row 2's to row 3 (row_bcast:15), then rows 0-1's total to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// The value of the next lane (lane 63: 0), by a DPP wavefront shift.
__device__ __forceinline__ uint32_t wave_next(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x130, 0xF, 0xF, true);   // wave_shl:1
}

// Maximum over the wavefront (wavefront-uniform result).
__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xF, 0xF, false));   // row_ror:1
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xF, 0xF, false));   // row_ror:2
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false));   // row_ror:4
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false));   // row_ror:8
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return max(max(a, b), max(c, d));
}

// Minimum over each row of 16 lanes, in every lane of the row (DPP row rotations 1, 2, 4, 8).
__device__ __forceinline__ uint32_t row_min16(uint32_t x)
{
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xF, 0xF, false));   // row_ror:1
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xF, 0xF, false));   // row_ror:2
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false));   // row_ror:4
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false));   // row_ror:8
    return x;
}

// Minimum over the wavefront (wavefront-uniform result): row minima, then the four rows' lanes 0.
__device__ __forceinline__ uint32_t wave_min(uint32_t x)
{
    x = row_min16(x);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return min(min(a, b), min(c, d));
}

// ---------------------------------------------------------------------------------------------
// decoupled look-back helpers (one wavefront reads a window of 64 predecessor flags at once)

__device__ __forceinline__ uint64_t ld_flag(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// First index i in [0, n) whose entry satisfies pred (n if none), for a predicate that is false
// then true along the sorted array.  Called by a whole wavefront: each step probes 64 evenly spaced
// entries, so a search costs about log64(n) + 1 dependent loads.
template <typename T, typename Pred>
__device__ __forceinline__ uint32_t wave_partition_point(const T *a, uint32_t n, Pred pred)
{
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t lo = 0, hi = n;   // the answer lies in [lo, hi]
    while (hi - lo > 64) {
        const uint32_t step = (hi - lo + 63) / 64;
        const uint32_t idx = lo + lane * step;
        const uint64_t t = __ballot(idx >= hi || pred(a[idx]));
        if (t == 0) {          // every probe is before the answer
            lo = lo + 63 * step + 1;
            continue;
        }
        const uint32_t k = (uint32_t)__ffsll((unsigned long long)t) - 1u;
        const uint32_t nlo = k == 0 ? lo : lo + (k - 1) * step + 1;
        hi = min(hi, lo + k * step);
        lo = nlo;
    }
    const uint32_t idx = lo + lane;
    const uint64_t t = __ballot(idx >= hi || pred(a[idx]));
    return t ? lo + (uint32_t)__ffsll((unsigned long long)t) - 1u : hi;
}

template <typename T>
__device__ __forceinline__ uint32_t wave_lower_bound(const T *a, uint32_t n, T x)
{
    return wave_partition_point(a, n, [x](T v) { return v >= x; });
}

template <typename T>
__device__ __forceinline__ uint32_t wave_upper_bound(const T *a, uint32_t n, T x)
{
    return wave_partition_point(a, n, [x](T v) { return v > x; });
}

// rank word held by a pair-table slot for key, NO_RANK if neither candidate holds it (an empty slot is
// all ones: its key field exceeds every (left << 21 | right))
__device__ __forceinline__ uint32_t slot_rkx(uint64_t s0, uint64_t s1, uint64_t key)
{
    return (s0 >> 22) == key ? (uint32_t)(s0 & RKX_MASK) : ((s1 >> 22) == key ? (uint32_t)(s1 & RKX_MASK) : NO_RANK);
}

// Rank words of two pairs, each with an operand >= 256 (not byte pairs), looked up only where need0 /
// need1: all candidate slots read at once, so a merge step that needs both waits for one round trip
__device__ __forceinline__ void pair_rkx2(const DevVocab &v, uint32_t a0, uint32_t b0, bool need0, uint32_t a1,
                                          uint32_t b1, bool need1, uint32_t &r0, uint32_t &r1)
{
    const uint64_t k0 = ((uint64_t)a0 << 21) | b0, k1 = ((uint64_t)a1 << 21) | b1;
    uint32_t i0, j0, i1, j1;
    ck_slots(k0, v.pseed, v.slot_cap, i0, j0);
    ck_slots(k1, v.pseed, v.slot_cap, i1, j1);
    uint64_t s0 = EMPTY_SLOT, t0 = EMPTY_SLOT, s1 = EMPTY_SLOT, t1 = EMPTY_SLOT;
    if (need0) {
        s0 = v.slots[i0];
        t0 = v.slots[j0];
    }
    if (need1) {
        s1 = v.slots[i1];
        t1 = v.slots[j1];
    }
    r0 = slot_rkx(s0, t0, k0);
    r1 = slot_rkx(s1, t1, k1);
}

// Rank word of the pair (a, b), NO_RANK if no merge joins them: byte pairs from the dense table, the
// others from the pair table (both candidate slots in one round trip)
__device__ __forceinline__ uint32_t pair_rkx(const DevVocab &v, uint32_t a, uint32_t b)
{
    if ((a | b) < 256u) return __ldg(v.r2 + ((a << 8) | b));
    const uint64_t key = ((uint64_t)a << 21) | b;
    uint32_t i, j;
    ck_slots(key, v.pseed, v.slot_cap, i, j);
    return slot_rkx(v.slots[i], v.slots[j], key);
}

__device__ __forceinline__ uint32_t pair_rank(const DevVocab &v, uint32_t a, uint32_t b)
{
    return rkx_rank(pair_rkx(v, a, b));
}

// the same for two elements (ID | L | R bits): NO_RANK without a lookup when the bits rule a merge out
__device__ __forceinline__ uint32_t element_rkx(const DevVocab &v, uint32_t a, uint32_t b)
{
    return may_merge(a, b) ? pair_rkx(v, a & ID_MASK, b & ID_MASK) : NO_RANK;
}

// calls f(id) for every token whose byte string equals s[0, len); the table key was computed by the
// caller as str_key(H(s), len)
template <typename F>
__device__ __forceinline__ void str_find(const DevVocab &v, const uint8_t *s, uint32_t len, uint64_t key, F f)
{
    uint32_t i = (uint32_t)str_slot(key, v.str_shift);
    for (;;) {
        const uint4 e = v.str[i];
        if (e.w == 0) return;
        if (e.w == len && ((uint64_t)e.x | ((uint64_t)e.y << 32)) == key) {
            const uint8_t *t = v.tok_bytes + v.tok_off[e.z];
            bool eq = true;
            for (uint32_t k = 0; k < len && eq; ++k) eq = t[k] == s[k];
            if (eq) f(e.z);
        }
        i = (i + 1) & v.str_mask;
    }
}

// ignore_merges: the smallest ID of a token whose bytes are s[0, len) (len up to the longest token),
// NO_PIECE if there is none
__device__ __forceinline__ uint32_t whole_token(const DevVocab &v, const uint8_t *s, uint32_t len)
{
    uint64_t h = 0;
    for (uint32_t k = 0; k < len; ++k) h = h * STR_P + s[k];
    uint32_t best = NO_PIECE;
    str_find(v, s, len, str_key(h, len), [&](uint32_t id) { best = min(best, id); });
    return best;
}

// ---------------------------------------------------------------------------------------------
// device control block at the start of the workspace (cleared by the init kernel)
enum : uint32_t { ST_BAD_UTF8 = 1, ST_BAD_OFFSETS = 2 };

struct Ctrl {
    uint32_t status;
    uint32_t tile_ctr_pre;     // dynamic tile ids for the piece kernel
    uint32_t n_pieces;
    uint32_t n_tokens;
    uint32_t bin_count[3];     // wave, block, giant bins
    uint32_t miss_count[6];    // pieces left for BPE: <= 8, 9..12, 13..16, 17..32, 33..64, 65..128 bytes
    uint32_t n_chunks;         // chunk slots reserved for giant pieces
    uint32_t done_giant;       // workgroups of k_bpe_giant done (the last one joins the chunks)
    uint32_t pad[49];
};
static_assert(sizeof(Ctrl) == 256, "control block is 256 bytes");

// ---------------------------------------------------------------------------------------------
// workspace layout for n input bytes
struct Layout {
    uint64_t ctrl, cc, tbwd, tdoc, twin, tflag_state, tcnt, tfirst, gsum, tcount, tsb, tbase, pstart, pval, tokoff, scratch,
        bin_wave, bin_block, bin_giant, miss[6], g_ids, g_rank_a, g_rank_b, tspill, prs, cstart, clen, ccount, gc0, gnc, gdone, gsafe,
        cpiece, total;
    uint32_t n_tiles, cap_wave, cap_block, cap_giant, cap_chunks, n_safe_words;
    // a plan captured for a size bucket: the request's sizes are read from dsz (device: total bytes,
    // document count) when it is replayed, at most cap_n bytes and cap_docs documents; else NULL
    const uint64_t *dsz;
    uint64_t cap_n;
    uint32_t cap_docs;
};

inline uint64_t align256(uint64_t x) { return (x + 255) & ~255ull; }

inline Layout make_layout(uint64_t n)
{
    Layout L;
    L.n_tiles = (uint32_t)((n + TILE - 1) / TILE);
    L.dsz = nullptr;
    L.cap_n = n;
    L.cap_docs = 0;
    L.cap_wave = (uint32_t)(n / (LANE_MAX + 1) + 1);
    L.cap_block = (uint32_t)(n / (WAVE_MAX + 1) + 1);
    L.cap_giant = (uint32_t)(n / (BLOCK_MAX + 1) + 1);
    L.cap_chunks = (uint32_t)(2 * (n / GCH) + 2ull * L.cap_giant + 2);
    L.n_safe_words = (uint32_t)(n / 32 + n / 4096 + 4);
    uint64_t o = 0;
    L.ctrl = o;        o += align256(sizeof(Ctrl));
    L.cc = o;
    L.tbwd = o;        o += align256((uint64_t)L.n_tiles + 1);
    L.tdoc = o;        o += align256(16ull * L.n_tiles);
    L.twin = o;        o += align256(4ull * L.n_tiles);         // entry state of the next tile, if fixed
    L.tflag_state = o; o += align256(16ull * L.n_tiles);
    L.tcnt = o;        o += align256(4ull * L.n_tiles);         // pieces starting in each tile
    L.tfirst = o;      o += align256(4ull * L.n_tiles);         // each tile's first piece start
    L.gsum = o;        o += align256(4ull * (L.n_tiles / 64 + 1));  // pieces summed over 64 tiles
    L.tcount = o;      o += align256(4ull * (L.n_tiles + 1));   // tokens of the pieces starting in each tile
    L.tsb = o;         o += align256(4ull * (L.n_tiles / 64 + 1));  // the same summed over 64 tiles
    L.tbase = o;       o += align256(4ull * (L.n_tiles + 1));
    L.pstart = o;      o += align256(4ull * (n + 2));
    L.pval = o;        o += align256(4ull * (n + 1));
    L.tokoff = o;      o += align256(4ull * (n + 2));
    L.scratch = o;     o += align256(4ull * (n + 1));
    L.bin_wave = o;    o += align256(4ull * L.cap_wave);
    L.bin_block = o;   o += align256(4ull * L.cap_block);
    L.bin_giant = o;   o += align256(4ull * L.cap_giant);
    // BPE lists: their items (pieces and chunks of giant pieces) are disjoint byte ranges, so at most
    // n / (shortest length) of them; only chunks are a single byte long
    {
        const uint64_t shortest[6] = {2, 9, 13, 17, 33, 65};
        for (int r = 0; r < 6; ++r) {
            L.miss[r] = o;
            o += align256(4ull * (n / shortest[r] + 1 + (r == 0 ? L.cap_chunks : 0u)));
        }
    }
    L.g_ids = o;       o += align256(4ull * (n + 1));
    // the giant kernel's first rank buffer: the tile encoder's list of 8..32-byte pieces (tokoff),
    // used only inside k_tiles, earlier in the chain
    L.g_rank_a = L.tokoff;
    L.g_rank_b = o;    o += align256(4ull * (n + 1));
    // the tile encoder's BPE queue beyond its LDS part, at the tile's first piece index: used only
    // inside k_tiles, so it shares g_rank_b (only k_bpe_giant, later in the chain, uses that)
    L.tspill = L.g_rank_b;
    // each tile's piece starts at the tile's own place (16-bit offsets at [tile * TILE, ...)), from
    // the pieces kernel to the compaction kernel: shares g_ids (only k_bpe_giant uses that)
    L.prs = L.g_ids;
    L.cstart = o;      o += align256(4ull * L.cap_chunks);
    L.clen = o;        o += align256(4ull * L.cap_chunks);
    L.ccount = o;      o += align256(4ull * L.cap_chunks);
    L.gc0 = o;         o += align256(4ull * L.cap_giant);
    L.gnc = o;         o += align256(4ull * L.cap_giant);
    L.gdone = o;       o += align256(4ull * L.cap_giant);       // seam workgroups done, per giant piece
    L.gsafe = o;       o += align256(4ull * L.n_safe_words);
    L.cpiece = o;      o += align256(4ull * L.cap_chunks);
    L.total = o;
    return L;
}

// The request's sizes.  Kernels get the total byte count, the document count and a layout for a
// capacity; in a plan captured for a size bucket (L.dsz set) the request's own sizes are read from
// device memory when the plan is replayed (the workspace's arrays stay where the capacity puts
// them).  Returns the request's tile count.  A request larger than the bucket, or without documents,
// encodes nothing (*bad set; the first kernel flags it in the status word).  (The layout is only
// read: a kernel that wrote to its layout argument would keep a copy of it in private memory.)
__device__ __forceinline__ uint32_t request_sizes(const Layout &L, uint64_t &n, uint32_t &n_docs, bool *bad = nullptr)
{
    if (!L.dsz) return L.n_tiles;
    const uint64_t rn = L.dsz[0], rd = L.dsz[1];
    const bool ok = rn <= L.cap_n && rd >= 1 && rd <= L.cap_docs;
    if (bad) *bad = !ok;
    n = ok ? rn : 0;
    n_docs = ok ? (uint32_t)rd : 0u;
    return (uint32_t)((n + TILE - 1) / TILE);
}

// whole-piece lookup: a piece whose BPE result is a single token is found with one probe.  The
// tables hold exactly the tokens t whose own byte string encodes to [t] (established at load time
// by these same kernels), so a hit is the exact BPE result.

// Bytes src[0, len) as little-endian 64-bit words k[0..NW), zero past len (len <= 8 * NW).  The
// words are assembled from aligned 8-byte loads: NW + 1 load instructions per wavefront instead of
// one byte gather per byte.  Only aligned words that hold at least one byte of src[0, len) are read,
// and such a word never leaves the page of that byte; the neighbouring bytes it brings are masked.
template <int NW>
__device__ __forceinline__ void load_words(const uint8_t *src, uint32_t len, uint64_t (&k)[NW])
{
    const uintptr_t p = (uintptr_t)src;
    const uint64_t *al = (const uint64_t *)(p & ~(uintptr_t)7);
    const uint32_t off = (uint32_t)(p & 7u), sh = 8u * off;
    uint64_t w[NW + 1];
#pragma unroll
    for (int i = 0; i <= NW; ++i) w[i] = 8u * i < off + len ? al[i] : 0ull;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint64_t x = sh ? (w[i] >> sh) | (w[i + 1] << (64u - sh)) : w[i];
        const uint32_t rem = len > 8u * i ? len - 8u * i : 0u;
        k[i] = rem >= 8u ? x : (x & ((1ull << (8u * rem)) - 1ull));
    }
}

// The whole-piece lookup split into two steps, so that a thread can keep the probes of several pieces
// in flight: wp_make reads the piece's bytes and hashes them; wp_step reads both candidate slots and
// answers WP_HIT (id set) or WP_MISS.
enum : uint32_t { WP_MORE = 0, WP_HIT = 1, WP_MISS = 2 };
struct WPQ {
    uint64_t k0, k1, k2, k3;
    uint32_t len, i, j, kind;   // kind 0: no table applies, 1: short table, 2: long table; i, j: candidates
};

// (for len 1, q.k0 is the piece's byte, which is its token ID)
__device__ __forceinline__ WPQ wp_make(const DevVocab &v, const uint8_t *__restrict__ src, uint32_t len)
{
    WPQ q{0, 0, 0, 0, len, 0, 0, 0};
    if (len == 0 || len > (uint32_t)TABLE_MAX) return q;
    uint64_t k4[4];
    load_words<4>(src, len, k4);
    q.k0 = k4[0]; q.k1 = k4[1]; q.k2 = k4[2]; q.k3 = k4[3];
    if (len <= WA_MAX) {
        if (len == 1 || !v.wa) return q;
        q.k0 |= (uint64_t)len << 56;
        ck_slots(q.k0, v.wseed, v.wa_cap, q.i, q.j);
        q.kind = 1;
        return q;
    }
    if (!v.wb) return q;
    ck_slots(wb_digest(k4[0], k4[1], k4[2], k4[3], len), v.bseed, v.wb_cap, q.i, q.j);
    q.kind = 2;
    return q;
}

// an 8..32-byte entry (three 16-byte words) equal to the key?
__device__ __forceinline__ bool wb_match(uint4 a, uint4 b, uint4 c, uint64_t k0, uint64_t k1, uint64_t k2,
                                         uint64_t k3, uint32_t len)
{
    return c.x == len && ((uint64_t)a.x | ((uint64_t)a.y << 32)) == k0 && ((uint64_t)a.z | ((uint64_t)a.w << 32)) == k1 &&
           ((uint64_t)b.x | ((uint64_t)b.y << 32)) == k2 && ((uint64_t)b.z | ((uint64_t)b.w << 32)) == k3;
}

__device__ __forceinline__ uint32_t wp_step(const DevVocab &v, WPQ &q, uint32_t *id)
{
    if (q.kind == 0) return WP_MISS;
    if (q.kind == 1) {
        const uint4 a = v.wa[q.i], b = v.wa[q.j];
        if (((uint64_t)a.x | ((uint64_t)a.y << 32)) == q.k0) { *id = a.z; return WP_HIT; }
        if (((uint64_t)b.x | ((uint64_t)b.y << 32)) == q.k0) { *id = b.z; return WP_HIT; }
        return WP_MISS;
    }
    const uint4 *e = v.wb + 3ull * q.i, *f = v.wb + 3ull * q.j;
    const uint4 a0 = e[0], a1 = e[1], a2 = e[2], b0 = f[0], b1 = f[1], b2 = f[2];
    if (wb_match(a0, a1, a2, q.k0, q.k1, q.k2, q.k3, q.len)) { *id = a2.y; return WP_HIT; }
    if (wb_match(b0, b1, b2, q.k0, q.k1, q.k2, q.k3, q.len)) { *id = b2.y; return WP_HIT; }
    return WP_MISS;
}

// Per-piece result word (pval).  Bit 31 clear: the piece is one token and the word is its ID.  Bit 31
// set: the piece has (word & PV_COUNT) tokens stored at scratch[piece start byte ...]; bit 30 also set
// for pieces longer than 64 bytes, whose IDs are copied by a separate gather.
constexpr uint32_t PV_MULTI = 1u << 31, PV_LONG = 1u << 30, PV_COUNT = PV_LONG - 1u;

// Result of piece p (first byte b0): n >= 1 tokens, first ID id0 (the others already in scratch
// when n > 1).  The tokens are added to the counters of the input tile of b0 and of its group of 64
// tiles, from which the compaction kernel derives each tile's first output position.
__device__ __forceinline__ void put_piece(uint8_t *ws, const Layout &L, uint32_t p, uint32_t b0, uint32_t n,
                                          uint32_t id0, bool is_long)
{
    ((uint32_t *)(ws + L.pval))[p] = (n == 1 && !is_long) ? id0 : (PV_MULTI | (is_long ? PV_LONG : 0u) | n);
    atomicAdd((uint32_t *)(ws + L.tcount) + b0 / (uint32_t)TILE, n);
    atomicAdd((uint32_t *)(ws + L.tsb) + b0 / (uint32_t)TILE / 64u, n);
}

// List a piece belongs to when it is not resolved directly: 0..5 BPE miss lists (<= 8, 9..12, 13..16,
// 17..32, 33..64, 65..SEG2_MAX bytes), 6..8 length bins (..WAVE_MAX, ..BLOCK_MAX, longer).
constexpr uint32_t NMISS = 6, NROUTES = 9;
__device__ __forceinline__ uint32_t route_of(uint32_t len)
{
    return len <= 8u ? 0u : len <= 12u ? 1u : len <= 16u ? 2u : len <= 32u ? 3u : len <= (uint32_t)LANE_MAX ? 4u :
           len <= (uint32_t)SEG2_MAX ? 5u : len <= (uint32_t)WAVE_MAX ? 6u : len <= (uint32_t)BLOCK_MAX ? 7u : 8u;
}

__device__ __forceinline__ uint32_t *route_list(uint8_t *ws, const Layout &L, uint32_t r)
{
    // (selects, not an index into the layout's array: an indexed kernel argument is copied to
    // private memory)
    const uint64_t o = r == 0 ? L.miss[0] : r == 1 ? L.miss[1] : r == 2 ? L.miss[2] : r == 3 ? L.miss[3] :
                       r == 4 ? L.miss[4] : r == 5 ? L.miss[5] : r == 6 ? L.bin_wave : r == 7 ? L.bin_block : L.bin_giant;
    return (uint32_t *)(ws + o);
}

__device__ __forceinline__ uint32_t *route_count(Ctrl *ctrl, uint32_t r)
{
    return r < NMISS ? &ctrl->miss_count[r] : &ctrl->bin_count[r - NMISS];
}

constexpr uint32_t NO_START = 0xFFFFFFFFu;   // a tile without piece starts

// a piece longer than SHORT_MAX bytes goes on the list of its length bin (encoded before the tile
// encoder, which only collects its result)
__device__ __forceinline__ void list_long(uint8_t *ws, const Layout &L, Ctrl *ctrl, uint32_t p, uint32_t len)
{
    const uint32_t r = route_of(len);
    route_list(ws, L, r)[atomicAdd(route_count(ctrl, r), 1u)] = p;
}

// Called by every thread of a workgroup when it has written its results: true in the workgroup that
// finishes last, which then sees every other workgroup's writes (each thread's writes are fenced at
// agent scope before the count; the last workgroup's threads fence again before their loads).
__device__ __forceinline__ bool last_workgroup(uint32_t *done)
{
    __shared__ uint32_t s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
    __syncthreads();
    const bool last = s_last != 0;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return last;
}

// Wavefront form of the per-tile token counters of the tile encoder's pieces, called by all 64 lanes:
// lane i adds x tokens (0: none) of the piece starting at byte b0 to the counter of b0's input tile
// and of its group of 64 tiles; lanes are combined over runs of equal tiles in lane order and each
// run's last lane issues the atomics.
__device__ __forceinline__ void add_tile_tokens(uint8_t *ws, const Layout &L, uint32_t b0, uint32_t x)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t key = x ? b0 / (uint32_t)TILE : 0xFFFFFFFFu;
    const uint32_t prev = __shfl_up(key, 1, 64);
    const uint64_t heads = __ballot(lane == 0 || prev != key);
    const uint32_t hpos = 63u - (uint32_t)__clzll((unsigned long long)(heads & ((2ull << lane) - 1ull)));
    uint32_t v = x;
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(v, d, 64);
        if (lane >= hpos + d) v += y;
    }
    const bool tail = lane == 63 || ((heads >> (lane + 1)) & 1ull);
    if (tail && key != 0xFFFFFFFFu && v) {
        atomicAdd((uint32_t *)(ws + L.tcount) + key, v);
        atomicAdd((uint32_t *)(ws + L.tsb) + key / 64u, v);
    }
}

// kernel launchers (each in its own translation unit); all enqueue on `s` and return the launch
// status from hipGetLastError
struct Batch {
    const uint8_t *bytes;
    const uint64_t *offsets;
    uint32_t n_docs;
    uint64_t n;
    uint8_t *ws;
    Layout L;
};

// launch indices of the encode chain (TOKTIER_K_* in toktier.h)
enum : int { TK_SUMMARY = 0, TK_PIECES = 1, TK_TILES = 2, TK_GIANT_SEAMS = 3, TK_BPE = 4, TK_BPE_GIANT = 5, TK_EMIT = 6,
             TK_COUNT = 7 };

// optional events recorded around each kernel launch (indices: TOKTIER_K_* in toktier.h)
struct Events {
    void *const *before;
    void *const *after;
};

struct LaunchScope {   // records before[k] on construction and after[k] on destruction
    const Events *ev;
    int k;
    hipStream_t s;
    LaunchScope(const Events *e, int kk, hipStream_t ss) : ev(e), k(kk), s(ss)
    {
        if (ev && ev->before && ev->before[k]) (void)hipEventRecord((hipEvent_t)ev->before[k], s);
    }
    ~LaunchScope()
    {
        if (ev && ev->after && ev->after[k]) (void)hipEventRecord((hipEvent_t)ev->after[k], s);
    }
};

// ---------------------------------------------------------------------------------------------
// added tokens: literals taken out leftmost-longest before the pre-tokenizer

struct DevAdded {
    const uint8_t *bytes;     // the literals' bytes, concatenated
    const uint32_t *off;      // n + 1 offsets into bytes
    const uint32_t *id;       // n output IDs
    const uint32_t *pmap;     // 65536-bit map of the first two bytes (b0 | b1 << 8) of literals >= 2 bytes
    const uint32_t *pre;      // 65537 offsets into list: the literals >= 2 bytes with those first two
    const uint32_t *list;     //   bytes, longest first
    const uint32_t *one;      // 256: the index of the one-byte literal of each byte, or NO_LIT
    uint32_t n, lmin, lmax;
};
constexpr uint32_t NO_LIT = 0xFFFFFFFFu;
constexpr uint32_t LIT_TILE = 4096;          // bytes per workgroup of the literal search
constexpr uint32_t LIT_TAKEN = 1u << 31;     // candidate flag: taken by the leftmost-longest scan

// control words of the literal pass (its own block: the pipeline clears its control block)
struct LitCtrl {
    uint32_t status;      // ST_BAD_OFFSETS
    uint32_t n_cand;      // candidates (a literal starts and ends inside the document)
    uint32_t n_lit;       // literals taken
    uint32_t pad[61];
};

// Workspace of an encode with added tokens: the pipeline's layout first (its control block stays at
// offset 0), then these regions.  K_cap = n / lmin literals at most; S_cap = n_docs + 2 K_cap
// documents after cutting.
struct AddLayout {
    uint64_t lctrl, tcount, tbase, cand, lits, lstart, lcnt, lpref, offs2, oo2, ids2, spans2, total;
    uint32_t n_ltiles;
    uint64_t k_cap, s_cap;
};

inline AddLayout make_add_layout(uint64_t base, uint64_t n, uint32_t n_docs, uint32_t lmin)
{
    AddLayout A;
    A.n_ltiles = (uint32_t)((n + LIT_TILE - 1) / LIT_TILE);
    A.k_cap = n / (lmin ? lmin : 1) + 1;
    A.s_cap = (uint64_t)n_docs + 2 * A.k_cap + 1;
    uint64_t o = base;
    A.lctrl = o;  o += align256(sizeof(LitCtrl));
    A.tcount = o; o += align256(4ull * (A.n_ltiles + 1));
    A.tbase = o;  o += align256(4ull * (A.n_ltiles + 1));
    A.cand = o;   o += align256(8ull * (n + 1));
    A.lits = o;   o += align256(16ull * A.k_cap);
    A.lstart = o; o += align256(4ull * (A.k_cap + 1));
    A.lcnt = o;   o += align256(4ull * (A.k_cap + 1));
    A.lpref = o;  o += align256(4ull * (A.k_cap + 1));
    A.offs2 = o;  o += align256(8ull * A.s_cap);
    A.oo2 = o;    o += align256(8ull * A.s_cap);
    A.ids2 = o;   o += align256(4ull * (n + 1));
    A.spans2 = o; o += align256(4ull * (n + 1));
    A.total = o;
    return A;
}

// the literal search and leftmost-longest scan; the count of taken literals is left in LitCtrl
hipError_t launch_literals(const DevAdded &a, const Batch &b, const AddLayout &A, hipStream_t s);
// the documents cut at the n_lit taken literals (offsets for the pipeline), before it runs
hipError_t launch_literal_docs(const Batch &b, const AddLayout &A, uint32_t n_lit, hipStream_t s);
// after the pipeline encoded the cut documents: final IDs, spans and document offsets
hipError_t launch_literal_merge(const DevAdded &a, const Batch &b, const AddLayout &A, uint32_t n_lit,
                                uint32_t *out_ids, uint64_t *out_offsets, uint32_t *out_spans, hipStream_t s);

hipError_t launch_pretokenize(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev, bool compact);
// pieces longer than BLOCK_MAX: merge-safe seams and chunks (before the tile encoder lists its pieces)
hipError_t launch_giant_prep(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev);
// BPE of every listed piece and chunk, by length: the short lists, then wavefront, workgroup and
// giant pieces (after the tile encoder)
hipError_t launch_bpe(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev);
hipError_t launch_export_starts(const Batch &b, uint32_t *out_starts, hipStream_t s);
hipError_t launch_route(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev);
hipError_t launch_tiles(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev);
hipError_t launch_emit(const DevVocab &v, const Batch &b, uint32_t *out_ids, uint64_t *out_offsets,
                       uint32_t *out_spans, hipStream_t s, const Events *ev);

}  // namespace tt
