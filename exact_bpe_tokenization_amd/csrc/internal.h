// internal.h -- shared definitions of the gfx950 tokenizer library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

// ---------------------------------------------------------------------------------------------
// stage-1 geometry: one workgroup per 4 KiB tile, 16 input bytes per thread
constexpr int PRE_THREADS = 256;
constexpr int PRE_CHUNK = 16;
constexpr int TILE = PRE_THREADS * PRE_CHUNK;  // 4096
constexpr int HALO = 16;                       // look-ahead bytes past a tile

// token-offset scan: one workgroup per 4096 pieces
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_PER_THREAD = 16;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_PER_THREAD;

// BPE length bins (piece bytes): lane <= LANE_MAX < wave <= WAVE_MAX < block <= BLOCK_MAX < giant
constexpr int LANE_MAX = 16;
constexpr int WAVE_MAX = 1024;
constexpr int BLOCK_MAX = 4096;
constexpr int BLOCK_THREADS = 256;
constexpr int GIANT_THREADS = 1024;

// ---------------------------------------------------------------------------------------------
// per-byte character code written by the classify kernel
//   bits 0-2 category; bit 3 CR or LF; bit 4 U+0020; bits 5-6 contraction length code at an
//   apostrophe (0 none, 1 two chars "'x", 2 three chars "'xy"); bit 7 first char of a document
enum : uint8_t { CAT_LU = 0, CAT_LL = 1, CAT_LO = 2, CAT_N = 3, CAT_W = 4, CAT_M = 5, CAT_O = 6,
                 CAT_CONT = 7 };
constexpr uint8_t CC_CRLF = 8, CC_SP = 16, CC_CONTR_SHIFT = 5, CC_DOC = 128;
constexpr uint8_t CC_EOF = 0xFF;   // placed past the end of the batch

// ---------------------------------------------------------------------------------------------
// pre-tokenizer automaton: the state before a character says what the running match expects
enum : int { S_ST = 0, S_LRUN, S_NALL, S_N1, S_N2, S_ORUN, S_ORNL, S_ONL, S_WNL, S_WNS, S_C1,
             S_C2, S_LA, S_LB, S_LEND, NSTATES };
static_assert(NSTATES == 15, "a transition map packs 15 states into 60 bits");

// character context: self code (13) x first-of-document (2) x next-char code (6) x flag (2)
constexpr int NSELF = 13, NNEXT = 6, NCTX = NSELF * 2 * NNEXT * 2;
constexpr uint64_t MAP_IDENTITY = 0x0EDCBA9876543210ull;
constexpr uint64_t NIBBLE_ONES = 0x0111111111111111ull;

// ---------------------------------------------------------------------------------------------
// merge tables.  Pair hash slot: bits 63..21 = (left << 21 | right), bits 20..0 = rank.
constexpr uint32_t NO_RANK = 0xFFFFFFFFu;
constexpr uint64_t EMPTY_SLOT = ~0ull;

struct DevVocab {
    const uint32_t *r2;       // 65536 byte-pair ranks
    const uint64_t *slots;    // pair hash, 2^k slots, linear probing
    const uint32_t *merges;   // 2 * n_merges (left, right)
    const uint64_t *fmap;     // NCTX transition maps
    const uint32_t *fstart;   // NCTX start masks (bit s: a piece starts here when in state s)
    uint32_t mask;
    uint32_t shift;
    uint32_t n_merges;
    int family;
};

__device__ __forceinline__ uint32_t pair_rank(const DevVocab &v, uint32_t a, uint32_t b)
{
    if ((a | b) < 256u) return __ldg(v.r2 + ((a << 8) | b));
    uint64_t key = ((uint64_t)a << 21) | b;
    uint32_t h = (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> v.shift);
    for (;;) {
        uint64_t s = __ldg(v.slots + h);
        if (s == EMPTY_SLOT) return NO_RANK;
        if ((s >> 21) == key) return (uint32_t)(s & 0x1FFFFFu);
        h = (h + 1) & v.mask;
    }
}

// ---------------------------------------------------------------------------------------------
// device control block at the start of the workspace (cleared by the init kernel)
enum : uint32_t { ST_BAD_UTF8 = 1, ST_BAD_OFFSETS = 2 };

struct Ctrl {
    uint32_t status;
    uint32_t tile_ctr_pre;     // dynamic tile ids for the piece kernel
    uint32_t tile_ctr_scan;    // dynamic tile ids for the token-offset scan
    uint32_t n_pieces;
    uint32_t n_tokens;
    uint32_t bin_count[3];     // wave, block, giant bins
    uint32_t pad[56];
};
static_assert(sizeof(Ctrl) == 256, "control block is 256 bytes");

// ---------------------------------------------------------------------------------------------
// workspace layout for n input bytes
struct Layout {
    uint64_t ctrl, cc, tbwd, tflag_state, tflag_cnt, pstart, ntok, tokoff, scratch, bin_wave,
        bin_block, bin_giant, g_ids, g_rank_a, g_rank_b, sflag, total;
    uint32_t n_tiles, n_scan_tiles, cap_wave, cap_block, cap_giant;
};

inline uint64_t align256(uint64_t x) { return (x + 255) & ~255ull; }

inline Layout make_layout(uint64_t n)
{
    Layout L;
    L.n_tiles = (uint32_t)((n + TILE - 1) / TILE);
    L.n_scan_tiles = (uint32_t)((n + 1 + SCAN_TILE - 1) / SCAN_TILE);
    L.cap_wave = (uint32_t)(n / (LANE_MAX + 1) + 1);
    L.cap_block = (uint32_t)(n / (WAVE_MAX + 1) + 1);
    L.cap_giant = (uint32_t)(n / (BLOCK_MAX + 1) + 1);
    uint64_t o = 0;
    L.ctrl = o;        o += align256(sizeof(Ctrl));
    L.cc = o;          o += align256((uint64_t)L.n_tiles * TILE + HALO);  // tiles are whole
    L.tbwd = o;        o += align256((uint64_t)L.n_tiles + 1);
    L.tflag_state = o; o += align256(8ull * L.n_tiles);
    L.tflag_cnt = o;   o += align256(8ull * L.n_tiles);
    L.sflag = o;       o += align256(8ull * L.n_scan_tiles);
    L.pstart = o;      o += align256(4ull * (n + 2));
    L.ntok = o;        o += align256(4ull * (n + 1));
    L.tokoff = o;      o += align256(4ull * (n + 2));
    L.scratch = o;     o += align256(4ull * (n + 1));
    L.bin_wave = o;    o += align256(4ull * L.cap_wave);
    L.bin_block = o;   o += align256(4ull * L.cap_block);
    L.bin_giant = o;   o += align256(4ull * L.cap_giant);
    L.g_ids = o;       o += align256(4ull * (n + 1));
    L.g_rank_a = o;    o += align256(4ull * (n + 1));
    L.g_rank_b = o;    o += align256(4ull * (n + 1));
    L.total = o;
    return L;
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

hipError_t launch_pretokenize(const DevVocab &v, const Batch &b, hipStream_t s);
hipError_t launch_bpe(const DevVocab &v, const Batch &b, hipStream_t s);
hipError_t launch_compact(const Batch &b, uint32_t *out_ids, uint64_t *out_offsets, hipStream_t s);
hipError_t launch_export_starts(const Batch &b, uint32_t *out_starts, hipStream_t s);

}  // namespace tt
