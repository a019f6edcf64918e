// tiles.hip -- the tile encoder and the output writer.
//
// TokTier (arXiv 2607.29678), GPU BPE paragraph and Figure 6 (lower part): pieces are encoded
// independently, dispatched by length to the smallest unit that holds them, with merge ranks and
// whole vocabulary entries looked up in device hash tables; GPU full-tokenization paragraph: the
// path ends with output compaction, and counts stay on the device.
//
//   k_tiles  per 8 KiB input tile, the pieces that start in it: their global numbers (pieces before
//            the tile from the 64-tile group sums and the tile counts the pieces kernel left) and
//            global starts (from the tile's 16-bit offsets; the last piece ends at the next tile's
//            first start); the tile's bytes and the 128 after it are staged in LDS (a piece of up to
//            SHORT_MAX bytes that starts in the tile lies in that window); one byte is its own ID;
//            2..32 bytes are looked up in the whole-piece tables (key built from LDS, the lowest
//            token IDs in LDS, the others with four pieces per thread in flight); longer pieces are
//            listed by length for the workgroup and giant units; the others are queued in LDS and
//            appended to the BPE lists by length, one run per list and tile.  The tile's token count
//            so far goes to its counter and to the counter of its group of 64 tiles (the BPE
//            kernels add the tokens of the pieces they encode).
//   k_emit   per two tiles: their first output index from the counters (the groups before their own,
//            then the tiles before them in their group); groups of eight rounds of 256 pieces whose results
//            and starts are loaded at once, placed by wavefront scans of each round's token counts
//            and one exchange of the per-wavefront totals (consecutive pieces write consecutive IDs);
//            one-token pieces written at once, multi-token ones listed in LDS and copied one per
//            thread with all their loads in flight; per-document token offsets; optional token
//            spans.  Up to 32 more workgroups copy the IDs of the giant pieces.  No workgroup waits
//            for another.
#include "internal.h"

namespace tt {

namespace {

constexpr int NT = 256;                           // threads per tile
constexpr int NW = NT / 64;
constexpr int WIN = TILE + SHORT_MAX + 32;        // LDS byte window [lo, lo + WIN), zero past the batch

constexpr int MQ = 256;                           // pieces a tile lists for BPE through LDS
constexpr int LQ = 1024;                          // 8..32-byte pieces a tile queues in LDS

struct ResolveSmem {
    uint32_t win[WIN / 4];            // the byte window as words
    uint4 hot[HOT_SLOTS];             // the hot sets of the short whole-piece table
    uint32_t q[MQ];                   // pieces left for BPE (index in the tile | length << 16)
    uint32_t lq[LQ];                  // 8..32-byte pieces for the long table (past LQ: device memory)
    uint32_t wsum[NW];
    uint32_t qn, ln;                  // pieces listed for BPE / for the 8..32-byte table
    uint32_t rn[NMISS], rb[NMISS];    // per BPE list: this tile's items, their first list slot
    uint32_t base, next;              // pieces before the tile; the first piece start after it
};

constexpr int ET = 2;             // most tiles per k_emit workgroup
// tiles per k_emit workgroup, from the launch's tile capacity (host and kernel agree): two where the
// launch has tiles enough to fill the CUs, so that a pair shares one set-up; one below that, so that
// a single request's tiles spread over twice the workgroups
__host__ __device__ inline uint32_t emit_tiles_per_wg(uint32_t cap_tiles) { return cap_tiles >= 1024u ? 2u : 1u; }
constexpr int ER = 8;             // rounds of NT pieces whose loads k_emit issues together (pick())
constexpr int MLQ = NT;           // multi-token pieces k_emit lists in LDS per group of rounds

struct EmitSmem {
    uint32_t docbits[ET * TILE / 32]; // document starts in the workgroup's tiles
    uint32_t wtot[ER][NW];            // tokens per round and wavefront of the current group
    uint32_t ma[MLQ], mo[MLQ], mc[MLQ];   // listed multi-token pieces: start byte, output index, count
    uint32_t mn;                      // multi-token pieces listed
    uint32_t base, p0, p1;
    uint4 dd;
};

template <typename S>
__device__ __forceinline__ uint32_t win_byte(const S &sm, uint32_t j)
{
    return (sm.win[j >> 2] >> (8u * (j & 3u))) & 255u;
}

// bytes win[j, j + len) as little-endian 64-bit words k[0..NWD), zero past len (len <= 8 NWD); reads
// only the 32-bit words that hold bytes of the piece
template <int NWD, typename S>
__device__ __forceinline__ void win_words(const S &sm, uint32_t j, uint32_t len, uint64_t (&k)[NWD])
{
    const uint32_t q0 = j >> 2, sh = j & 3u;
    uint32_t x[2 * NWD + 1];
#pragma unroll
    for (int i = 0; i <= 2 * NWD; ++i) x[i] = 4u * (uint32_t)i < sh + len ? sm.win[q0 + i] : 0u;
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
        const uint32_t lo = sh ? __builtin_amdgcn_alignbyte(x[2 * i + 1], x[2 * i], sh) : x[2 * i];
        const uint32_t hi = sh ? __builtin_amdgcn_alignbyte(x[2 * i + 2], x[2 * i + 1], sh) : x[2 * i + 1];
        const uint64_t w = (uint64_t)lo | ((uint64_t)hi << 32);
        const uint32_t rem = len > 8u * i ? len - 8u * i : 0u;
        k[i] = rem >= 8u ? w : (w & ((1ull << (8u * rem)) - 1ull));
    }
}

// the byte window [lo, lo + WIN), zero past the batch.  Every thread issues all of its loads before
// storing any (a loop that waits for each load pays one memory latency per iteration): interior
// tiles with 16-byte aligned input read aligned 16-byte words; otherwise 32-bit words from two
// aligned loads each (never leaving the pages of the bytes they hold), zero past the batch.
template <typename S>
__device__ __forceinline__ void load_window(S &sm, const uint8_t *__restrict__ bytes, uint64_t n, uint64_t lo)
{
    constexpr int NV = WIN / 16;                    // 16-byte words of the window
    constexpr int PER = (NV + NT - 1) / NT;
    static_assert(WIN % 16 == 0, "window of whole 16-byte words");
    const uint32_t tid = threadIdx.x;
    if (lo + WIN <= n && ((uintptr_t)(bytes + lo) & 15u) == 0) {
        const uint4 *src = (const uint4 *)(bytes + lo);
        uint4 x[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const uint32_t w = tid + k * NT;
            x[k] = w < (uint32_t)NV ? src[w] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const uint32_t w = tid + k * NT;
            if (w < (uint32_t)NV) *(uint4 *)&sm.win[4 * w] = x[k];
        }
        return;
    }
    constexpr int PER4 = (WIN / 4 + NT - 1) / NT;
    uint32_t x[PER4];
#pragma unroll
    for (int k = 0; k < PER4; ++k) {
        const uint32_t w = tid + k * NT;
        const uint64_t q = lo + 4ull * w;
        uint32_t y = 0;
        if (w < (uint32_t)WIN / 4 && q + 4 <= n) {
            const uintptr_t ad = (uintptr_t)(bytes + q);
            const uint32_t *al = (const uint32_t *)(ad & ~(uintptr_t)3);
            const uint32_t sh = (uint32_t)(ad & 3u);
            const uint32_t w0 = al[0], w1 = sh ? al[1] : 0u;
            y = sh ? __builtin_amdgcn_alignbyte(w1, w0, sh) : w0;
        } else if (w < (uint32_t)WIN / 4) {
            for (uint32_t t = 0; t < 4; ++t)
                if (q + t < n) y |= (uint32_t)bytes[q + t] << (8 * t);
        }
        x[k] = y;
    }
#pragma unroll
    for (int k = 0; k < PER4; ++k) {
        const uint32_t w = tid + k * NT;
        if (w < (uint32_t)WIN / 4) sm.win[w] = x[k];
    }
}

// exclusive sum over the workgroup; *total receives the sum
template <typename S>
__device__ __forceinline__ uint32_t wg_excl_sum(S &sm, uint32_t x, uint32_t *total)
{
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_sum(x);
    if (lane == 63) sm.wsum[wid] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t s = sm.wsum[w];
        if ((uint32_t)w < wid) before += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + inc - x;
}

// The c IDs of a multi-token piece of at most SEG2_MAX bytes, copied by one thread from
// scratch[a ...] to out_ids[o ...] (eight loads in flight per step); with spans, each token's start
// byte from the piece's start and the token lengths.
template <bool SPANS>
__device__ __forceinline__ void copy_ids(const uint32_t *scratch, uint32_t a, uint32_t o, uint32_t c,
                                         uint32_t *out_ids, uint32_t *out_spans, const uint32_t *tok_len)
{
    uint32_t sp = a;
    for (uint32_t t0 = 0; t0 < c; t0 += 8) {
        uint32_t x[8];
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) x[u] = t0 + u < c ? scratch[a + t0 + u] : 0u;
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {
            if (t0 + u < c) {
                out_ids[o + t0 + u] = x[u];
                if (SPANS) {
                    out_spans[o + t0 + u] = sp;
                    sp += tok_len[x[u]];
                }
            }
        }
    }
}

// x[k] for a k that is not known at compile time, by selects with constant indices (a loop here
// would leave the array in private memory)
__device__ __forceinline__ uint32_t pick(const uint32_t (&x)[8], uint32_t k)
{
    const uint32_t lo4 = k == 0 ? x[0] : k == 1 ? x[1] : k == 2 ? x[2] : x[3];
    const uint32_t hi4 = k == 4 ? x[4] : k == 5 ? x[5] : k == 6 ? x[6] : x[7];
    return k < 4 ? lo4 : hi4;
}

// The IDs of a piece of 129..BLOCK_MAX bytes, encoded before the tile encoder, copied by one
// wavefront from scratch[a ...] to out_ids[o ...] (eight tokens per lane and step, their loads in
// flight together); with spans, a wavefront scan of the token lengths from the piece's start.
template <bool SPANS>
__device__ void copy_long(const uint8_t *ws, const Layout &L, uint32_t a, uint32_t o, uint32_t cnt,
                          uint32_t *out_ids, uint32_t *out_spans, const uint32_t *tok_len)
{
    constexpr uint32_t U = 8;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t *src = (const uint32_t *)(ws + L.scratch) + a;
    uint32_t carry = a;
    for (uint32_t t0 = 0; t0 < cnt; t0 += 64u * U) {
        uint32_t id[U];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t t = t0 + 64u * u + lane;
            id[u] = t < cnt ? src[t] : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t t = t0 + 64u * u + lane;
            if (t < cnt) out_ids[o + t] = id[u];
            if (SPANS) {
                const uint32_t l = t < cnt ? tok_len[id[u]] : 0u;
                const uint32_t inc = wave_incl_sum(l);
                if (t < cnt) out_spans[o + t] = carry + inc - l;
                carry += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
            }
        }
    }
}

// Workgroups past the tiles: the IDs of the giant pieces (longer than BLOCK_MAX), chunk by chunk.
// Each giant piece gets a share of these workgroups; a workgroup finds the piece's first output
// index itself (its tile's first index from the counters, plus the tokens of the tile's pieces
// before it).  Chunk k's IDs sit at scratch[its start byte ...] and go to the piece's output at the
// chunk's place (recorded by the giant join in clen).  The share's workgroups walk the chunks in
// blocks of NT: a chunk of at most SMALL_CHUNK tokens is copied by one thread (of the workgroup the
// chunk's index selects), a longer one by all of them, each workgroup taking its part of the
// chunk's tokens.  With spans, a chunk's spans run from its start byte.
constexpr uint32_t SMALL_CHUNK = 64;

// WG-wide inclusive sum helper for emit_giant (returns the workgroup total to every thread)
__device__ __forceinline__ uint32_t wg_total(uint32_t x, uint32_t *red)
{
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    x = wave_incl_sum(x);
    if (lane == 63) red[wid] = x;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) t += red[k];
    __syncthreads();
    return t;
}

template <bool SPANS>
__device__ void emit_giant(const uint8_t *ws, const Layout &L, uint32_t w, uint32_t nw, uint32_t *out_ids,
                           uint32_t *out_spans, const uint32_t *tok_len)
{
    __shared__ uint32_t s_red[NW], s_big[NT], s_nbig;
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t count = ctrl->bin_count[2];
    if (count == 0) return;
    const uint32_t tid = threadIdx.x;
    const uint32_t *list = (const uint32_t *)(ws + L.bin_giant);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart), *pval = (const uint32_t *)(ws + L.pval);
    const uint32_t *tbase = (const uint32_t *)(ws + L.tbase), *tcount = (const uint32_t *)(ws + L.tcount);
    const uint32_t *tsb = (const uint32_t *)(ws + L.tsb);
    const uint32_t *gc0 = (const uint32_t *)(ws + L.gc0), *gnc = (const uint32_t *)(ws + L.gnc);
    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *cdest = (const uint32_t *)(ws + L.clen);
    const uint32_t *ccount = (const uint32_t *)(ws + L.ccount);
    const uint32_t *scratch = (const uint32_t *)(ws + L.scratch);
    // workgroups per piece (at least one); this workgroup's pieces g = w / per, w / per + nw / per, ...
    const uint32_t per = count >= nw ? 1u : nw / count;
    const uint32_t sub = w % per;
    for (uint32_t g = w / per; g < count; g += nw / per) {
        const uint32_t p = list[g], t = pstart[p] / (uint32_t)TILE, q0 = tbase[t];
        // first output index of p: groups of 64 tiles before t's, tiles before t in its group, pieces
        // of t before p
        uint32_t x = 0;
        for (uint32_t k = tid; k < t / 64u; k += NT) x += tsb[k];
        for (uint32_t k = 64u * (t / 64u) + tid; k < t; k += NT) x += tcount[k];
        for (uint32_t q = q0 + tid; q < p; q += NT) {
            const uint32_t pv = pval[q];
            x += (pv & PV_MULTI) ? (pv & PV_COUNT) : 1u;
        }
        const uint32_t o = wg_total(x, s_red), c0 = gc0[g], nc = gnc[g];
        for (uint32_t k0 = 0; k0 < nc; k0 += NT) {
            if (tid == 0) s_nbig = 0;
            __syncthreads();
            const uint32_t k = k0 + tid;
            if (k < nc) {
                const uint32_t ck = c0 + k, cnt = ccount[ck];
                if (cnt > SMALL_CHUNK) {
                    s_big[atomicAdd(&s_nbig, 1u)] = ck;
                } else if (k % per == sub) {
                    const uint32_t cs = cstart[ck], dst = o + cdest[ck];
                    uint32_t sp = cs;
                    for (uint32_t t0 = 0; t0 < cnt; t0 += 8) {
                        uint32_t id[8];
#pragma unroll
                        for (uint32_t u = 0; u < 8; ++u) id[u] = t0 + u < cnt ? scratch[cs + t0 + u] : 0u;
#pragma unroll
                        for (uint32_t u = 0; u < 8; ++u) {
                            if (t0 + u < cnt) {
                                out_ids[dst + t0 + u] = id[u];
                                if (SPANS) {
                                    out_spans[dst + t0 + u] = sp;
                                    sp += tok_len[id[u]];
                                }
                            }
                        }
                    }
                }
            }
            __syncthreads();
            // the long chunks of this block: every workgroup of the share takes its part of each
            const uint32_t nb = s_nbig;
            for (uint32_t b = 0; b < nb; ++b) {
                const uint32_t ck = s_big[b], cs = cstart[ck], dst = o + cdest[ck], cnt = ccount[ck];
                const uint32_t r0 = (uint32_t)((uint64_t)cnt * sub / per), r1 = (uint32_t)((uint64_t)cnt * (sub + 1) / per);
                uint32_t carry = cs;
                if (SPANS) {   // the lengths of the chunk's tokens before this part
                    uint32_t y = 0;
                    for (uint32_t q = tid; q < r0; q += NT) y += tok_len[scratch[cs + q]];
                    carry += wg_total(y, s_red);
                }
                constexpr uint32_t U = 8;
                for (uint32_t t0 = r0; t0 < r1; t0 += U * NT) {
                    uint32_t id[U];
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) {
                        const uint32_t q = t0 + u * NT + tid;
                        id[u] = q < r1 ? scratch[cs + q] : 0u;
                    }
#pragma unroll
                    for (uint32_t u = 0; u < U; ++u) {
                        const uint32_t q = t0 + u * NT + tid;
                        if (q < r1) out_ids[dst + q] = id[u];
                        if (SPANS) {
                            const uint32_t l = q < r1 ? tok_len[id[u]] : 0u;
                            const uint32_t lane = tid & 63u, wid = tid >> 6;
                            const uint32_t inc = wave_incl_sum(l);
                            if (lane == 63) s_red[wid] = inc;
                            __syncthreads();
                            uint32_t before = 0, tot = 0;
#pragma unroll
                            for (int k2 = 0; k2 < NW; ++k2) {
                                const uint32_t z = s_red[k2];
                                tot += z;
                                before += (uint32_t)k2 < wid ? z : 0u;
                            }
                            __syncthreads();
                            if (q < r1) out_spans[dst + q] = carry + before + inc - l;
                            carry += tot;
                        }
                    }
                }
            }
            __syncthreads();   // s_big and s_nbig are rewritten by the next block
        }
    }
}

}  // namespace

// key of a 2..7-byte piece at window offset j: its bytes (little-endian) | len << 56
template <typename S>
__device__ __forceinline__ uint64_t short_key(const S &sm, uint32_t j, uint32_t len)
{
    const uint32_t q0 = j >> 2, sh = j & 3u;
    const uint32_t x0 = sm.win[q0], x1 = sm.win[q0 + 1], x2 = sm.win[q0 + 2];
    const uint32_t lo = sh ? __builtin_amdgcn_alignbyte(x1, x0, sh) : x0;
    const uint32_t hi = sh ? __builtin_amdgcn_alignbyte(x2, x1, sh) : x1;
    const uint64_t w = (uint64_t)lo | ((uint64_t)hi << 32);
    return (w & ((1ull << (8u * len)) - 1ull)) | ((uint64_t)len << 56);
}

// Resolve pass over the tile's pieces.  Each piece, by length:
//   1 byte          its own ID
//   2..7 bytes      the hot sets in LDS (the lowest token IDs), else: 2 bytes the byte-pair rank
//                   table (one merge or none decides it; ignore_merges vocabularies look them up like
//                   3..7 bytes), 3..7 bytes the short whole-piece table (four pieces per thread with
//                   their loads in flight)
//   8..32 bytes     listed in the tile's slice of a second list, probed in a second compact pass
//   33..128 bytes   (and table misses) listed in the tile's slice of the BPE list
//   longer          encoded before this kernel: its result word is read
template <bool IGN>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(IGN ? 4 : 5, 8))) void k_tiles(DevVocab v, const uint8_t *__restrict__ bytes, uint64_t n, uint8_t *ws,
                                              Layout L)
{
    __shared__ ResolveSmem sm;
    {
        uint32_t nd = 0;
        if (blockIdx.x >= request_sizes(L, n, nd)) return;   // (a request smaller than the plan's size bucket)
    }
    uint32_t *__restrict__ pstart = (uint32_t *)(ws + L.pstart);
    uint32_t *pval = (uint32_t *)(ws + L.pval);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    const uint32_t tile = blockIdx.x;
    const uint64_t lo = (uint64_t)tile * TILE;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    // the tile's piece starts, as the pieces kernel left them: a count and 16-bit offsets at the
    // tile's own place; this kernel gives them their global places (pieces before the tile: the
    // 64-tile group sums before its group, then the tiles of its group before it)
    const uint32_t *tcnt = (const uint32_t *)(ws + L.tcnt);
    const uint16_t *prs = (const uint16_t *)(ws + L.prs) + lo;
    const uint32_t cnt = tcnt[tile];
    if (wid == 0) {
        const uint32_t *gsum = (const uint32_t *)(ws + L.gsum);
        const uint32_t g = tile / 64u;
        uint32_t x = 0;
        for (uint32_t k = lane; k < g; k += 64u) x += gsum[k];
        if (64u * g + lane < tile) x += tcnt[64u * g + lane];
        x = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(x), 63);
        if (lane == 0) sm.base = x;
    } else if (wid == 1) {
        // the first start after the tile (the end of its last piece), else the end of the batch
        const uint32_t *tfirst = (const uint32_t *)(ws + L.tfirst);
        uint32_t nd = 0;
        uint64_t nn = n;
        const uint32_t n_tiles = request_sizes(L, nn, nd);
        uint32_t nx = (uint32_t)nn;
        for (uint32_t t0 = tile + 1; t0 < n_tiles; t0 += 64u) {
            const uint32_t t = t0 + lane;
            const uint32_t f = t < n_tiles ? tfirst[t] : NO_START;
            const uint64_t has = __ballot(f != NO_START);
            if (has) {
                nx = (uint32_t)__builtin_amdgcn_readlane((int)f, __ffsll((unsigned long long)has) - 1);
                break;
            }
        }
        if (lane == 0) sm.next = nx;
    }

    // the window and the hot sets (their loads issued together)
    {
        constexpr int PH = HOT_SLOTS / NT;
        uint4 h[PH];
#pragma unroll
        for (int k = 0; k < PH; ++k) h[k] = v.hot ? v.hot[tid + k * NT] : make_uint4(0u, 0u, 0u, 0u);
        load_window(sm, bytes, n, lo);
#pragma unroll
        for (int k = 0; k < PH; ++k) sm.hot[tid + k * NT] = h[k];
    }
    if (tid == 0) {
        sm.qn = 0;
        sm.ln = 0;
    }
    __syncthreads();
    const uint32_t p0 = sm.base, next = sm.next;
    if (tid == 0) {
        ((uint32_t *)(ws + L.tbase))[tile] = p0;
        uint32_t nd = 0;
        uint64_t nn = n;
        const uint32_t n_tiles = request_sizes(L, nn, nd);
        if (tile == n_tiles - 1) {   // the last tile: the piece count, the batch end, the tile bases' end
            ctrl->n_pieces = p0 + cnt;
            pstart[p0 + cnt] = (uint32_t)nn;
            ((uint32_t *)(ws + L.tbase))[n_tiles] = p0 + cnt;
        }
    }
    uint32_t *llist = (uint32_t *)(ws + L.tokoff) + p0;   // the 8..32-byte pieces past LQ
    // a piece left for BPE: queued (index in the tile | length << 16) in LDS, past its capacity in
    // the tile's own slice of a device array; at the end the queue goes to the BPE lists in one run
    // per list
    uint32_t *spill = (uint32_t *)(ws + L.tspill) + p0;
    auto list_miss = [&](uint32_t i, uint32_t len) {
        const uint32_t slot = atomicAdd(&sm.qn, 1u);
        if (slot < (uint32_t)MQ) sm.q[slot] = i | (len << 16);
        else spill[slot - MQ] = i | (len << 16);
    };

    uint32_t mytok = 0;
    constexpr int K = 4;
    // a step's start offsets (this piece's and the next one's) are loaded during the step before,
    // while that step's table reads are in flight: indices clamped into the tile's part of the array
    // (a load under a branch would be waited for at once), the values used only in the next step
    uint32_t o0[K], o1[K];
    auto load_offsets = [&](uint32_t i0) {
        const uint32_t last = cnt ? cnt - 1 : 0u;
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const uint32_t i = i0 + u * NT + tid;
            o0[u] = prs[min(i, last)];
            o1[u] = prs[min(i + 1, last)];
        }
    };
    load_offsets(0);
    for (uint32_t i0 = 0; i0 < cnt; i0 += K * NT) {
        uint32_t a[K], e[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const uint32_t i = i0 + u * NT + tid;
            a[u] = i < cnt ? (uint32_t)lo + o0[u] : 0u;
            e[u] = i + 1 < cnt ? (uint32_t)lo + o1[u] : next;
        }
        // kind: 0 nothing to load, 2 byte pair, 3 short table (both candidate slots).  Each piece's
        // result word is written once, in one coalesced store per row of the step (the pieces resolved
        // later -- by the long table below or by the BPE kernels -- get a placeholder overwritten then):
        // scattered partial stores would leave partly written cache lines to be written back repeatedly
        // The step's global stores are issued after its table reads have been waited for (the wait
        // counter covers loads and stores in issue order), the next offsets with the reads.
        uint32_t kind[K], si[K], sj[K], res[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const uint32_t i = i0 + u * NT + tid;
            kind[u] = 0;
            si[u] = 0;
            sj[u] = 0;
            res[u] = 0;
            if (i >= cnt) continue;
            const uint32_t j = a[u] - (uint32_t)lo, len = e[u] - a[u];
            if (len == 1) {
                res[u] = win_byte(sm, j);
                ++mytok;
            } else if (len <= WA_MAX) {
                const uint64_t key = short_key(sm, j, len);
                const uint32_t set = hot_set(key);
                const uint4 h0 = sm.hot[2 * set], h1 = sm.hot[2 * set + 1];
                const uint64_t k0 = (uint64_t)h0.x | ((uint64_t)h0.y << 32), k1 = (uint64_t)h1.x | ((uint64_t)h1.y << 32);
                if (k0 == key || k1 == key) {
                    res[u] = k0 == key ? h0.z : h1.z;
                    ++mytok;
                } else if (len == 2 && !IGN) {
                    kind[u] = 2;
                    si[u] = (win_byte(sm, j) << 8) | win_byte(sm, j + 1);
                } else if (v.wa) {
                    kind[u] = 3;
                    ck_slots(key, v.wseed, v.wa_cap, si[u], sj[u]);
                } else {
                    list_miss(i, len);
                }
            } else if (len <= (uint32_t)TABLE_MAX) {
                const uint32_t slot = atomicAdd(&sm.ln, 1u), ent = i | (j << 13) | (len << 26);
                if (slot < (uint32_t)LQ) sm.lq[slot] = ent;
                else llist[slot] = ent;
            } else if (len <= (uint32_t)SHORT_MAX) {
                uint32_t w = NO_PIECE;
                if (IGN && len <= v.lmax) w = whole_token(v, bytes + a[u], len);
                if (w != NO_PIECE) {
                    res[u] = w;
                    ++mytok;
                } else {
                    list_miss(i, len);
                }
            } else {   // longer pieces: listed by length for the workgroup and giant units
                list_long(ws, L, ctrl, p0 + i, len);
            }
        }
        // the global lookups of the pieces the hot sets did not answer: all loads in flight at once,
        // issued without branches (a lane with nothing to look up reads entry 0)
        uint4 x[K], y[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            if (v.wa) {
                x[u] = v.wa[kind[u] == 3 ? si[u] : 0u];
                y[u] = v.wa[kind[u] == 3 ? sj[u] : 0u];
            }
            const uint32_t r = __ldg(v.r2 + (kind[u] == 2 ? si[u] : 0u));
            if (kind[u] == 2) x[u].x = r;
        }
        if (i0 + K * NT < cnt) load_offsets(i0 + K * NT);
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const uint32_t i = i0 + u * NT + tid;
            if (kind[u] == 2) {
                const uint32_t r = x[u].x;   // the pair's rank word
                if (r != NO_RANK) {
                    res[u] = 256u + (r >> 2);
                    ++mytok;
                } else {   // no merge joins the two bytes: two tokens
                    res[u] = PV_MULTI | 2u;
                    scratch[a[u]] = si[u] >> 8;
                    scratch[a[u] + 1] = si[u] & 255u;
                    mytok += 2;
                }
            } else if (kind[u] == 3) {
                // the key again from the window (cheaper than holding it across the loads)
                const uint32_t len = e[u] - a[u];
                const uint64_t k = short_key(sm, a[u] - (uint32_t)lo, len);
                const uint64_t ka = (uint64_t)x[u].x | ((uint64_t)x[u].y << 32);
                const uint64_t kb = (uint64_t)y[u].x | ((uint64_t)y[u].y << 32);
                if (ka == k || kb == k) {
                    res[u] = ka == k ? x[u].z : y[u].z;
                    ++mytok;
                } else {
                    list_miss(i, len);
                }
            }
            if (i < cnt) pval[p0 + i] = res[u];
        }
#pragma unroll
        for (int u = 0; u < K; ++u) {   // the global piece starts, for the kernels after this one
            const uint32_t i = i0 + u * NT + tid;
            if (i < cnt) pstart[p0 + i] = a[u];
        }
    }
    __syncthreads();

    // 8..32-byte pieces, compacted (in LDS, past LQ in the tile's slice of a device array): the long
    // whole-piece table.  An entry holds the piece's index in
    // the tile, its window offset and its length (13 + 13 + 6 bits); the table reads of a pass are
    // issued together and without branches (an idle slot reads entry 0)
    const uint32_t nl = sm.ln;
    for (uint32_t k0 = 0; k0 < nl; k0 += NT) {
        const uint32_t k = k0 + tid;
        const uint32_t ent = k < nl ? (k < (uint32_t)LQ ? sm.lq[k] : llist[k]) : 0u;
        const uint32_t i = ent & 0x1FFFu, j = (ent >> 13) & 0x1FFFu, len = ent >> 26;
        uint64_t k4[4];
        win_words<4>(sm, j, len, k4);
        uint32_t ci = 0, cj = 0;
        if (v.wb && len) ck_slots(wb_digest(k4[0], k4[1], k4[2], k4[3], len), v.bseed, v.wb_cap, ci, cj);
        uint4 ea[3], eb[3];
        if (v.wb) {
            const uint4 *ep = v.wb + 3ull * ci, *fp = v.wb + 3ull * cj;
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                ea[w] = ep[w];
                eb[w] = fp[w];
            }
        }
        if (!len) continue;   // (no entry)
        bool hit = false;
        uint32_t id = 0;
        if (v.wb) {
            if (wb_match(ea[0], ea[1], ea[2], k4[0], k4[1], k4[2], k4[3], len)) {
                hit = true;
                id = ea[2].y;
            } else if (wb_match(eb[0], eb[1], eb[2], k4[0], k4[1], k4[2], k4[3], len)) {
                hit = true;
                id = eb[2].y;
            }
        }
        if (hit) {
            pval[p0 + i] = id;
            ++mytok;
        } else {
            list_miss(i, len);
        }
    }

    // the queued pieces to the BPE lists: count per list, one reservation per list, then the tile's
    // items in one run per list (the slice is read back by the threads that wrote it or, after the
    // barrier, by others of this workgroup)
    __syncthreads();
    const uint32_t nq = sm.qn;
    if (tid < NMISS) sm.rn[tid] = 0;
    __syncthreads();
    auto queued = [&](uint32_t k) { return k < (uint32_t)MQ ? sm.q[k] : spill[k - MQ]; };
    for (uint32_t k = tid; k < nq; k += NT) atomicAdd(&sm.rn[route_of(queued(k) >> 16)], 1u);
    __syncthreads();
    if (tid < NMISS) {
        const uint32_t c = sm.rn[tid];
        sm.rb[tid] = c ? atomicAdd(&ctrl->miss_count[tid], c) : 0u;
        sm.rn[tid] = 0;
    }
    __syncthreads();
    for (uint32_t k = tid; k < nq; k += NT) {
        const uint32_t e = queued(k), r = route_of(e >> 16);
        route_list(ws, L, r)[sm.rb[r] + atomicAdd(&sm.rn[r], 1u)] = p0 + (e & 0xFFFFu);
    }

    // tokens of the pieces resolved here (the BPE kernels add the others)
    uint32_t tile_tok;
    (void)wg_excl_sum(sm, mytok, &tile_tok);
    if (tid == 0) {
        ((uint32_t *)(ws + L.tcount))[tile] = tile_tok;
        if (tile_tok) atomicAdd((uint32_t *)(ws + L.tsb) + tile / 64u, tile_tok);
    }
}

template <bool SPANS>
__global__ __launch_bounds__(NT) void k_emit(DevVocab v, const uint64_t *__restrict__ offsets, uint32_t n_docs,
                                             uint64_t n, uint8_t *ws, Layout L, uint32_t *__restrict__ out_ids,
                                             uint64_t *__restrict__ out_offsets, uint32_t *__restrict__ out_spans)
{
    __shared__ EmitSmem sm;
    const uint32_t et = emit_tiles_per_wg(L.n_tiles);
    const uint32_t grid_tiles = (L.n_tiles + et - 1) / et;   // the launch's tile workgroups (a plan's size bucket)
    if (blockIdx.x >= grid_tiles) {   // the giant pieces' IDs
        emit_giant<SPANS>(ws, L, blockIdx.x - grid_tiles, gridDim.x - grid_tiles, out_ids, out_spans, v.tok_len);
        return;
    }
    const uint32_t n_tiles = request_sizes(L, n, n_docs);
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    if (n_tiles == 0) {   // an empty request in a plan's size bucket: every document is empty
        if (blockIdx.x == 0) {
            for (uint32_t d = threadIdx.x; d <= n_docs; d += NT) out_offsets[d] = 0;
            if (threadIdx.x == 0) ctrl->n_tokens = 0;
        }
        return;
    }
    if (blockIdx.x * et >= n_tiles) return;
    const uint32_t *__restrict__ pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *__restrict__ tbase = (const uint32_t *)(ws + L.tbase);
    const uint32_t *__restrict__ tcount = (const uint32_t *)(ws + L.tcount);
    const uint32_t *__restrict__ tsb = (const uint32_t *)(ws + L.tsb);
    const uint32_t *__restrict__ pval = (const uint32_t *)(ws + L.pval);
    const uint32_t *__restrict__ scratch = (const uint32_t *)(ws + L.scratch);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    // this workgroup's tiles [tile, t1)
    const uint32_t tile = blockIdx.x * et, t1 = min(tile + et, n_tiles);
    const uint64_t lo = (uint64_t)tile * TILE;
    const uint64_t hi = min((uint64_t)t1 * TILE, n);
    auto count_of = [](uint32_t pv) -> uint32_t { return (pv & PV_MULTI) ? (pv & PV_COUNT) : 1u; };

    // the loads that depend on nothing, at once: the tiles' piece range and document window; wave 0:
    // the first output index of the first tile (the groups of 64 tiles before its group, then the
    // tiles before it in its group; counts are final: every kernel that adds to them has finished)
    for (uint32_t i = tid; i < et * (TILE / 32); i += NT) sm.docbits[i] = 0;
    if (wid == 0) {
        const uint32_t g = tile / 64u;
        uint32_t x = 0;
        for (uint32_t t = lane; t < g; t += 64) x += tsb[t];
        if (64 * g + lane < tile) x += tcount[64 * g + lane];
        x = wave_incl_sum(x);
        if (lane == 63) sm.base = x;
        if (lane == 0) sm.mn = 0;
    } else if (tid == 64) {
        sm.p0 = tbase[tile];
        sm.p1 = tbase[t1];
        const uint4 d0 = ((const uint4 *)(ws + L.tdoc))[tile], d1 = ((const uint4 *)(ws + L.tdoc))[t1 - 1];
        sm.dd = make_uint4(d0.x, d1.y, 0u, 0u);   // documents of the windows of the first and last tile
    }
    __syncthreads();
    const uint32_t p0 = sm.p0, cnt = sm.p1 - p0;
    const uint4 dd = sm.dd;
    // document starts in [lo, hi) (k_summary found the documents of a window around the tile); the
    // first group's barrier orders these bits before their use
    for (uint32_t d = dd.x + tid; d < dd.y; d += NT) {
        const uint64_t od = offsets[d];
        if (od >= lo && od < hi) atomicOr(&sm.docbits[(od - lo) >> 5], 1u << ((od - lo) & 31u));
    }

    // Groups of ER rounds of NT pieces (piece g0 + NT k + tid of the tile in round k): the results and
    // starts of the whole group are loaded at once; one exchange of every round's per-wavefront token
    // totals places every piece; one-token pieces are written at once, multi-token ones are listed in
    // LDS and copied one per thread, all their loads in flight together; long pieces are copied by
    // their wavefront.
    const uint32_t *tok_len = v.tok_len;
    uint32_t run = sm.base;
    for (uint32_t g0 = 0; g0 < cnt; g0 += ER * NT) {
        uint32_t pv[ER], a[ER], o[ER];
#pragma unroll
        for (int k = 0; k < ER; ++k) {
            const uint32_t q = g0 + (uint32_t)k * NT + tid;
            pv[k] = q < cnt ? pval[p0 + q] : 0u;
            a[k] = q < cnt ? pstart[p0 + q] : 0u;
        }
#pragma unroll
        for (int k = 0; k < ER; ++k) {
            const uint32_t c = g0 + (uint32_t)k * NT + tid < cnt ? count_of(pv[k]) : 0u;
            const uint32_t inc = wave_incl_sum(c);
            o[k] = inc - c;
            if (lane == 63) sm.wtot[k][wid] = inc;
        }
        __syncthreads();
        static_assert(NW == 4, "one uint4 of wavefront totals per round");
#pragma unroll
        for (int k = 0; k < ER; ++k) {
            const uint4 t = *(const uint4 *)sm.wtot[k];
            o[k] += run + (wid > 0 ? t.x : 0u) + (wid > 1 ? t.y : 0u) + (wid > 2 ? t.z : 0u);
            run += t.x + t.y + t.z + t.w;
        }
        // one-token pieces now; bit k of pend / lng / dst: the piece of round k has several tokens
        // (up to SEG2_MAX bytes) / is long (up to BLOCK_MAX bytes; the giant ones are copied by the
        // workgroups past the tiles) / starts a document
        uint32_t pend = 0, lng = 0, dst = 0;
#pragma unroll
        for (int k = 0; k < ER; ++k) {
            if (g0 + (uint32_t)k * NT + tid < cnt) {
                if (!(pv[k] & PV_MULTI)) {
                    out_ids[o[k]] = pv[k];
                    if (SPANS) out_spans[o[k]] = a[k];
                } else if (!(pv[k] & PV_LONG)) {
                    pend |= 1u << k;
                } else {
                    lng |= 1u << k;
                }
                const uint32_t j = (uint32_t)(a[k] - lo);
                dst |= ((sm.docbits[j >> 5] >> (j & 31u)) & 1u) << k;
            }
        }
        // the long pieces: each copied by its wavefront
        while (__ballot(lng != 0)) {
            const int b = __ffsll((unsigned long long)__ballot(lng != 0)) - 1;
            const uint32_t k = (uint32_t)__builtin_amdgcn_readlane((int)(__ffs(lng) - 1), b);
            if ((int)lane == b) lng &= lng - 1;
            const uint32_t la = (uint32_t)__builtin_amdgcn_readlane((int)pick(a, k), b);
            const uint32_t lo_ = (uint32_t)__builtin_amdgcn_readlane((int)pick(o, k), b);
            const uint32_t lc = (uint32_t)__builtin_amdgcn_readlane((int)(pick(pv, k) & PV_COUNT), b);
            const uint32_t le = pstart[p0 + g0 + k * NT + (uint32_t)b + 64u * wid + 1u];
            if (le - la <= (uint32_t)BLOCK_MAX) copy_long<SPANS>(ws, L, la, lo_, lc, out_ids, out_spans, tok_len);
        }
        // documents that start with one of this thread's pieces (every document offset below n is a
        // piece start): the first document with that offset, by binary search, and any empty ones after it
        while (dst) {
            const uint32_t k = __ffs(dst) - 1;
            dst &= dst - 1;
            const uint32_t ak = pick(a, k), ok_ = pick(o, k);
            uint32_t lo_d = dd.x, hi_d = dd.y;
            while (lo_d < hi_d) {
                const uint32_t m = (lo_d + hi_d) >> 1;
                if (offsets[m] < ak) lo_d = m + 1; else hi_d = m;
            }
            for (uint32_t d = lo_d; d < dd.y && offsets[d] == ak; ++d) out_offsets[d] = ok_;
        }
        // the multi-token pieces: listed in LDS (MLQ at a time) and copied one per thread, the loads of
        // all of them in flight together
        bool more = __syncthreads_or(pend != 0);
        while (more) {
#pragma unroll
            for (int k = 0; k < ER; ++k) {
                if ((pend >> k) & 1u) {
                    const uint32_t slot = atomicAdd(&sm.mn, 1u);
                    if (slot < (uint32_t)MLQ) {
                        sm.ma[slot] = a[k];
                        sm.mo[slot] = o[k];
                        sm.mc[slot] = pv[k] & PV_COUNT;
                        pend &= ~(1u << k);
                    }
                }
            }
            __syncthreads();
            const uint32_t mn = min(sm.mn, (uint32_t)MLQ);
            for (uint32_t i = tid; i < mn; i += NT)
                copy_ids<SPANS>(scratch, sm.ma[i], sm.mo[i], sm.mc[i], out_ids, out_spans, tok_len);
            __syncthreads();
            if (tid == 0) sm.mn = 0;
            more = __syncthreads_or(pend != 0);
        }
    }
    // the last tile: documents that start at the end of the batch (empty ones), the total
    if (t1 == n_tiles && wid == NW - 1) {
        const uint32_t d0 = wave_lower_bound(offsets, n_docs + 1, (uint64_t)n);
        for (uint32_t d = d0 + lane; d <= n_docs; d += 64) out_offsets[d] = run;
        if (lane == 0) ctrl->n_tokens = run;
    }
}

// n == 0: every document is empty
__global__ void k_tiles_empty(uint32_t n_docs, uint64_t *out_offsets, uint8_t *ws, Layout L)
{
    for (uint32_t d = threadIdx.x; d <= n_docs; d += blockDim.x) out_offsets[d] = 0;
    if (threadIdx.x == 0) ((Ctrl *)(ws + L.ctrl))->n_tokens = 0;
}

hipError_t launch_tiles(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev)
{
    const Layout &L = b.L;
    if (L.n_tiles == 0) return hipGetLastError();
    LaunchScope k(ev, TK_TILES, s);
    if (v.flags & VF_IGNORE_MERGES)
        hipLaunchKernelGGL(k_tiles<true>, dim3(L.n_tiles), dim3(NT), 0, s, v, b.bytes, b.n, b.ws, L);
    else
        hipLaunchKernelGGL(k_tiles<false>, dim3(L.n_tiles), dim3(NT), 0, s, v, b.bytes, b.n, b.ws, L);
    return hipGetLastError();
}

hipError_t launch_emit(const DevVocab &v, const Batch &b, uint32_t *out_ids, uint64_t *out_offsets,
                       uint32_t *out_spans, hipStream_t s, const Events *ev)
{
    const Layout &L = b.L;
    LaunchScope k(ev, TK_EMIT, s);
    if (L.n_tiles == 0) {
        hipLaunchKernelGGL(k_tiles_empty, dim3(1), dim3(256), 0, s, b.n_docs, out_offsets, b.ws, L);
        return hipGetLastError();
    }
    // the tiles (one or two per workgroup), then up to 32 workgroups for the giant pieces (they exit
    // at once when there are none)
    const uint32_t et = emit_tiles_per_wg(L.n_tiles);
    const uint32_t g = (L.n_tiles + et - 1) / et + (L.cap_giant < 32 ? L.cap_giant : 32);
    if (out_spans)
        hipLaunchKernelGGL(k_emit<true>, dim3(g), dim3(NT), 0, s, v, b.offsets, b.n_docs, b.n, b.ws, L, out_ids,
                           out_offsets, out_spans);
    else
        hipLaunchKernelGGL(k_emit<false>, dim3(g), dim3(NT), 0, s, v, b.offsets, b.n_docs, b.n, b.ws, L, out_ids,
                           out_offsets, out_spans);
    return hipGetLastError();
}

}  // namespace tt
