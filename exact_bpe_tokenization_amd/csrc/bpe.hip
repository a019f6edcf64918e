// bpe.hip -- stage 2: segmented byte-level BPE of every piece on gfx950.
//
// TokTier (arXiv 2607.29678), GPU BPE paragraph and Figure 6 (lower part): pieces are encoded
// independently; work is dispatched by piece length to the smallest execution unit that holds the
// piece's state; merge ranks live in device hash tables.  Two facts license the parallel schedule:
// a round's minimum rank names one pair, and merging all leftmost non-overlapping occurrences of
// that pair equals iterated single merges (for rank-consistent merge lists, which the loader
// enforces); only pairs next to a completed merge need a new lookup.
//
//   k_route       (vocabulary load) every piece: a single byte is its ID, a whole-piece table hit
//                 is its result; the others are listed by length (the tile encoder does the same for
//                 the encode chain)
//   k_giant_prep  pieces longer than 4096 bytes: every position tested for a seam no merge crosses,
//                 then (the last workgroup done with a piece) the piece cut into chunks at such seams
//   k_bpe_small   every list up to 4096 bytes, one launch with a workgroup range per list: <= 8,
//                 9..12, 13..16 and 17..32 bytes, one lane per piece and 64 consecutive list items
//                 per wavefront, the textbook loop over an LDS row per lane (leftmost lowest rank,
//                 merge, re-probe the two neighbours); 33..64 bytes, 64 lanes per piece; 65..128
//                 bytes, a wavefront with two elements per lane: rounds on ballot masks; 129..1024
//                 bytes, a wavefront per piece (four per workgroup), 1025..4096 bytes, a workgroup per
//                 piece: sequence in LDS, rounds of block minimum, selection of the leftmost
//                 non-overlapping occurrences, prefix-sum compaction, neighbour re-probes
//   k_bpe_giant   one 1024-lane workgroup per chunk longer than that; the same rounds over device
//                 memory (double-buffered); the last workgroup joins each giant piece's chunks
// Every kernel writes the piece's result word (a single ID, or the count of IDs it stored at
// scratch[piece start byte ...]; a piece never has more IDs than bytes) and adds its token count to
// the counters of its input tile (tcount) and of that tile's group of 64 tiles (tsb).
#include "internal.h"

namespace tt {

constexpr uint32_t PENDING = 0xFFFFFFFEu;

// ---------------------------------------------------------------------------------------------
// lane per piece

// k_route: every piece.  Single bytes and whole-piece table hits get their result word here; the
// others are listed for BPE by length.  Each workgroup owns a contiguous range of pieces and keeps
// RT_PPT pieces per thread in flight (their loads and table probes overlap).  List entries are queued
// in LDS and flushed with one reservation atomic per list at the end (a full queue spills straight
// to the global list).
constexpr int RT_THREADS = 512;
constexpr int RT_PPT = 2;   // pieces per thread in flight (more costs occupancy: slower)
constexpr uint32_t RTQ[NROUTES] = {1024, 512, 256, 256, 64, 64, 64, 64, 64};
constexpr uint32_t RTQ_OFF[NROUTES + 1] = {0, 1024, 1536, 1792, 2048, 2112, 2176, 2240, 2304, 2368};

// IGN: the vocabulary ignores merges (pieces longer than the whole-piece tables are looked up in the
// token string hash); a template flag so that the usual instantiation carries none of that code
template <bool IGN>
__global__ __launch_bounds__(RT_THREADS) void k_route(DevVocab v, const uint8_t *__restrict__ bytes, uint8_t *ws,
                                                      Layout L)
{
    __shared__ uint32_t q[RTQ_OFF[NROUTES]];
    __shared__ uint32_t qn[NROUTES], qbase[NROUTES];
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *__restrict__ pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *__restrict__ pval = (uint32_t *)(ws + L.pval);
    const uint32_t np = ctrl->n_pieces;
    const uint32_t tid = threadIdx.x;
    const uint32_t chunk = (np + gridDim.x - 1) / gridDim.x;
    const uint64_t start64 = (uint64_t)blockIdx.x * chunk;
    const uint32_t start = start64 < np ? (uint32_t)start64 : np;
    const uint32_t end = min(np, start + chunk);
    if (tid < NROUTES) qn[tid] = 0;
    __syncthreads();
    auto list_piece = [&](uint32_t p, uint32_t len) {
        const uint32_t r = route_of(len);
        const uint32_t slot = atomicAdd(&qn[r], 1u);
        if (slot < RTQ[r]) q[RTQ_OFF[r] + slot] = p;
        else route_list(ws, L, r)[atomicAdd(route_count(ctrl, r), 1u)] = p;
    };
    for (uint32_t p0 = start; p0 < end; p0 += RT_PPT * RT_THREADS) {
        uint32_t pp[RT_PPT], a0[RT_PPT], len[RT_PPT], id[RT_PPT], st[RT_PPT];
        WPQ q[RT_PPT];
#pragma unroll
        for (int u = 0; u < RT_PPT; ++u) {
            pp[u] = p0 + u * RT_THREADS + tid;
            const bool ok = pp[u] < end;
            a0[u] = ok ? pstart[pp[u]] : 0u;
            len[u] = ok ? pstart[pp[u] + 1] - a0[u] : 0u;
        }
#pragma unroll
        for (int u = 0; u < RT_PPT; ++u) {
            q[u] = wp_make(v, bytes + a0[u], len[u]);
            id[u] = (uint32_t)q[u].k0 & 0xFFu;   // single bytes
            st[u] = q[u].kind ? WP_MORE : (len[u] == 1 ? WP_HIT : WP_MISS);
        }
        for (;;) {
            bool more = false;
#pragma unroll
            for (int u = 0; u < RT_PPT; ++u) {
                if (st[u] == WP_MORE) st[u] = wp_step(v, q[u], &id[u]);
                more |= st[u] == WP_MORE;
            }
            if (!more) break;
        }
#pragma unroll
        for (int u = 0; u < RT_PPT; ++u) {
            if (pp[u] >= end) continue;
            if (IGN && st[u] != WP_HIT && len[u] > (uint32_t)TABLE_MAX && len[u] <= v.lmax) {
                id[u] = whole_token(v, bytes + a0[u], len[u]);
                if (id[u] != NO_PIECE) st[u] = WP_HIT;
            }
            if (st[u] == WP_HIT) pval[pp[u]] = id[u];
            else list_piece(pp[u], len[u]);
        }
    }
    __syncthreads();
    if (tid < NROUTES) {
        const uint32_t c = min(qn[tid], RTQ[tid]);
        qn[tid] = c;
        if (c) qbase[tid] = atomicAdd(route_count(ctrl, tid), c);
    }
    __syncthreads();
#pragma unroll
    for (uint32_t r = 0; r < NROUTES; ++r) {
        uint32_t *dst = route_list(ws, L, r) + qbase[r];
        for (uint32_t i = tid; i < qn[r]; i += RT_THREADS) dst[i] = q[RTQ_OFF[r] + i];
    }
}

// ---------------------------------------------------------------------------------------------
// lane per piece (unresolved pieces of <= 32 bytes)

// One item per lane, the textbook loop: merge the leftmost pair of lowest rank, re-probe its two new
// neighbour pairs.  The lane's sequence lives in its own LDS row at fixed byte positions: ranks in
// words [0, 32), elements (ID | operand bits) in [32, 64), 4 words of padding so that the 16-byte
// rank reads of 16 consecutive lanes fall on distinct banks.  A rank word is (rkx << 5) | position
// (NO_RANK at dead positions and at the last live one), so the minimum over the row is the lowest
// rank at its leftmost position in one pass; the live positions are a bit mask (a merge at p kills
// the next live position q; p's neighbours are the live positions around it).  A round is one pass of
// 16-byte LDS reads, a few bit operations, two element reads, three writes and the probes.  Called by
// all 64 lanes of a wavefront; len 0 = idle.
// Row layout of a lane unit: MAXL rank words, then (at lane_el_off) MAXL element words, padded by 4
// words against bank conflicts.  Units of up to 16 bytes take 36-word rows, 256 lanes per workgroup;
// 17..32-byte units take 68-word rows, 128 lanes per workgroup (the same LDS).
template <int MAXL> constexpr int lane_el_off() { return MAXL <= 16 ? 16 : 32; }
template <int MAXL> constexpr int lane_row_words() { return 2 * lane_el_off<MAXL>() + 4; }
template <int MAXL> constexpr uint32_t lane_unit_lanes() { return MAXL <= 16 ? 256u : 128u; }

template <int MAXL>
__device__ __forceinline__ uint32_t lane_bpe(const DevVocab &v, const uint8_t *__restrict__ bytes, uint8_t *ws,
                                             const Layout &L, uint32_t *row, uint32_t e, uint32_t b0, uint32_t len)
{
    static_assert(MAXL % 4 == 0 && MAXL <= 32, "row layout");
    uint32_t *pval = (uint32_t *)(ws + L.pval);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    uint32_t *ccount = (uint32_t *)(ws + L.ccount);
    const bool active = len != 0;
    const bool chunk = (e & CHUNK_ITEM) != 0;
    const uint32_t p = e & ~CHUNK_ITEM;
    uint32_t *el = row + lane_el_off<MAXL>();
    {
        uint64_t w[MAXL / 8 + (MAXL % 8 ? 1 : 0)];
        load_words<MAXL / 8 + (MAXL % 8 ? 1 : 0)>(bytes + b0, len, w);
        uint32_t c[MAXL + 1];
#pragma unroll
        for (int k = 0; k < MAXL; ++k) c[k] = (uint32_t)(w[k >> 3] >> (8 * (k & 7))) & 0xFFu;
        c[MAXL] = 0;
        uint32_t r[MAXL];
#pragma unroll
        for (int k = 0; k < MAXL; ++k) r[k] = (uint32_t)(k + 1) < len ? __ldg(v.r2 + ((c[k] << 8) | c[k + 1])) : NO_RANK;
#pragma unroll
        for (int k = 0; k < MAXL; k += 4) {
            uint4 x, y;
            x.x = r[k] == NO_RANK ? NO_RANK : (r[k] << 5) | k;
            x.y = r[k + 1] == NO_RANK ? NO_RANK : (r[k + 1] << 5) | (k + 1);
            x.z = r[k + 2] == NO_RANK ? NO_RANK : (r[k + 2] << 5) | (k + 2);
            x.w = r[k + 3] == NO_RANK ? NO_RANK : (r[k + 3] << 5) | (k + 3);
            y = make_uint4(c[k] | EL_BYTE, c[k + 1] | EL_BYTE, c[k + 2] | EL_BYTE, c[k + 3] | EL_BYTE);
            *(uint4 *)(row + k) = x;
            *(uint4 *)(el + k) = y;
        }
    }
    uint32_t live = len >= 32 ? 0xFFFFFFFFu : (1u << len) - 1u;
    for (;;) {
        uint32_t best = NO_RANK;
#pragma unroll
        for (int k = 0; k < MAXL; k += 4) {
            const uint4 x = *(const uint4 *)(row + k);
            best = min(best, min(min(x.x, x.y), min(x.z, x.w)));
        }
        if (best == NO_RANK) break;
        const uint32_t pos = best & 31u, nid = merged_element(best >> 5);
        const uint32_t above = ~((2u << pos) - 1u);             // positions > pos (none when pos = 31)
        const uint32_t q = (uint32_t)__ffs(live & above) - 1u;   // the right element of the pair
        live &= ~(1u << q);
        const uint32_t lo = live & ((1u << pos) - 1u), hi = live & above;
        const uint32_t l = lo ? 31u - (uint32_t)__clz(lo) : 0u, r = hi ? (uint32_t)__ffs(hi) - 1u : 0u;
        const uint32_t idl = lo ? el[l] : 0u, idr = hi ? el[r] : 0u;
        el[pos] = nid;
        row[q] = NO_RANK;
        uint32_t rl, rr;   // both neighbours' probes in one round trip (nid >= 256: no byte pair)
        pair_rkx2(v, idl & ID_MASK, nid & ID_MASK, lo && may_merge(idl, nid), nid & ID_MASK, idr & ID_MASK,
                  hi && may_merge(nid, idr), rl, rr);
        if (lo) row[l] = rl == NO_RANK ? NO_RANK : (rl << 5) | l;
        row[pos] = rr == NO_RANK ? NO_RANK : (rr << 5) | pos;
    }
    const uint32_t n = (uint32_t)__popc(live & (len >= 32 ? 0xFFFFFFFFu : (1u << len) - 1u));
    if (n > 1 || chunk) {
        uint32_t t = 0;
#pragma unroll
        for (int k = 0; k < MAXL; k += 4) {
            const uint4 x = *(const uint4 *)(el + k);
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((uint32_t)(k + j) < len && ((live >> (k + j)) & 1u)) scratch[b0 + t++] = xs[j] & ID_MASK;
        }
    }
    if (active && chunk) ccount[p] = n;
    else if (active) pval[p] = n == 1 ? el[0] & ID_MASK : (PV_MULTI | n);
    return active ? n : 0u;
}

// A list of <= 32-byte items (r: <= 8, 9..12, 13..16 or 17..32 bytes, MAXL its longest), 64 consecutive
// items per wavefront.  The tile encoder lists each tile's pieces in one run, so a wavefront's pieces
// mostly share one or two input tiles and its token counts take that many atomics.
template <int MAXL>
__device__ __forceinline__ void bpe_lane(const DevVocab &v, const uint8_t *__restrict__ bytes, uint8_t *ws, const Layout &L,
                         uint32_t *rows, uint32_t r, uint32_t blk, uint32_t nblk)
{
    constexpr uint32_t LANES = lane_unit_lanes<MAXL>();
    if (threadIdx.x >= LANES) return;   // (whole wavefronts)
    uint32_t *row = rows + threadIdx.x * lane_row_words<MAXL>();
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *list = route_list(ws, L, r);
    const uint32_t count = ctrl->miss_count[r];
    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *clen = (const uint32_t *)(ws + L.clen);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (blk * LANES + threadIdx.x) >> 6;
    const uint32_t nwaves = (nblk * LANES) >> 6;
    for (uint32_t q0 = wave * 64u; q0 < count; q0 += nwaves * 64u) {   // wavefront-uniform
        const uint32_t q = q0 + lane;
        uint32_t e = 0, b0 = 0, len = 0;
        if (q < count) {
            e = list[q];
            const uint32_t p = e & ~CHUNK_ITEM;
            if (e & CHUNK_ITEM) { b0 = cstart[p]; len = clen[p]; }
            else { b0 = pstart[p]; len = pstart[p + 1] - b0; }
        }
        const uint32_t n = lane_bpe<MAXL>(v, bytes, ws, L, row, e, b0, len);
        add_tile_tokens(ws, L, b0, (e & CHUNK_ITEM) ? 0u : n);
    }
}

// ---------------------------------------------------------------------------------------------
// G lanes per piece (G = 16, 32 or 64; 64 / G pieces per wavefront), element k of a piece in lane
// k of its segment.  One round per distinct minimum rank, everything in registers:
//   segment minimum of the pair ranks (xor butterfly inside the segment),
//   H = ballot of the pairs holding it,
//   leftmost non-overlapping selection in closed form on H: a chain of consecutive hits (only a
//   pair (x, x) makes one) keeps the hits at an even distance from its first hit,
//   keep mask K = valid lanes that are not the right half of a selected pair, new position =
//   popcount of K below the lane inside its segment (a permutation of the segment: dropped lanes
//   go after the kept ones), moved with ds_permute,
//   re-probe of the pairs whose left or right element was merged.
// A segment never spills into the next one: its last element has no pair, so chains and
// selections stay inside it.

__device__ __forceinline__ uint32_t lane_push(uint32_t dst_lane, uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_ds_permute((int)(dst_lane << 2), (int)x);
}

template <int G>
__device__ __forceinline__ void bpe_seg(const DevVocab &v, const uint8_t *__restrict__ bytes, uint8_t *ws, const Layout &L, uint32_t r,
                        uint32_t blk, uint32_t nblk)
{
    static_assert(G == 16 || G == 32 || G == 64, "segment width");
    constexpr uint32_t SEGS = 64 / G;
    constexpr uint64_t EVEN = 0x5555555555555555ull, ODD = ~EVEN;
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *pval = (uint32_t *)(ws + L.pval);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    const uint32_t *list = route_list(ws, L, r);
    const uint32_t count = ctrl->miss_count[r];
    const uint32_t lane = threadIdx.x & 63u, seg = lane / G, k = lane % G, sbase = seg * G;
    const uint64_t segmask = G == 64 ? ~0ull : (((1ull << (G % 64)) - 1ull) << sbase);
    const uint64_t below = (1ull << lane) - 1ull;
    const uint32_t wave = (blk * blockDim.x + threadIdx.x) >> 6;
    const uint32_t nwaves = (nblk * blockDim.x) >> 6;

    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *clen = (const uint32_t *)(ws + L.clen);
    uint32_t *ccount = (uint32_t *)(ws + L.ccount);
    for (uint32_t q0 = wave * SEGS; q0 < count; q0 += nwaves * SEGS) {
        const uint32_t q = q0 + seg;
        uint32_t p = 0, b0 = 0, n = 0;
        bool chunk = false;
        if (q < count) {
            const uint32_t e = list[q];
            chunk = (e & CHUNK_ITEM) != 0;
            p = e & ~CHUNK_ITEM;
            b0 = chunk ? cstart[p] : pstart[p];
            n = chunk ? clen[p] : pstart[p + 1] - b0;   // up to G bytes
        }
        uint32_t id = k < n ? (uint32_t)bytes[b0 + k] : 0u;
        uint32_t nx = wave_next(id);
        uint32_t rk = k + 1 < n ? __ldg(v.r2 + ((id << 8) | nx)) : NO_RANK;
        id |= EL_BYTE;
        for (;;) {
            uint32_t m = rk;
            if (G == 64) m = wave_min(m);
            else if (G == 16) m = row_min16(m);
            else {
#pragma unroll
                for (int d = G / 2; d >= 1; d >>= 1) m = min(m, (uint32_t)__shfl_xor(m, d, 64));
            }
            const uint64_t H = __ballot(rk == m && m != NO_RANK);
            if (H == 0) break;
            const uint64_t rsE = H & ~(H << 1) & EVEN;          // chains starting at an even lane
            const uint64_t runsE = H & ~(H + rsE);              // the hits of those chains
            const uint64_t sel = (runsE & EVEN) | (H & ~runsE & ODD);
            const uint64_t K = __ballot(k < n) & ~(sel << 1);
            const bool me_sel = (sel >> lane) & 1u;
            const bool nx_sel = lane < 63 && ((sel >> (lane + 1)) & 1u);
            const uint32_t kept_seg = (uint32_t)__popcll(K & segmask);
            const uint32_t dst = ((K >> lane) & 1u)
                                     ? sbase + (uint32_t)__popcll(K & segmask & below)
                                     : sbase + kept_seg + (uint32_t)__popcll(~K & segmask & below);
            id = lane_push(dst, me_sel ? merged_element(m) : id);
            rk = lane_push(dst, (me_sel || nx_sel) ? PENDING : rk);
            n = kept_seg;
            nx = wave_next(id);
            if (k >= n) rk = NO_RANK;
            else if (rk == PENDING) rk = k + 1 < n ? element_rkx(v, id, nx) : NO_RANK;
        }
        id &= ID_MASK;
        if (k < n && (n > 1 || chunk)) scratch[b0 + k] = id;
        const bool head = k == 0 && q < count;
        if (head && chunk) ccount[p] = n;
        else if (head) pval[p] = n == 1 ? id : (PV_MULTI | n);
        // the segments' counts, moved to lanes 0 .. SEGS - 1 so that equal tiles are adjacent
        const uint32_t src = (lane % SEGS) * G;
        const uint32_t x = __shfl((head && !chunk) ? n : 0u, (int)src, 64), xb = __shfl(b0, (int)src, 64);
        add_tile_tokens(ws, L, xb, lane < SEGS ? x : 0u);
    }
}

// One wavefront per piece of 65..SEG2_MAX bytes, two elements per lane (element e in lane e % 64 of
// row e / 64): the rounds of k_bpe_seg on 128-bit masks (two ballots; shifts and the addition carry
// between the words), compaction through a 128-entry LDS row per wavefront (a wavefront's LDS
// accesses are performed in order, so no barrier is needed).

__device__ __forceinline__ void shl128(uint64_t lo, uint64_t hi, uint64_t &rlo, uint64_t &rhi)
{
    rhi = (hi << 1) | (lo >> 63);
    rlo = lo << 1;
}

__device__ __forceinline__ void bpe_seg2(const DevVocab &v, const uint8_t *__restrict__ bytes, uint8_t *ws, const Layout &L,
                         uint32_t blk, uint32_t nblk)
{
    constexpr uint64_t EVEN = 0x5555555555555555ull, ODD = ~EVEN;
    __shared__ uint32_t sid[4][2 * 64], srk[4][2 * 64];
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *pval = (uint32_t *)(ws + L.pval);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    const uint32_t *list = route_list(ws, L, 5);
    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *clen = (const uint32_t *)(ws + L.clen);
    uint32_t *ccount = (uint32_t *)(ws + L.ccount);
    const uint32_t count = ctrl->miss_count[5];
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t below = (1ull << lane) - 1ull;
    const uint32_t wave = (blk * blockDim.x + threadIdx.x) >> 6;
    const uint32_t nwaves = (nblk * blockDim.x) >> 6;
    for (uint32_t q = wave; q < count; q += nwaves) {
        const uint32_t e = list[q];
        const bool chunk = (e & CHUNK_ITEM) != 0;
        const uint32_t p = e & ~CHUNK_ITEM;
        const uint32_t b0 = chunk ? cstart[p] : pstart[p];
        uint32_t n = chunk ? clen[p] : pstart[p + 1] - b0;   // up to 128 bytes
        uint32_t id0 = lane < n ? (uint32_t)bytes[b0 + lane] : 0u;
        uint32_t id1 = 64 + lane < n ? (uint32_t)bytes[b0 + 64 + lane] : 0u;
        uint32_t nx0 = wave_next(id0), nx1 = wave_next(id1);
        if (lane == 63) nx0 = (uint32_t)__builtin_amdgcn_readlane((int)id1, 0);
        uint32_t rk0 = lane + 1 < n ? __ldg(v.r2 + ((id0 << 8) | nx0)) : NO_RANK;
        uint32_t rk1 = 65 + lane < n ? __ldg(v.r2 + ((id1 << 8) | nx1)) : NO_RANK;
        id0 |= EL_BYTE;
        id1 |= EL_BYTE;
        for (;;) {
            uint32_t m = min(rk0, rk1);
            m = wave_min(m);
            if (m == NO_RANK) break;
            const uint64_t H0 = __ballot(rk0 == m), H1 = __ballot(rk1 == m);
            uint64_t s0, s1;
            shl128(H0, H1, s0, s1);
            const uint64_t rsE0 = H0 & ~s0 & EVEN, rsE1 = H1 & ~s1 & EVEN;
            const uint64_t a0 = H0 + rsE0;
            const uint64_t a1 = H1 + rsE1 + (a0 < H0 ? 1ull : 0ull);
            const uint64_t runsE0 = H0 & ~a0, runsE1 = H1 & ~a1;
            const uint64_t sel0 = (runsE0 & EVEN) | (H0 & ~runsE0 & ODD);
            const uint64_t sel1 = (runsE1 & EVEN) | (H1 & ~runsE1 & ODD);
            uint64_t l0, l1;
            shl128(sel0, sel1, l0, l1);
            const uint64_t K0 = __ballot(lane < n) & ~l0, K1 = __ballot(64 + lane < n) & ~l1;
            const bool ms0 = (sel0 >> lane) & 1u, ms1 = (sel1 >> lane) & 1u;
            const bool ns0 = lane < 63 ? ((sel0 >> (lane + 1)) & 1u) : (sel1 & 1u);
            const bool ns1 = lane < 63 && ((sel1 >> (lane + 1)) & 1u);
            const uint32_t k0 = (uint32_t)__popcll(K0);
            if ((K0 >> lane) & 1u) {
                const uint32_t o = (uint32_t)__popcll(K0 & below);
                sid[w][o] = ms0 ? merged_element(m) : id0;
                srk[w][o] = (ms0 || ns0) ? PENDING : rk0;
            }
            if ((K1 >> lane) & 1u) {
                const uint32_t o = k0 + (uint32_t)__popcll(K1 & below);
                sid[w][o] = ms1 ? merged_element(m) : id1;
                srk[w][o] = (ms1 || ns1) ? PENDING : rk1;
            }
            n = k0 + (uint32_t)__popcll(K1);
            id0 = sid[w][lane];
            rk0 = srk[w][lane];
            id1 = sid[w][64 + lane];
            rk1 = srk[w][64 + lane];
            nx0 = wave_next(id0);
            nx1 = wave_next(id1);
            if (lane == 63) nx0 = (uint32_t)__builtin_amdgcn_readlane((int)id1, 0);
            if (rk0 == PENDING || rk1 == PENDING) {
                // both rows' probes in one round trip; a pending pair holds a merged token (>= 256); a
                // row is probed only when it is pending and the operand bits allow a merge
                uint32_t q0, q1;
                pair_rkx2(v, id0 & ID_MASK, nx0 & ID_MASK, rk0 == PENDING && may_merge(id0, nx0), id1 & ID_MASK,
                          nx1 & ID_MASK, rk1 == PENDING && may_merge(id1, nx1), q0, q1);
                if (rk0 == PENDING) rk0 = q0;
                if (rk1 == PENDING) rk1 = q1;
            }
            if (lane + 1 >= n) rk0 = NO_RANK;
            if (65 + lane >= n) rk1 = NO_RANK;
        }
        id0 &= ID_MASK;
        id1 &= ID_MASK;
        if (n > 1 || chunk) {
            if (lane < n) scratch[b0 + lane] = id0;
            if (64 + lane < n) scratch[b0 + 64 + lane] = id1;
        }
        if (lane == 0) {
            if (chunk) ccount[p] = n;
            else pval[p] = n == 1 ? id0 : (PV_MULTI | n);
        }
        add_tile_tokens(ws, L, b0, (lane == 0 && !chunk) ? n : 0u);
    }
}

// ---------------------------------------------------------------------------------------------
// workgroup primitives (NT threads, NT a multiple of 64)

template <int NT>
__device__ __forceinline__ uint32_t block_min(uint32_t x, uint32_t *red)
{
    x = wave_min(x);
    if (NT == 64) return x;
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = x;
    __syncthreads();
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = min(r, red[w]);
    __syncthreads();
    return r;
}

// exclusive sum; *total receives the block total
template <int NT>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t x, uint32_t *red, uint32_t *total)
{
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(inc, d, 64);
        if (lane >= (uint32_t)d) inc += y;
    }
    if (NT == 64) {
        *total = __shfl(inc, 63, 64);
        return inc - x;
    }
    if (lane == 63) red[wid] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        uint32_t r = red[w];
        if ((uint32_t)w < wid) before += r;
        tot += r;
    }
    __syncthreads();
    *total = tot;
    return before + inc - x;
}

// exclusive max over threads of int32 values (identity -1)
template <int NT>
__device__ __forceinline__ int32_t block_excl_max(int32_t x, int32_t *red)
{
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    int32_t inc = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int32_t y = __shfl_up(inc, d, 64);
        if (lane >= (uint32_t)d) inc = max(inc, y);
    }
    int32_t ex = __shfl_up(inc, 1, 64);
    if (lane == 0) ex = -1;
    if (NT == 64) return ex;
    if (lane == 63) red[wid] = inc;
    __syncthreads();
    int32_t before = -1;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
        if ((uint32_t)w < wid) before = max(before, red[w]);
    __syncthreads();
    return max(before, ex);
}

// ---------------------------------------------------------------------------------------------
// piece per wavefront / workgroup, sequence in LDS

// barrier of a unit: the workgroup, or (NT = 64) the unit's own wavefront, so that the wavefronts of a
// workgroup can work on different pieces
template <int NT>
__device__ __forceinline__ void unit_sync()
{
    if (NT == 64) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        __syncthreads();
    }
}

// LDS of one workgroup unit: ids, ranks, selection bytes and the reduction slots
template <int NT, int MAXN>
constexpr uint32_t block_unit_lds()
{
    return 4u * MAXN + 4u * MAXN + ((MAXN + 1 + 15) & ~15) + 4u * (NT / 64 + 1) + 4u * (NT / 64 + 1);
}

// One unit of NT lanes (a workgroup, or one wavefront of it when NT = 64) per piece of list `bin` (0:
// 129..WAVE_MAX bytes, 1: ..BLOCK_MAX bytes) and per chunk of a giant piece in the same size range;
// unit blk of nblk.  `smem` holds the unit's block_unit_lds bytes.
template <int NT, int MAXN>
__device__ __forceinline__ void bpe_block(const DevVocab &v, const uint8_t *__restrict__ bytes, uint8_t *ws, const Layout &L, int bin,
                          uint8_t *smem, uint32_t blk, uint32_t nblk)
{
    constexpr int E = MAXN / NT;
    static_assert(E <= 32, "selection masks are 32-bit");
    uint32_t *sid = (uint32_t *)smem;
    uint32_t *srk = sid + MAXN;
    uint8_t *ssel = (uint8_t *)(srk + MAXN);
    uint32_t *red = (uint32_t *)(ssel + ((MAXN + 1 + 15) & ~15));
    int32_t *redi = (int32_t *)(red + (NT / 64 + 1));

    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *pval = (uint32_t *)(ws + L.pval);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    const uint32_t *list = (const uint32_t *)(ws + (bin == 0 ? L.bin_wave : L.bin_block));
    const uint32_t count = ctrl->bin_count[bin];
    // chunks of giant pieces of this kernel's size range come after the bin's pieces (their results
    // go to ccount): up to WAVE_MAX bytes for the wavefront kernel, up to BLOCK_MAX for the other
    const uint32_t n_chunks = ctrl->n_chunks;
    const uint32_t cmin = bin == 0 ? (uint32_t)SEG2_MAX + 1u : (uint32_t)WAVE_MAX + 1u;
    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *clen = (const uint32_t *)(ws + L.clen);
    uint32_t *ccount = (uint32_t *)(ws + L.ccount);
    const uint32_t tid = threadIdx.x % NT;
    const uint32_t k0 = tid * E;

    for (uint32_t q = blk; q < count + n_chunks; q += nblk) {
        const bool is_chunk = q >= count;
        uint32_t p = 0, b0, n;
        if (!is_chunk) {
            p = list[q];
            b0 = pstart[p];
            n = pstart[p + 1] - b0;
        } else {
            b0 = cstart[q - count];
            n = clen[q - count];
            if (n < cmin || n > (uint32_t)MAXN) continue;   // unused slot, or a chunk for another kernel
        }
        if ((v.flags & VF_IGNORE_MERGES) && !is_chunk && n <= v.lmax) {
            // ignore_merges: a piece that is a token's byte string is that token
            if (tid == 0) red[0] = whole_token(v, bytes + b0, n);
            unit_sync<NT>();
            const uint32_t w = red[0];
            unit_sync<NT>();
            if (w != NO_PIECE) {
                if (tid == 0) {
                    scratch[b0] = w;
                    put_piece(ws, L, p, b0, 1u, 0u, true);
                }
                continue;
            }
        }
        for (uint32_t k = tid; k < n; k += NT) sid[k] = bytes[b0 + k];
        unit_sync<NT>();
        for (uint32_t k = tid; k < n; k += NT)
            srk[k] = k + 1 < n ? rkx_rank(__ldg(v.r2 + ((sid[k] << 8) | sid[k + 1]))) : NO_RANK;
        unit_sync<NT>();
        for (;;) {
            uint32_t lmin = NO_RANK;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (k0 + e < n) lmin = min(lmin, srk[k0 + e]);
            const uint32_t rmin = block_min<NT>(lmin, red);
            if (rmin >= v.n_merges) break;   // NO_RANK: nothing left to merge
            uint32_t hitm = 0;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (k0 + e < n && srk[k0 + e] == rmin) hitm |= 1u << e;
            uint32_t selm = hitm;
            {
                // leftmost non-overlapping occurrences: consecutive hits only arise for a pair (x, x);
                // inside each chain of consecutive hits keep the ones at an even distance from the
                // chain's start (for any other pair every hit starts its own chain)
                const bool prev_hit = k0 >= 1 && k0 - 1 < n && srk[k0 - 1] == rmin;
                int32_t last_start = -1;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    bool h = (hitm >> e) & 1u, hp = e ? ((hitm >> (e - 1)) & 1u) : prev_hit;
                    if (h && !hp) last_start = (int32_t)(k0 + e);
                }
                int32_t cs = block_excl_max<NT>(last_start, redi);
                selm = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    bool h = (hitm >> e) & 1u, hp = e ? ((hitm >> (e - 1)) & 1u) : prev_hit;
                    if (h && !hp) cs = (int32_t)(k0 + e);
                    if (h && (((int32_t)(k0 + e) - cs) & 1) == 0) selm |= 1u << e;
                }
            }
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (k0 + e < n) ssel[k0 + e] = (selm >> e) & 1u;
            if (tid == 0) ssel[n] = 0;
            unit_sync<NT>();
            // keep = not the right half of a selected pair
            uint32_t keepm = 0, cnt = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                uint32_t k = k0 + e;
                if (k < n && !(k >= 1 && ssel[k - 1])) { keepm |= 1u << e; ++cnt; }
            }
            uint32_t nnew;
            const uint32_t off = block_excl_sum<NT>(cnt, red, &nnew);
            uint32_t nid[E], nrk[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                uint32_t k = k0 + e;
                nid[e] = 0;
                nrk[e] = NO_RANK;
                if ((keepm >> e) & 1u) {
                    bool s = (selm >> e) & 1u;
                    nid[e] = s ? 256u + rmin : sid[k];
                    nrk[e] = (s || ssel[k + 1]) ? PENDING : srk[k];
                }
            }
            unit_sync<NT>();
            uint32_t o = off;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((keepm >> e) & 1u) { sid[o] = nid[e]; srk[o] = nrk[e]; ++o; }
            unit_sync<NT>();
            for (uint32_t j = off; j < off + cnt; ++j)
                if (srk[j] == PENDING) srk[j] = j + 1 < nnew ? pair_rank(v, sid[j], sid[j + 1]) : NO_RANK;
            unit_sync<NT>();
            n = nnew;
        }
        for (uint32_t k = tid; k < n; k += NT) scratch[b0 + k] = sid[k];
        if (tid == 0) {
            if (is_chunk) ccount[q - count] = n;
            else put_piece(ws, L, p, b0, n, 0u, true);
        }
        unit_sync<NT>();
    }
}

// The lists of short unresolved pieces are independent and each role above is bound by its
// dependent table probes, so they run as one launch: the workgroups are split into six ranges, one
// per list, and all of them progress at the same time.
__global__ __launch_bounds__(256) void k_bpe_small(DevVocab v, const uint8_t *__restrict__ bytes, uint8_t *ws, Layout L,
                                                  uint32_t gb, uint32_t gw, uint32_t g8, uint32_t g12, uint32_t g16,
                                                  uint32_t g32, uint32_t g64, uint32_t g128)
{
    // the lane units' rows; the workgroup units' sequences (one allocation).  With the 65..128-byte
    // units' rows the launch takes 41,088 B of LDS: three workgroups per CU.  Four per CU (those
    // rows carved out of this area) measured slower on the 18.4 MB batch, 66.8 -> 71.4 us: the
    // launch is bound per CU, and four workgroups pack the working ones onto fewer CUs.
    constexpr uint32_t WAVE_UNIT = (block_unit_lds<64, WAVE_MAX>() + 15u) & ~15u;
    constexpr uint32_t LANE_LDS = 4u * lane_row_words<16>() * lane_unit_lanes<16>();
    static_assert(4u * lane_row_words<32>() * lane_unit_lanes<32>() <= LANE_LDS, "lane rows");
    constexpr uint32_t BLOCK_LDS = (block_unit_lds<256, BLOCK_MAX>() + 15u) & ~15u;
    constexpr uint32_t SMEM0 = LANE_LDS > BLOCK_LDS ? LANE_LDS : BLOCK_LDS;
    constexpr uint32_t SMEM = SMEM0 > 4 * WAVE_UNIT ? SMEM0 : 4 * WAVE_UNIT;
    static_assert(SMEM <= 40960, "unit area within 40 KiB");
    __shared__ __align__(16) uint32_t rows[SMEM / 4];
    // workgroup ranges in order of the units' round counts (longest first): workgroups are dispatched
    // in order, so the long chains start at once and the many short ones fill in around them.  The
    // ranges are cut to what the lists hold (the grid is sized for the largest possible lists), so
    // that the workgroups with work come first and the idle ones are dispatched last.
    {
        const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
        const uint32_t *cnt = ctrl->miss_count;
        const uint32_t nch = ctrl->n_chunks;       // (chunk slots: every list's unit looks at them)
        gb = min(gb, ctrl->bin_count[1] + nch);    // a piece per workgroup
        gw = min(gw, (ctrl->bin_count[0] + nch + 3u) / 4u);   // a piece per wavefront
        g128 = min(g128, (cnt[5] + 3u) / 4u);     // a piece per wavefront
        g64 = min(g64, (cnt[4] + 3u) / 4u);
        g32 = min(g32, (cnt[3] + 127u) / 128u);   // a piece per lane (128 lanes per workgroup)
        g16 = min(g16, (cnt[2] + 255u) / 256u);
        g12 = min(g12, (cnt[1] + 255u) / 256u);
        g8 = min(g8, (cnt[0] + 255u) / 256u);
    }
    uint32_t b = blockIdx.x;
    if (b < gb) {
        bpe_block<256, BLOCK_MAX>(v, bytes, ws, L, 1, (uint8_t *)rows, b, gb);
    } else if ((b -= gb) < gw) {
        const uint32_t w = threadIdx.x >> 6;
        bpe_block<64, WAVE_MAX>(v, bytes, ws, L, 0, (uint8_t *)rows + w * WAVE_UNIT, 4 * b + w, 4 * gw);
    } else if ((b -= gw) < g128) {
        bpe_seg2(v, bytes, ws, L, b, g128);
    } else if ((b -= g128) < g64) {
        bpe_seg<64>(v, bytes, ws, L, 4, b, g64);
    } else if ((b -= g64) < g32) {
        bpe_lane<32>(v, bytes, ws, L, rows, 3, b, g32);
    } else if ((b -= g32) < g16) {
        bpe_lane<16>(v, bytes, ws, L, rows, 2, b, g16);
    } else if ((b -= g16) < g12) {
        bpe_lane<12>(v, bytes, ws, L, rows, 1, b, g12);
    } else if ((b -= g12) < g8) {
        bpe_lane<8>(v, bytes, ws, L, rows, 0, b, g8);
    }
}

// ---------------------------------------------------------------------------------------------
// giant pieces: seams no merge can cross.  A merge that would join bytes on both sides of position
// j joins a token x ending at j with a token y starting at j, so if no pair (x, y) of such tokens
// has a rank, BPE never merges across j and the piece's IDs are those of its two sides encoded on
// their own, concatenated (merges on one side never change the tokens on the other).  Every token
// whose byte string is a suffix (prefix) of the text before (after) j is found through the token
// string hash, duplicates included; a candidate with more than SEAM_MAXT of either is rejected.

constexpr int SEAM_MAXT = 8;

// may the piece s[0, n) be cut before byte j (0 < j < n)?  Tokens ending at j are collected first;
// each token starting at j is checked against them as soon as it is found.
__device__ bool seam_safe(const DevVocab &v, const uint8_t *s, uint32_t n, uint32_t j)
{
    uint32_t xs[SEAM_MAXT];
    uint32_t nx = 0;
    bool over = false;
    uint64_t h = 0, pw = 1;
    const uint32_t lx = min(v.lmax, j), ly = min(v.lmax, n - j);
    for (uint32_t l = 1; l <= lx && !over; ++l) {
        h += (uint64_t)s[j - l] * pw;
        pw *= STR_P;
        str_find(v, s + j - l, l, str_key(h, l), [&](uint32_t id) {
            if (nx < (uint32_t)SEAM_MAXT) xs[nx++] = id;
            else over = true;
        });
    }
    if (over) return false;
    bool ranked = false;
    h = 0;
    for (uint32_t l = 1; l <= ly && !ranked; ++l) {
        h = h * STR_P + s[j + l - 1];
        str_find(v, s + j, l, str_key(h, l), [&](uint32_t id) {
            for (uint32_t a = 0; a < nx && !ranked; ++a) ranked = pair_rank(v, xs[a], id) != NO_RANK;
        });
    }
    return !ranked;
}

// Safe-seam bitmap of the giant pieces: bit (a % 32) of word a / 32 + b0 / 4096 says the piece
// starting at byte b0 may be cut before byte a (b0 < a < b0 + n).  The b0 / 4096 term keeps the
// words of two giant pieces (each longer than 4096 bytes) apart.
__device__ __forceinline__ uint32_t safe_word(uint32_t a, uint32_t b0)
{
    return a / 32 + b0 / 4096;
}

// first and last safe position of window [lo, hi) of the piece at b0 (NO_PIECE if none); lo > b0
__device__ __forceinline__ void window_safe(const uint32_t *bm, uint32_t b0, uint32_t lo, uint32_t hi, uint32_t &f,
                                            uint32_t &l)
{
    f = l = NO_PIECE;
    for (uint32_t w = lo / 32; w * 32 < hi; ++w) {
        uint32_t bits = bm[safe_word(w * 32, b0)];
        if (w == lo / 32) bits &= ~0u << (lo % 32);
        if (w == hi / 32) bits &= (hi % 32) ? ((1u << (hi % 32)) - 1u) : 0u;
        if (!bits) continue;
        if (f == NO_PIECE) f = w * 32 + (uint32_t)__ffs(bits) - 1u;
        l = w * 32 + 31u - (uint32_t)__clz(bits);
    }
}

// giant_cut: a workgroup of 1024 turns piece g's bitmap into chunks.  The piece is divided into
// windows of GCH positions; every window with a safe position is cut at its first one (chunks of
// about GCH bytes where seams are common), and a window followed by one without any safe position
// is also cut at its last one, so that a stretch without seams (typically a repeated character,
// which needs few merge rounds) is a chunk of its own.  Cuts come out sorted; a workgroup scan
// places them.  Chunks take consecutive slots of the chunk table (unused reserved slots: length 0);
// chunks of up to SEG2_MAX bytes are also listed for the lane and segment kernels.
__device__ __forceinline__ void giant_cut(const DevVocab &v, uint8_t *ws, const Layout &L, uint32_t g)
{
    constexpr uint32_t NT = 1024, NW = NT / 64;
    __shared__ uint32_t swsum[NW];
    __shared__ uint32_t s_c0, s_nc;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *list = (const uint32_t *)(ws + L.bin_giant);
    const uint32_t *bm = (const uint32_t *)(ws + L.gsafe);
    uint32_t *cstart = (uint32_t *)(ws + L.cstart), *clen = (uint32_t *)(ws + L.clen);
    uint32_t *gc0 = (uint32_t *)(ws + L.gc0), *gnc = (uint32_t *)(ws + L.gnc);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    {
        const uint32_t p = list[g];
        const uint32_t b0 = pstart[p], n = pstart[p + 1] - b0, end = b0 + n;
        const uint32_t nwin = v.str ? (n + GCH - 1) / GCH : 0u;
        const uint32_t reserve = 2 * nwin + 2;
        if (tid == 0) {
            s_c0 = atomicAdd(&ctrl->n_chunks, reserve);
            cstart[s_c0] = b0;
            s_nc = 1;
        }
        __syncthreads();
        const uint32_t c0 = s_c0;
        for (uint32_t k0 = 0; k0 < nwin; k0 += NT) {
            const uint32_t k = k0 + tid;
            uint32_t f = NO_PIECE, l = NO_PIECE, fn = NO_PIECE, ln;
            if (k < nwin) {
                window_safe(bm, b0, max(b0 + 1, b0 + k * GCH), min(end, b0 + (k + 1) * GCH), f, l);
                if (k + 1 < nwin) window_safe(bm, b0, b0 + (k + 1) * GCH, min(end, b0 + (k + 2) * GCH), fn, ln);
            }
            const bool cf = k >= 1 && f != NO_PIECE;
            const bool cl = l != NO_PIECE && k + 1 < nwin && fn == NO_PIECE && !(cf && l == f);
            const uint32_t e = (cf ? 1u : 0u) + (cl ? 1u : 0u);
            uint32_t inc = e;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t y = __shfl_up(inc, d, 64);
                if (lane >= (uint32_t)d) inc += y;
            }
            if (lane == 63) swsum[wid] = inc;
            __syncthreads();
            uint32_t before = s_nc, tot = 0;
            for (uint32_t w = 0; w < NW; ++w) {
                if (w < wid) before += swsum[w];
                tot += swsum[w];
            }
            uint32_t o = before + inc - e;
            if (cf) cstart[c0 + o++] = f;
            if (cl) cstart[c0 + o] = l;
            __syncthreads();
            if (tid == 0) s_nc += tot;
            __syncthreads();
        }
        __threadfence();   // chunk starts are read by other threads below
        __syncthreads();
        const uint32_t nc = s_nc;
        // lengths; chunks of up to SEG2_MAX bytes also go to the BPE lists (one atomic per list and
        // wavefront step), longer ones are found in the table by the workgroup kernels
        for (uint32_t i0 = wid * 64; i0 < reserve; i0 += NT) {
            const uint32_t i = i0 + lane;
            const uint32_t len = i < nc ? (i + 1 < nc ? cstart[c0 + i + 1] : end) - cstart[c0 + i] : 0u;
            if (i < reserve) {
                clen[c0 + i] = len;
                ((uint32_t *)(ws + L.cpiece))[c0 + i] = i < nc ? p : NO_PIECE;
            }
            const uint32_t r = len >= 1 && len <= (uint32_t)SEG2_MAX ? route_of(len) : NMISS;
#pragma unroll
            for (uint32_t rl = 0; rl < NMISS; ++rl) {
                const uint64_t m = __ballot(r == rl);
                if (!m) continue;
                const uint32_t leader = (uint32_t)__ffsll((unsigned long long)m) - 1u;
                uint32_t base = 0;
                if (lane == leader) base = atomicAdd(&ctrl->miss_count[rl], (uint32_t)__popcll(m));
                base = __shfl(base, (int)leader, 64);
                if (r == rl)
                    route_list(ws, L, rl)[base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull))] = CHUNK_ITEM | (c0 + i);
            }
        }
        if (tid == 0) {
            gc0[g] = c0;
            gnc[g] = nc;
        }
        __syncthreads();
    }
}

// k_giant_prep: every position of every giant piece is tested for a seam, the workgroups sharing out
// 1024-position blocks (aligned to absolute positions) of each piece in turn; the last workgroup to
// finish its blocks of a piece (a counter per piece, cleared by the summary kernel) cuts it.  Without
// the token string hash (no seams) each piece is one chunk, cut by workgroup g mod grid.
__global__ __launch_bounds__(1024) void k_giant_prep(DevVocab v, const uint8_t *__restrict__ bytes, uint8_t *ws, Layout L)
{
    __shared__ uint32_t s_last;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *list = (const uint32_t *)(ws + L.bin_giant);
    uint32_t *bm = (uint32_t *)(ws + L.gsafe);
    uint32_t *gdone = (uint32_t *)(ws + L.gdone);
    const uint32_t count = ctrl->bin_count[2];
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    if (count == 0) return;
    if (!v.str) {
        for (uint32_t g = blockIdx.x; g < count; g += gridDim.x) giant_cut(v, ws, L, g);
        return;
    }
    for (uint32_t g = 0; g < count; ++g) {
        const uint32_t p = list[g];
        const uint32_t b0 = pstart[p], n = pstart[p + 1] - b0;
        const uint32_t first = b0 / 1024, last = (b0 + n - 1) / 1024, nb = last - first + 1;
        if (blockIdx.x >= nb) continue;   // no block of this piece for this workgroup
        for (uint32_t blk = first + blockIdx.x; blk <= last; blk += gridDim.x) {
            const uint32_t a = blk * 1024 + tid;
            const bool ok = a > b0 && a < b0 + n && seam_safe(v, bytes + b0, n, a - b0);
            const uint64_t m = __ballot(ok);
            const uint32_t a0 = a - lane;   // multiple of 64
            // a word is written by the piece whose positions (b0, b0 + n) it covers
            if (lane == 0 && a0 + 31 > b0 && a0 < b0 + n) bm[safe_word(a0, b0)] = (uint32_t)m;
            if (lane == 32 && a0 + 63 > b0 && a0 + 32 < b0 + n) bm[safe_word(a0 + 32, b0)] = (uint32_t)(m >> 32);
        }
        // the piece's bitmap words are complete once every participating workgroup has counted
        __syncthreads();
        if (tid == 0) {
            __threadfence();
            s_last = atomicAdd(&gdone[g], 1u) == min(nb, gridDim.x) - 1u;
            __threadfence();
        }
        __syncthreads();
        if (s_last) giant_cut(v, ws, L, g);
    }
}

// giant_join: the last workgroup of k_bpe_giant, piece by piece.  A scan of the chunks' token counts
// gives each chunk's place in the piece's output (cdest, in the chunk-length array, no longer
// needed); the piece's token count is recorded, and the output gather copies each chunk from scratch.
__device__ void giant_join(uint8_t *ws, const Layout &L)
{
    constexpr uint32_t NT = 1024, NW = NT / 64;
    __shared__ uint32_t swsum[NW];
    __shared__ uint32_t s_acc;
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *list = (const uint32_t *)(ws + L.bin_giant);
    const uint32_t *ccount = (const uint32_t *)(ws + L.ccount);
    uint32_t *cdest = (uint32_t *)(ws + L.clen);
    const uint32_t *gc0 = (const uint32_t *)(ws + L.gc0), *gnc = (const uint32_t *)(ws + L.gnc);
    const uint32_t count = ctrl->bin_count[2];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    for (uint32_t g = 0; g < count; ++g) {
        const uint32_t p = list[g], c0 = gc0[g], nc = gnc[g];
        if (tid == 0) s_acc = 0;
        __syncthreads();
        for (uint32_t i0 = 0; i0 < nc; i0 += NT) {
            const uint32_t i = i0 + tid;
            const uint32_t x = i < nc ? ccount[c0 + i] : 0u;
            uint32_t inc = x;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t y = __shfl_up(inc, d, 64);
                if (lane >= (uint32_t)d) inc += y;
            }
            if (lane == 63) swsum[wid] = inc;
            __syncthreads();
            uint32_t before = s_acc, tot = 0;
            for (uint32_t w = 0; w < NW; ++w) {
                if (w < wid) before += swsum[w];
                tot += swsum[w];
            }
            if (i < nc) cdest[c0 + i] = before + inc - x;
            __syncthreads();
            if (tid == 0) s_acc += tot;
            __syncthreads();
        }
        if (tid == 0) put_piece(ws, L, p, ((const uint32_t *)(ws + L.pstart))[p], s_acc, 0u, true);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------
// giant pieces: one workgroup each; the sequence lives in device memory (double-buffered) and each
// round streams it through LDS in coalesced tiles, carrying the chain state and the output offset
// from tile to tile.  The next round's minimum rank is gathered while writing and re-probing.

constexpr int GE = 8;                       // elements per thread per tile
constexpr int GTILE = GIANT_THREADS * GE;   // 8192

__global__ __launch_bounds__(GIANT_THREADS) void k_bpe_giant(DevVocab v, const uint8_t *__restrict__ bytes,
                                                             uint8_t *ws, Layout L)
{
    constexpr int NT = GIANT_THREADS;
    __shared__ uint32_t sid[GTILE];
    __shared__ uint32_t srk[GTILE + 1];
    __shared__ uint8_t ssel[GTILE + 1];
    __shared__ uint32_t red[NT / 64 + 1];
    __shared__ int32_t redi[NT / 64 + 1];
    __shared__ int32_t s_last_cs;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *pval = (uint32_t *)(ws + L.pval);
    if (ctrl->bin_count[2] == 0) return;   // no giant pieces: no chunks to encode or join
    const uint32_t count = ctrl->n_chunks;
    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *clen = (const uint32_t *)(ws + L.clen);
    uint32_t *ccount = (uint32_t *)(ws + L.ccount);
    const uint32_t tid = threadIdx.x;
    const uint32_t i0 = tid * GE;

    for (uint32_t q = blockIdx.x; q < count; q += gridDim.x) {
        const uint32_t b0 = cstart[q];
        uint32_t n = clen[q];
        if (n <= (uint32_t)BLOCK_MAX) continue;   // unused slot, or a chunk for the workgroup kernel
        uint32_t *idA = (uint32_t *)(ws + L.scratch) + b0, *idB = (uint32_t *)(ws + L.g_ids) + b0;
        uint32_t *rkA = (uint32_t *)(ws + L.g_rank_a) + b0, *rkB = (uint32_t *)(ws + L.g_rank_b) + b0;
        for (uint32_t k = tid; k < n; k += NT) idA[k] = bytes[b0 + k];
        uint32_t lmin = NO_RANK;
        for (uint32_t k = tid; k < n; k += NT) {
            uint32_t r = k + 1 < n ? rkx_rank(__ldg(v.r2 + ((uint32_t)bytes[b0 + k] << 8 | bytes[b0 + k + 1]))) : NO_RANK;
            rkA[k] = r;
            lmin = min(lmin, r);
        }
        uint32_t rmin = block_min<NT>(lmin, red);   // (contains a barrier: idA/rkA are visible)
        while (rmin < v.n_merges) {
            uint32_t out = 0;                  // uniform: output elements written so far
            bool c_hit = false, c_sel = false; // previous tile's last element
            int32_t c_cs = -1;                 // chain start of that element (when it is a hit)
            uint32_t nmin = NO_RANK;
            for (uint32_t t0 = 0; t0 < n; t0 += GTILE) {
                const uint32_t cnt_t = min((uint32_t)GTILE, n - t0);
                for (uint32_t i = tid; i < cnt_t; i += NT) { sid[i] = idA[t0 + i]; srk[i] = rkA[t0 + i]; }
                if (tid == 0) srk[cnt_t] = t0 + cnt_t < n ? rkA[t0 + cnt_t] : NO_RANK;
                __syncthreads();
                // selection: leftmost non-overlapping occurrences of the minimum-rank pair
                uint32_t hitm = 0;
#pragma unroll
                for (int e = 0; e < GE; ++e)
                    if (i0 + e < cnt_t && srk[i0 + e] == rmin) hitm |= 1u << e;
                const bool prev_hit = i0 == 0 ? c_hit : (i0 <= cnt_t && srk[i0 - 1] == rmin);
                int32_t last_start = -1;
#pragma unroll
                for (int e = 0; e < GE; ++e) {
                    bool h = (hitm >> e) & 1u, hp = e ? ((hitm >> (e - 1)) & 1u) : prev_hit;
                    if (h && !hp) last_start = (int32_t)(t0 + i0 + e);
                }
                int32_t cs = max(block_excl_max<NT>(last_start, redi), c_hit ? c_cs : -1);
                uint32_t selm = 0;
#pragma unroll
                for (int e = 0; e < GE; ++e) {
                    bool h = (hitm >> e) & 1u, hp = e ? ((hitm >> (e - 1)) & 1u) : prev_hit;
                    if (h && !hp) cs = (int32_t)(t0 + i0 + e);
                    if (h && (((int32_t)(t0 + i0 + e) - cs) & 1) == 0) selm |= 1u << e;
                }
#pragma unroll
                for (int e = 0; e < GE; ++e)
                    if (i0 + e < cnt_t) ssel[i0 + e] = (selm >> e) & 1u;
                if (i0 < cnt_t && i0 + GE >= cnt_t) {
                    // the thread holding the tile's last element: chain state for the next tile, and
                    // whether the next tile's first element is selected
                    const uint32_t last = cnt_t - 1 - i0;
                    const bool lh = (hitm >> last) & 1u;
                    s_last_cs = lh ? cs : -1;
                    bool nh = srk[cnt_t] == rmin;
                    int32_t ncs = lh ? cs : (int32_t)(t0 + cnt_t);
                    ssel[cnt_t] = nh && (((int32_t)(t0 + cnt_t) - ncs) & 1) == 0;
                }
                __syncthreads();
                uint32_t keepm = 0, cnt = 0;
#pragma unroll
                for (int e = 0; e < GE; ++e) {
                    const uint32_t i = i0 + e;
                    const bool dropped = i == 0 ? c_sel : (i < cnt_t + 1 && ssel[i - 1]);
                    if (i < cnt_t && !dropped) { keepm |= 1u << e; ++cnt; }
                }
                uint32_t tot;
                const uint32_t off = block_excl_sum<NT>(cnt, red, &tot);
                uint32_t o = out + off;
#pragma unroll
                for (int e = 0; e < GE; ++e) {
                    if (!((keepm >> e) & 1u)) continue;
                    const uint32_t i = i0 + e;
                    const bool sl = (selm >> e) & 1u;
                    const uint32_t r = (sl || ssel[i + 1]) ? PENDING : srk[i];
                    idB[o] = sl ? 256u + rmin : sid[i];
                    rkB[o] = r;
                    if (r != PENDING) nmin = min(nmin, r);
                    ++o;
                }
                c_hit = srk[cnt_t - 1] == rmin;
                c_sel = ssel[cnt_t - 1];
                c_cs = s_last_cs;
                out += tot;
                __syncthreads();
            }
            // re-probe the pairs next to a merge (their right neighbours are written now)
            for (uint32_t j = tid; j < out; j += NT) {
                if (rkB[j] != PENDING) continue;
                const uint32_t r = j + 1 < out ? pair_rank(v, idB[j], idB[j + 1]) : NO_RANK;
                rkB[j] = r;
                nmin = min(nmin, r);
            }
            rmin = block_min<NT>(nmin, red);
            uint32_t *t = idA; idA = idB; idB = t;
            t = rkA; rkA = rkB; rkB = t;
            n = out;
        }
        uint32_t *dst = (uint32_t *)(ws + L.scratch) + b0;
        if (idA != dst)
            for (uint32_t k = tid; k < n; k += NT) dst[k] = idA[k];
        if (tid == 0) ccount[q] = n;
        __syncthreads();
    }
    if (last_workgroup(&ctrl->done_giant)) giant_join(ws, L);
}

// ---------------------------------------------------------------------------------------------

hipError_t launch_route(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev)
{
    if (b.n == 0) return hipGetLastError();
    const uint64_t g = (b.n + 4095) / 4096;   // about 4 KiB of input (1-2K pieces) per workgroup, at most 1024
    LaunchScope k(nullptr, 0, s);   // (not part of the encode chain)
    if (v.flags & VF_IGNORE_MERGES)
        hipLaunchKernelGGL(k_route<true>, dim3(g > 1024 ? 1024u : (uint32_t)g), dim3(RT_THREADS), 0, s, v, b.bytes, b.ws, b.L);
    else
        hipLaunchKernelGGL(k_route<false>, dim3(g > 1024 ? 1024u : (uint32_t)g), dim3(RT_THREADS), 0, s, v, b.bytes, b.ws, b.L);
    return hipGetLastError();
}

hipError_t launch_giant_prep(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev)
{
    const Layout &L = b.L;
    if (b.n == 0) return hipGetLastError();
    // giant pieces: safe-seam bitmap, then chunks (listed with the other BPE items by length)
    // (nothing to launch when no piece can be longer than BLOCK_MAX bytes: the layout holds at most
    // that many)
    LaunchScope k(ev, TK_GIANT_SEAMS, s);
    const uint32_t gs = (uint32_t)((b.n + 1023) / 1024);
    if (L.cap_n > (uint64_t)BLOCK_MAX)
        hipLaunchKernelGGL(k_giant_prep, dim3(gs < 256 ? gs : 256), dim3(1024), 0, s, v, b.bytes, b.ws, L);
    return hipGetLastError();
}

hipError_t launch_bpe(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev)
{
    const Layout &L = b.L;
    if (b.n == 0) return hipGetLastError();
    {
        // lists of <= 8, 9..12, 13..16, 17..32, 33..64 and 65..128 bytes: at most n / 2 (plus chunks),
        // n / 9, n / 13, n / 17, n / 33, n / 65 items; 256 lane items, 4 and 4 pieces per workgroup
        auto cap = [](uint64_t x, uint32_t c) { return x > c ? c : (uint32_t)x; };
        const uint32_t g8 = cap((b.n / 2 + L.cap_chunks) / 256 + 1, 2048), g12 = cap(b.n / 9 / 256 + 1, 2048);
        const uint32_t g16 = cap(b.n / 13 / 256 + 1, 2048), g32 = cap(b.n / 17 / 128 + 1, 2048);
        const uint32_t g64 = cap(b.n / 33 / 4 + 1, 256), g128 = cap(b.n / 65 / 4 + 1, 256);
        // and the lists of 129..1024 bytes (a wavefront per piece) and 1025..4096 bytes (a workgroup per
        // piece) in the same launch
        const uint32_t gw = cap(((uint64_t)L.cap_wave + L.cap_chunks + 3) / 4, 256);
        const uint32_t gb = cap((uint64_t)L.cap_block + L.cap_chunks, 256);
        LaunchScope k(ev, TK_BPE, s);
        hipLaunchKernelGGL(k_bpe_small, dim3(gb + gw + g8 + g12 + g16 + g32 + g64 + g128), dim3(256), 0, s, v, b.bytes,
                           b.ws, L, gb, gw, g8, g12, g16, g32, g64, g128);
    }
    const uint32_t gg = L.cap_giant < 64 ? L.cap_giant : 64;
    {
        LaunchScope k(ev, TK_BPE_GIANT, s);
        if (L.cap_n > (uint64_t)BLOCK_MAX)   // (no giant piece, no chunk, nothing to join)
            hipLaunchKernelGGL(k_bpe_giant, dim3(gg), dim3(GIANT_THREADS), 0, s, v, b.bytes, b.ws, L);
    }
    return hipGetLastError();
}

}  // namespace tt
