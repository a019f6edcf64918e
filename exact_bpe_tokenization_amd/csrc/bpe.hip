// bpe.hip -- stage 2: segmented byte-level BPE of every piece on gfx950.
//
// TokTier (arXiv 2607.29678), GPU BPE paragraph and Figure 6 (lower part): pieces are encoded
// independently; work is dispatched by piece length to the smallest execution unit that holds the
// piece's state; merge ranks live in device hash tables.  Two facts license the parallel schedule:
// a round's minimum rank names one pair, and merging all leftmost non-overlapping occurrences of
// that pair equals iterated single merges (for rank-consistent merge lists, which the loader
// enforces); only pairs next to a completed merge need a new lookup.
//
//   k_bpe_lane   one lane per piece of <= 16 bytes; sequence and ranks in registers; the textbook
//                loop (leftmost lowest rank, merge, re-probe the two neighbours)
//   k_bpe_block  one wavefront (pieces of 17..1024 bytes) or one 256-lane workgroup (up to 4096
//                bytes) per piece; sequence in LDS; rounds: block-min of ranks, selection of the
//                leftmost non-overlapping occurrences, prefix-sum compaction, neighbour re-probes
//   k_bpe_giant  one 1024-lane workgroup per piece longer than that; the same rounds over device
//                memory (double-buffered)
// Every kernel writes the piece's IDs at scratch[piece start byte ...] (a piece never has more IDs
// than bytes) and its ID count to ntok[piece].
#include "internal.h"

namespace tt {

constexpr uint32_t PENDING = 0xFFFFFFFEu;

// ---------------------------------------------------------------------------------------------
// lane per piece

__global__ __launch_bounds__(256) void k_bpe_lane(DevVocab v, const uint8_t *__restrict__ bytes,
                                                  uint8_t *ws, Layout L)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *ntok = (uint32_t *)(ws + L.ntok);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    const uint32_t np = ctrl->n_pieces;
    for (uint32_t p = blockIdx.x * blockDim.x + threadIdx.x; p < np; p += gridDim.x * blockDim.x) {
        const uint32_t b0 = pstart[p];
        const uint32_t len = pstart[p + 1] - b0;
        if (len > LANE_MAX) continue;
        uint32_t id[LANE_MAX], rk[LANE_MAX];
#pragma unroll
        for (int k = 0; k < LANE_MAX; ++k) id[k] = (uint32_t)k < len ? (uint32_t)bytes[b0 + k] : 0u;
#pragma unroll
        for (int k = 0; k < LANE_MAX; ++k)
            rk[k] = (uint32_t)(k + 1) < len ? __ldg(v.r2 + ((id[k] << 8) | id[(k + 1) % LANE_MAX])) : NO_RANK;
        uint32_t n = len;
        for (;;) {
            uint32_t best = NO_RANK, pos = 0;
#pragma unroll
            for (int k = 0; k < LANE_MAX - 1; ++k)
                if (rk[k] < best) { best = rk[k]; pos = k; }
            if (best == NO_RANK) break;
            const uint32_t nid = 256u + best;
            // id[pos] <- nid, drop id[pos+1], shift the tail left
#pragma unroll
            for (int j = 0; j < LANE_MAX; ++j) {
                uint32_t nx_id = j + 1 < LANE_MAX ? id[(j + 1) % LANE_MAX] : 0u;
                uint32_t nx_rk = j + 1 < LANE_MAX ? rk[(j + 1) % LANE_MAX] : NO_RANK;
                id[j] = (uint32_t)j < pos ? id[j] : ((uint32_t)j == pos ? nid : nx_id);
                rk[j] = (uint32_t)j < pos ? rk[j] : nx_rk;
            }
            --n;
            uint32_t left = 0, right = 0;
#pragma unroll
            for (int j = 0; j < LANE_MAX; ++j) {
                if ((uint32_t)j + 1 == pos) left = id[j];
                if ((uint32_t)j == pos + 1) right = id[j];
            }
            const uint32_t rl = pos > 0 ? pair_rank(v, left, nid) : NO_RANK;
            const uint32_t rr = pos + 1 < n ? pair_rank(v, nid, right) : NO_RANK;
#pragma unroll
            for (int j = 0; j < LANE_MAX; ++j) {
                if ((uint32_t)j + 1 == pos) rk[j] = rl;
                if ((uint32_t)j == pos) rk[j] = rr;
            }
        }
#pragma unroll
        for (int k = 0; k < LANE_MAX; ++k)
            if ((uint32_t)k < n) scratch[b0 + k] = id[k];
        ntok[p] = n;
    }
}

// ---------------------------------------------------------------------------------------------
// workgroup primitives (NT threads, NT a multiple of 64)

template <int NT>
__device__ __forceinline__ uint32_t block_min(uint32_t x, uint32_t *red)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = min(x, (uint32_t)__shfl_xor(x, d, 64));
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

template <int NT, int MAXN>
__global__ __launch_bounds__(NT) void k_bpe_block(DevVocab v, const uint8_t *__restrict__ bytes, uint8_t *ws,
                                                  Layout L, int bin)
{
    constexpr int E = MAXN / NT;
    static_assert(E <= 32, "selection masks are 32-bit");
    __shared__ uint32_t sid[MAXN];
    __shared__ uint32_t srk[MAXN];
    __shared__ uint8_t ssel[MAXN + 1];
    __shared__ uint32_t red[NT / 64 + 1];
    __shared__ int32_t redi[NT / 64 + 1];

    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *ntok = (uint32_t *)(ws + L.ntok);
    uint32_t *scratch = (uint32_t *)(ws + L.scratch);
    const uint32_t *list = (const uint32_t *)(ws + (bin == 0 ? L.bin_wave : L.bin_block));
    const uint32_t count = ctrl->bin_count[bin];
    const uint32_t tid = threadIdx.x;
    const uint32_t k0 = tid * E;

    for (uint32_t q = blockIdx.x; q < count; q += gridDim.x) {
        const uint32_t p = list[q];
        const uint32_t b0 = pstart[p];
        uint32_t n = pstart[p + 1] - b0;
        for (uint32_t k = tid; k < n; k += NT) sid[k] = bytes[b0 + k];
        __syncthreads();
        for (uint32_t k = tid; k < n; k += NT)
            srk[k] = k + 1 < n ? __ldg(v.r2 + ((sid[k] << 8) | sid[k + 1])) : NO_RANK;
        __syncthreads();
        for (;;) {
            uint32_t lmin = NO_RANK;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (k0 + e < n) lmin = min(lmin, srk[k0 + e]);
            const uint32_t rmin = block_min<NT>(lmin, red);
            if (rmin >= v.n_merges) break;   // NO_RANK: nothing left to merge
            const bool selfpair = v.merges[2 * rmin] == v.merges[2 * rmin + 1];
            uint32_t hitm = 0;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (k0 + e < n && srk[k0 + e] == rmin) hitm |= 1u << e;
            uint32_t selm = hitm;
            if (selfpair) {
                // overlapping occurrences (x, x)(x, x): inside each chain of consecutive hits keep
                // the ones at an even distance from the chain's start
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
            __syncthreads();
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
            __syncthreads();
            uint32_t o = off;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((keepm >> e) & 1u) { sid[o] = nid[e]; srk[o] = nrk[e]; ++o; }
            __syncthreads();
            for (uint32_t j = off; j < off + cnt; ++j)
                if (srk[j] == PENDING) srk[j] = j + 1 < nnew ? pair_rank(v, sid[j], sid[j + 1]) : NO_RANK;
            __syncthreads();
            n = nnew;
        }
        for (uint32_t k = tid; k < n; k += NT) scratch[b0 + k] = sid[k];
        if (tid == 0) ntok[p] = n;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------
// giant pieces: one workgroup each, sequence double-buffered in device memory

__global__ __launch_bounds__(GIANT_THREADS) void k_bpe_giant(DevVocab v, const uint8_t *__restrict__ bytes,
                                                             uint8_t *ws, Layout L)
{
    constexpr int NT = GIANT_THREADS;
    __shared__ uint32_t red[NT / 64 + 1];
    __shared__ int32_t redi[NT / 64 + 1];
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    uint32_t *ntok = (uint32_t *)(ws + L.ntok);
    const uint32_t *list = (const uint32_t *)(ws + L.bin_giant);
    const uint32_t count = ctrl->bin_count[2];
    const uint32_t tid = threadIdx.x;

    for (uint32_t q = blockIdx.x; q < count; q += gridDim.x) {
        const uint32_t p = list[q];
        const uint32_t b0 = pstart[p];
        uint32_t n = pstart[p + 1] - b0;
        uint32_t *idA = (uint32_t *)(ws + L.scratch) + b0, *idB = (uint32_t *)(ws + L.g_ids) + b0;
        uint32_t *rkA = (uint32_t *)(ws + L.g_rank_a) + b0, *rkB = (uint32_t *)(ws + L.g_rank_b) + b0;
        for (uint32_t k = tid; k < n; k += NT) idA[k] = bytes[b0 + k];
        __syncthreads();
        for (uint32_t k = tid; k < n; k += NT)
            rkA[k] = k + 1 < n ? __ldg(v.r2 + ((idA[k] << 8) | idA[k + 1])) : NO_RANK;
        __syncthreads();
        for (;;) {
            const uint32_t E = (n + NT - 1) / NT;
            const uint32_t k0 = min(n, tid * E), k1 = min(n, k0 + E);
            uint32_t lmin = NO_RANK;
            for (uint32_t k = k0; k < k1; ++k) lmin = min(lmin, rkA[k]);
            const uint32_t rmin = block_min<NT>(lmin, red);
            if (rmin >= v.n_merges) break;   // NO_RANK: nothing left to merge
            const bool selfpair = v.merges[2 * rmin] == v.merges[2 * rmin + 1];
            auto hit = [&](uint32_t k) -> bool { return k < n && rkA[k] == rmin; };
            // chain starts (only matter for self pairs)
            int32_t last_start = -1;
            if (selfpair)
                for (uint32_t k = k0; k < k1; ++k)
                    if (hit(k) && !(k >= 1 && hit(k - 1))) last_start = (int32_t)k;
            const int32_t carry = selfpair ? block_excl_max<NT>(last_start, redi) : -1;
            // selection of element k given the current chain start
            int32_t cs = carry;
            auto sel_at = [&](uint32_t k, int32_t &c) -> bool {
                bool h = hit(k);
                if (!selfpair) return h;
                if (h && !(k >= 1 && hit(k - 1))) c = (int32_t)k;
                return h && (((int32_t)k - c) & 1) == 0;
            };
            // was the element before my range selected?
            bool prev_sel = false;
            if (k0 >= 1 && k0 < k1) {
                int32_t c2 = carry;   // chain start covering k0 - 1 (valid when it is a hit)
                prev_sel = hit(k0 - 1) && (!selfpair || (((int32_t)(k0 - 1) - c2) & 1) == 0);
            }
            uint32_t cnt = 0;
            {
                bool ps = prev_sel;
                int32_t c = cs;
                for (uint32_t k = k0; k < k1; ++k) {
                    bool s = sel_at(k, c);
                    if (!ps) ++cnt;
                    ps = s;
                }
            }
            uint32_t nnew;
            const uint32_t off = block_excl_sum<NT>(cnt, red, &nnew);
            {
                bool ps = prev_sel;
                int32_t c = cs;
                uint32_t o = off;
                bool s = k0 < k1 ? sel_at(k0, c) : false;
                for (uint32_t k = k0; k < k1; ++k) {
                    int32_t cn = c;
                    bool sn = (k + 1 < n) ? sel_at(k + 1, cn) : false;
                    if (!ps) {
                        idB[o] = s ? 256u + rmin : idA[k];
                        rkB[o] = (s || sn) ? PENDING : rkA[k];
                        ++o;
                    }
                    ps = s;
                    s = sn;
                    c = cn;
                }
            }
            __syncthreads();
            for (uint32_t j = off; j < off + cnt; ++j)
                if (rkB[j] == PENDING) rkB[j] = j + 1 < nnew ? pair_rank(v, idB[j], idB[j + 1]) : NO_RANK;
            __syncthreads();
            uint32_t *t = idA; idA = idB; idB = t;
            t = rkA; rkA = rkB; rkB = t;
            n = nnew;
        }
        uint32_t *dst = (uint32_t *)(ws + L.scratch) + b0;
        if (idA != dst)
            for (uint32_t k = tid; k < n; k += NT) dst[k] = idA[k];
        if (tid == 0) ntok[p] = n;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------

hipError_t launch_bpe(const DevVocab &v, const Batch &b, hipStream_t s)
{
    const Layout &L = b.L;
    if (b.n == 0) return hipGetLastError();
    uint32_t g = (uint32_t)((b.n + 255) / 256);
    hipLaunchKernelGGL(k_bpe_lane, dim3(g > 4096 ? 4096 : g), dim3(256), 0, s, v, b.bytes, b.ws, L);
    uint32_t gw = L.cap_wave < 4096 ? L.cap_wave : 4096;
    hipLaunchKernelGGL((k_bpe_block<64, WAVE_MAX>), dim3(gw), dim3(64), 0, s, v, b.bytes, b.ws, L, 0);
    uint32_t gb = L.cap_block < 1024 ? L.cap_block : 1024;
    hipLaunchKernelGGL((k_bpe_block<BLOCK_THREADS, BLOCK_MAX>), dim3(gb), dim3(BLOCK_THREADS), 0, s, v, b.bytes,
                       b.ws, L, 1);
    uint32_t gg = L.cap_giant < 256 ? L.cap_giant : 256;
    hipLaunchKernelGGL(k_bpe_giant, dim3(gg), dim3(GIANT_THREADS), 0, s, v, b.bytes, b.ws, L);
    return hipGetLastError();
}

}  // namespace tt
