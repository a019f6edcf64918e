// added.hip -- added (special) tokens: a leftmost-longest literal pass in front of the pre-tokenizer.
//
// TokTier (arXiv 2607.29678), implementation paragraph on added and special tokens: they are literal
// strings that the model reserves as single IDs, taken out of the text by a leftmost-longest pass
// before the tokenizer family handles the remaining segments.  Within a document, scanning left to
// right, the longest literal that starts at the scan position and ends inside the document is taken
// and the scan resumes after it; the text between literals is tokenized as a document of its own.
//
//   k_lit_find<false>  per 4 KiB tile: count the candidate positions (where some literal starts and
//                      ends inside the document); also checks the document offsets
//   k_lit_scan         tile counts -> tile bases (one workgroup)
//   k_lit_find<true>   the candidates again, written in text order: (position, longest literal)
//   k_lit_resolve      the leftmost-longest choice among the candidates (one workgroup): a candidate
//                      that no earlier candidate overlaps is taken; a run of overlapping candidates
//                      (a cluster) is walked in order by the thread of its first one
//   k_lit_compact      the taken literals in order, with their documents
//   -- the host reads the number of literals --
//   k_lit_docs         document offsets of the text cut at the literals: each literal becomes a
//                      document of its own between two text documents
//   -- the pipeline encodes the cut documents --
//   k_lit_counts       token count of each literal document and their prefix sums
//   k_lit_scatter      final IDs (a literal document's tokens become the literal's one ID), spans and
//                      document offsets
#include "internal.h"

namespace tt {

namespace {

constexpr int LIT_THREADS = 256;
constexpr int LIT_PER_THREAD = LIT_TILE / LIT_THREADS;   // 16 positions per thread
constexpr int ONE_BLOCK = 1024;

// first index i in [0, n) with a[i] > x (n if none); lane-serial
template <typename T>
__device__ __forceinline__ uint32_t upper_idx(const T *a, uint32_t n, T x)
{
    uint32_t lo = 0, hi = n;
    while (lo < hi) {
        const uint32_t m = (lo + hi) >> 1;
        if (a[m] > x) hi = m; else lo = m + 1;
    }
    return lo;
}

// number of taken literals starting before byte x (the literal list is sorted by position)
__device__ __forceinline__ uint32_t lits_before(const uint4 *lits, uint32_t k, uint64_t x)
{
    uint32_t lo = 0, hi = k;
    while (lo < hi) {
        const uint32_t m = (lo + hi) >> 1;
        if ((uint64_t)lits[m].x < x) lo = m + 1; else hi = m;
    }
    return lo;
}

// end of the document holding byte p (the first document offset above p; n past the last)
__device__ __forceinline__ uint64_t doc_end(const uint64_t *offsets, uint32_t n_docs, uint64_t n, uint64_t p)
{
    const uint32_t i = upper_idx(offsets, n_docs + 1, p);
    return i <= n_docs ? min(offsets[i], n) : n;
}

// longest literal starting at byte p and ending inside p's document, NO_LIT if none
__device__ uint32_t literal_at(const DevAdded &a, const uint8_t *__restrict__ bytes, uint64_t n,
                               const uint64_t *offsets, uint32_t n_docs, uint64_t p)
{
    const uint32_t b0 = bytes[p];
    if (p + 1 < n && a.lmax >= 2) {
        const uint32_t x = b0 | ((uint32_t)bytes[p + 1] << 8);
        if ((a.pmap[x >> 5] >> (x & 31u)) & 1u) {
            const uint64_t de = doc_end(offsets, n_docs, n, p);
            for (uint32_t i = a.pre[x], e = a.pre[x + 1]; i < e; ++i) {   // longest first
                const uint32_t k = a.list[i];
                const uint32_t o = a.off[k], len = a.off[k + 1] - o;
                if (p + len > de) continue;
                bool eq = true;
                for (uint32_t j = 2; j < len && eq; ++j) eq = bytes[p + j] == a.bytes[o + j];
                if (eq) return k;
            }
        }
    }
    return a.one[b0];   // a one-byte literal always fits: byte p is inside its document
}

// exclusive prefix sum over a workgroup of NT threads (NT / 64 wavefronts); *total gets the sum
template <int NT>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t x, uint32_t *total)
{
    __shared__ uint32_t wsum[NT / 64];
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_sum(x);
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t s = wsum[w];
        before += (uint32_t)w < wid ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + inc - x;
}

// exclusive prefix maximum over a workgroup of NT threads (0 before the first); *total gets the max
template <int NT>
__device__ __forceinline__ uint64_t block_excl_max(uint64_t x, uint64_t *total)
{
    __shared__ uint64_t sv[NT];
    __shared__ uint64_t wmax[NT / 64];
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    sv[threadIdx.x] = x;
    __syncthreads();
    // inclusive maximum inside the wavefront (Hillis-Steele in LDS; 64-bit values)
    uint64_t m = x;
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint64_t o = lane >= d ? sv[threadIdx.x - d] : 0ull;
        __syncthreads();
        m = max(m, o);
        sv[threadIdx.x] = m;
        __syncthreads();
    }
    if (lane == 63) wmax[wid] = m;
    __syncthreads();
    uint64_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint64_t s = wmax[w];
        if ((uint32_t)w < wid) before = max(before, s);
        tot = max(tot, s);
    }
    const uint64_t excl_in_wave = lane ? sv[threadIdx.x - 1] : 0ull;
    __syncthreads();
    *total = tot;
    return max(before, excl_in_wave);
}

template <bool WRITE>
__global__ __launch_bounds__(LIT_THREADS) void k_lit_find(DevAdded a, const uint8_t *__restrict__ bytes,
                                                          const uint64_t *__restrict__ offsets, uint32_t n_docs,
                                                          uint64_t n, uint8_t *ws, AddLayout A)
{
    uint32_t *tcount = (uint32_t *)(ws + A.tcount);
    const uint32_t tile = blockIdx.x, tid = threadIdx.x;
    bool bad = false;
    if (!WRITE) {   // document offsets: from 0 to n, non-decreasing (a bad tile sets bit 31 of its count)
        bad = tile == 0 && tid == 0 && (offsets[0] != 0 || offsets[n_docs] != n);
        for (uint64_t d = (uint64_t)tile * LIT_THREADS + tid; d < n_docs; d += (uint64_t)gridDim.x * LIT_THREADS)
            bad |= offsets[d] > offsets[d + 1];
    }
    const uint64_t p0 = (uint64_t)tile * LIT_TILE + (uint64_t)tid * LIT_PER_THREAD;
    uint32_t kk[LIT_PER_THREAD];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < LIT_PER_THREAD; ++j) {
        const uint64_t p = p0 + j;
        kk[j] = p < n ? literal_at(a, bytes, n, offsets, n_docs, p) : NO_LIT;
        c += kk[j] != NO_LIT;
    }
    uint32_t total;
    const uint32_t before = block_excl_sum<LIT_THREADS>(c, &total);
    if (!WRITE) {
        const bool any_bad = __syncthreads_or(bad);
        if (tid == 0) tcount[tile] = total | (any_bad ? LIT_TAKEN : 0u);
        return;
    }
    if (!total) return;
    uint2 *cand = (uint2 *)(ws + A.cand) + ((const uint32_t *)(ws + A.tbase))[tile] + before;
#pragma unroll
    for (int j = 0; j < LIT_PER_THREAD; ++j)
        if (kk[j] != NO_LIT) *cand++ = make_uint2((uint32_t)(p0 + j), kk[j]);
}

__global__ __launch_bounds__(ONE_BLOCK) void k_lit_scan(uint8_t *ws, AddLayout A)
{
    const uint32_t *tcount = (const uint32_t *)(ws + A.tcount);
    uint32_t *tbase = (uint32_t *)(ws + A.tbase);
    uint32_t carry = 0;
    bool bad = false;
    for (uint32_t t0 = 0; t0 < A.n_ltiles; t0 += ONE_BLOCK) {
        const uint32_t t = t0 + threadIdx.x;
        const uint32_t f = t < A.n_ltiles ? tcount[t] : 0u;
        bad |= (f & LIT_TAKEN) != 0;
        uint32_t total;
        const uint32_t ex = block_excl_sum<ONE_BLOCK>(f & ~LIT_TAKEN, &total);
        if (t < A.n_ltiles) tbase[t] = carry + ex;
        carry += total;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {   // (this kernel writes the literal pass's control words first)
        LitCtrl *lc = (LitCtrl *)(ws + A.lctrl);
        lc->status = bad ? ST_BAD_OFFSETS : 0u;
        lc->n_cand = carry;
        lc->n_lit = 0;
    }
}

__global__ __launch_bounds__(ONE_BLOCK) void k_lit_resolve(DevAdded a, uint8_t *ws, AddLayout A)
{
    const uint32_t C = ((const LitCtrl *)(ws + A.lctrl))->n_cand;
    uint2 *cand = (uint2 *)(ws + A.cand);
    uint64_t carry = 0;   // the largest end of the candidates before the chunk
    for (uint32_t c0 = 0; c0 < C; c0 += ONE_BLOCK) {
        const uint32_t j = c0 + threadIdx.x;
        const bool have = j < C;
        const uint2 cj = have ? cand[j] : make_uint2(0u, 0u);
        const uint32_t k = cj.y & ~LIT_TAKEN;
        const uint64_t e = have ? (uint64_t)cj.x + (a.off[k + 1] - a.off[k]) : 0ull;
        uint64_t cmax;
        const uint64_t before = max(carry, block_excl_max<ONE_BLOCK>(e, &cmax));
        if (have && (uint64_t)cj.x >= before) {
            // no earlier candidate reaches this one: it is taken, and so is every later candidate of
            // its cluster that starts at or after the end of the last one taken
            uint64_t resume = e, reach = e;
            cand[j].y = k | LIT_TAKEN;
            for (uint32_t i = j + 1; i < C; ++i) {
                const uint2 ci = cand[i];
                if ((uint64_t)ci.x >= reach) break;   // the next cluster
                const uint32_t ki = ci.y & ~LIT_TAKEN;
                const uint64_t ei = (uint64_t)ci.x + (a.off[ki + 1] - a.off[ki]);
                if ((uint64_t)ci.x >= resume) {
                    cand[i].y = ki | LIT_TAKEN;
                    resume = ei;
                }
                reach = max(reach, ei);
            }
        }
        carry = max(carry, cmax);
        __syncthreads();
    }
}

__global__ __launch_bounds__(ONE_BLOCK) void k_lit_compact(DevAdded a, const uint64_t *__restrict__ offsets,
                                                           uint32_t n_docs, uint8_t *ws, AddLayout A)
{
    LitCtrl *lc = (LitCtrl *)(ws + A.lctrl);
    const uint32_t C = lc->n_cand;
    const uint2 *cand = (const uint2 *)(ws + A.cand);
    uint4 *lits = (uint4 *)(ws + A.lits);
    uint32_t carry = 0;
    for (uint32_t c0 = 0; c0 < C; c0 += ONE_BLOCK) {
        const uint32_t j = c0 + threadIdx.x;
        const uint2 cj = j < C ? cand[j] : make_uint2(0u, 0u);
        const bool taken = j < C && (cj.y & LIT_TAKEN);
        uint32_t total;
        const uint32_t ex = block_excl_sum<ONE_BLOCK>(taken ? 1u : 0u, &total);
        if (taken) {
            const uint32_t k = cj.y & ~LIT_TAKEN;
            // the document holding the literal: the last offset at or below its start
            const uint32_t u = upper_idx(offsets, n_docs + 1, (uint64_t)cj.x);
            const uint32_t d = u ? min(u - 1, n_docs - 1) : 0u;
            lits[carry + ex] = make_uint4(cj.x, k, d, a.off[k + 1] - a.off[k]);
        }
        carry += total;
    }
    if (threadIdx.x == 0) lc->n_lit = carry;
}

// offsets of the cut documents: document d of the batch starts the cut document d + 2 L(d), L(d) the
// number of literals before it; literal i (in document d_i) is the cut document d_i + 2 i + 1 and the
// text after it starts the one at d_i + 2 i + 2
__global__ __launch_bounds__(256) void k_lit_docs(const uint64_t *__restrict__ offsets, uint32_t n_docs,
                                                  uint8_t *ws, AddLayout A, uint32_t n_lit)
{
    const uint4 *lits = (const uint4 *)(ws + A.lits);
    uint64_t *offs2 = (uint64_t *)(ws + A.offs2);
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t <= n_docs) {
        const uint32_t l = lits_before(lits, n_lit, offsets[t]);
        offs2[t + 2ull * l] = offsets[t];
    }
    if (t < n_lit) {
        const uint4 li = lits[t];
        offs2[li.z + 2ull * t + 1] = li.x;
        offs2[li.z + 2ull * t + 2] = (uint64_t)li.x + li.w;
    }
}

// token range of each literal document in the intermediate output, and the prefix sums of (count - 1)
// (the tokens that the literals' single IDs replace); the final token count goes to the control block
__global__ __launch_bounds__(ONE_BLOCK) void k_lit_counts(uint8_t *ws, Layout L, AddLayout A, uint32_t n_lit,
                                                          uint32_t n_docs2)
{
    const uint4 *lits = (const uint4 *)(ws + A.lits);
    const uint64_t *oo2 = (const uint64_t *)(ws + A.oo2);
    uint32_t *lstart = (uint32_t *)(ws + A.lstart), *lcnt = (uint32_t *)(ws + A.lcnt);
    uint32_t *lpref = (uint32_t *)(ws + A.lpref);
    uint32_t carry = 0;
    for (uint32_t i0 = 0; i0 < n_lit; i0 += ONE_BLOCK) {
        const uint32_t i = i0 + threadIdx.x;
        uint32_t c = 0;
        if (i < n_lit) {
            const uint64_t di = lits[i].z + 2ull * i + 1;
            const uint32_t s = (uint32_t)oo2[di];
            c = (uint32_t)oo2[di + 1] - s;
            lstart[i] = s;
            lcnt[i] = c;
        }
        uint32_t total;
        const uint32_t ex = block_excl_sum<ONE_BLOCK>(i < n_lit ? c - 1u : 0u, &total);
        if (i < n_lit) lpref[i] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) {
        lpref[n_lit] = carry;
        ((Ctrl *)(ws + L.ctrl))->n_tokens = (uint32_t)oo2[n_docs2] - carry;
    }
}

__global__ __launch_bounds__(256) void k_lit_scatter(DevAdded a, const uint64_t *__restrict__ offsets,
                                                     uint32_t n_docs, uint8_t *ws, AddLayout A, uint32_t n_lit,
                                                     uint32_t n_docs2, uint64_t n_threads,
                                                     uint32_t *__restrict__ out_ids,
                                                     uint64_t *__restrict__ out_offsets,
                                                     uint32_t *__restrict__ out_spans)
{
    const uint4 *lits = (const uint4 *)(ws + A.lits);
    const uint64_t *oo2 = (const uint64_t *)(ws + A.oo2);
    const uint32_t *lstart = (const uint32_t *)(ws + A.lstart), *lcnt = (const uint32_t *)(ws + A.lcnt);
    const uint32_t *lpref = (const uint32_t *)(ws + A.lpref);
    const uint32_t *ids2 = (const uint32_t *)(ws + A.ids2), *spans2 = (const uint32_t *)(ws + A.spans2);
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_threads) return;
    const uint64_t t2 = oo2[n_docs2];
    if (t < t2) {
        const uint32_t tt = (uint32_t)t;
        const uint32_t l = upper_idx(lstart, n_lit, tt);   // literal documents starting at or before t
        if (l && tt < lstart[l - 1] + lcnt[l - 1]) {        // inside literal l - 1's document
            if (tt == lstart[l - 1]) {
                const uint4 li = lits[l - 1];
                const uint32_t o = tt - lpref[l - 1];
                out_ids[o] = a.id[li.y];
                if (out_spans) out_spans[o] = li.x;
            }
        } else {
            const uint32_t o = tt - lpref[l];
            out_ids[o] = ids2[tt];
            if (out_spans) out_spans[o] = spans2[tt];
        }
    }
    if (t <= n_docs) {
        const uint32_t l = lits_before(lits, n_lit, offsets[t]);
        out_offsets[t] = oo2[t + 2ull * l] - lpref[l];
    }
}

}  // namespace

hipError_t launch_literals(const DevAdded &a, const Batch &b, const AddLayout &A, hipStream_t s)
{
    const uint32_t g = A.n_ltiles ? A.n_ltiles : 1u;
    hipLaunchKernelGGL(k_lit_find<false>, dim3(g), dim3(LIT_THREADS), 0, s, a, b.bytes, b.offsets, b.n_docs, b.n,
                       b.ws, A);
    hipLaunchKernelGGL(k_lit_scan, dim3(1), dim3(ONE_BLOCK), 0, s, b.ws, A);
    hipLaunchKernelGGL(k_lit_find<true>, dim3(g), dim3(LIT_THREADS), 0, s, a, b.bytes, b.offsets, b.n_docs, b.n,
                       b.ws, A);
    hipLaunchKernelGGL(k_lit_resolve, dim3(1), dim3(ONE_BLOCK), 0, s, a, b.ws, A);
    hipLaunchKernelGGL(k_lit_compact, dim3(1), dim3(ONE_BLOCK), 0, s, a, b.offsets, b.n_docs, b.ws, A);
    return hipGetLastError();
}

hipError_t launch_literal_docs(const Batch &b, const AddLayout &A, uint32_t n_lit, hipStream_t s)
{
    const uint64_t nt = (uint64_t)b.n_docs + 1 > n_lit ? (uint64_t)b.n_docs + 1 : (uint64_t)n_lit;
    hipLaunchKernelGGL(k_lit_docs, dim3((uint32_t)((nt + 255) / 256)), dim3(256), 0, s, b.offsets, b.n_docs, b.ws,
                       A, n_lit);
    return hipGetLastError();
}

hipError_t launch_literal_merge(const DevAdded &a, const Batch &b, const AddLayout &A, uint32_t n_lit,
                                uint32_t *out_ids, uint64_t *out_offsets, uint32_t *out_spans, hipStream_t s)
{
    const uint32_t n_docs2 = b.n_docs + 2 * n_lit;
    hipLaunchKernelGGL(k_lit_counts, dim3(1), dim3(ONE_BLOCK), 0, s, b.ws, b.L, A, n_lit, n_docs2);
    const uint64_t nt = b.n > (uint64_t)b.n_docs ? b.n : (uint64_t)b.n_docs + 1;
    hipLaunchKernelGGL(k_lit_scatter, dim3((uint32_t)((nt + 255) / 256)), dim3(256), 0, s, a, b.offsets, b.n_docs,
                       b.ws, A, n_lit, n_docs2, nt, out_ids, out_offsets, out_spans);
    return hipGetLastError();
}

}  // namespace tt
