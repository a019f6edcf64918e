// compact.hip -- output compaction: per-piece ID runs -> one contiguous ID array per batch.
//
// TokTier (arXiv 2607.29678), GPU full-tokenization paragraph: the complete path ends with output
// compaction, and piece counts and output length stay in device memory (no host round trip between
// kernels).  k_emit does it in one pass per tile of 4096 pieces: coalesced loads of the per-piece
// result words, a workgroup scan, the tile's first token offset from the per-tile excess
// counters the BPE kernels maintain (no look-back between tiles, no tile tickets), the gather of each
// piece's IDs into out_ids (consecutive pieces write consecutive IDs), and the token offsets of the
// documents whose first piece lies in the tile.  Pieces longer than a
// lane's limit (a few, with many IDs each) are copied by k_gather_long, one workgroup per piece.
#include "internal.h"

namespace tt {

// SPANS: also write each token's source byte offset (a separate instantiation, so that the plain form
// keeps its few registers)
template <bool SPANS>
__global__ __launch_bounds__(SCAN_THREADS) void k_emit(uint8_t *ws, Layout L, const uint64_t *__restrict__ offsets,
                                                      uint32_t n_docs, uint64_t n, uint32_t *__restrict__ out_ids,
                                                      uint64_t *__restrict__ out_offsets,
                                                      uint32_t *__restrict__ out_spans,
                                                      const uint32_t *__restrict__ tok_len)
{
    constexpr int NW = SCAN_THREADS / 64;
    constexpr int IT = SCAN_TILE / SCAN_THREADS;   // iterations of 64 pieces per wavefront
    __shared__ uint32_t soff[SCAN_TILE + 1];       // token offset of each piece of the tile
    __shared__ uint32_t swsum[NW], sxs[NW];
    __shared__ uint32_t s_dA, s_dB;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *__restrict__ pval = (const uint32_t *)(ws + L.pval);
    const uint32_t *__restrict__ pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *__restrict__ scratch = (const uint32_t *)(ws + L.scratch);
    const uint32_t *__restrict__ tilex = (const uint32_t *)(ws + L.tilex);
    uint32_t *__restrict__ tokoff = (uint32_t *)(ws + L.tokoff);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    const uint32_t tile = blockIdx.x;
    const uint32_t np = ctrl->n_pieces;
    const uint64_t first64 = (uint64_t)tile * SCAN_TILE;
    if (first64 > np) return;                          // nothing at or below P in this tile
    const uint32_t first = (uint32_t)first64;
    const uint32_t end = min(first + (uint32_t)SCAN_TILE, np);
    const bool last = end == np;

    // wavefront wid owns pieces [wb, wb + 64 * IT) of the tile, 64 consecutive pieces per iteration
    // (lane-consecutive: coalesced loads and stores).  Only the result words stay in registers; the
    // token offsets go through LDS (few registers, so every tile of a large batch is resident at once).
    const uint32_t wb = first + wid * (64u * IT);
    uint32_t pv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const uint32_t i = wb + it * 64u + lane;
        pv[it] = i < end ? pval[i] : 0u;
    }
    // tokens before this tile: one per piece plus the excess counted by the BPE kernels (16-byte reads)
    uint32_t xs = 0;
    {
        const uint32_t nq = tile / 4u;
        const uint4 *tx4 = (const uint4 *)tilex;
        for (uint32_t t = tid; t < nq; t += SCAN_THREADS) {
            const uint4 x = tx4[t];
            xs += x.x + x.y + x.z + x.w;
        }
        if (tid < tile - 4u * nq) xs += tilex[4u * nq + tid];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) xs += __shfl_xor(xs, d, 64);
    uint32_t run = 0;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const uint32_t i = wb + it * 64u + lane;
        const uint32_t c = i >= end ? 0u : (pv[it] & PV_MULTI) ? (pv[it] & PV_COUNT) : 1u;
        const uint32_t inc = wave_incl_sum(c);
        soff[wid * (64u * IT) + it * 64u + lane] = run + inc - c;   // offset inside the wavefront's run
        run += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    }
    if (lane == 0) { swsum[wid] = run; sxs[wid] = xs; }
    __syncthreads();
    uint32_t before = 0, total = 0, tbase = first;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < (int)wid) before += swsum[w];
        total += swsum[w];
        tbase += sxs[w];
    }
    if (last && tid == 0) ctrl->n_tokens = tbase + total;
    const uint32_t obase = tbase + before;

    // IDs: a single-token piece's ID is its result word (coalesced); a short multi-token piece's IDs
    // are at scratch[its start byte ...]; a long piece gets its output offset for k_gather_long.
    // All start loads are issued first; the first IDs in two halves (fewer registers); the further
    // IDs of a piece four independent loads at a time.  With spans, every piece's start is loaded (it
    // is its first token's span) and each further token's span adds the length of the token before.
    uint32_t st[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const uint32_t i = wb + it * 64u + lane;
        const bool multi = i < end && (pv[it] & (PV_MULTI | PV_LONG)) == PV_MULTI;
        st[it] = multi || (SPANS && i < end) ? pstart[i] : 0u;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        constexpr int HI = IT / 2;
        uint32_t f0[HI];
#pragma unroll
        for (int u = 0; u < HI; ++u) {
            const int it = h * HI + u;
            const uint32_t i = wb + it * 64u + lane;
            const bool multi = i < end && (pv[it] & (PV_MULTI | PV_LONG)) == PV_MULTI;
            f0[u] = multi ? scratch[st[it]] : pv[it];
        }
#pragma unroll
        for (int u = 0; u < HI; ++u) {
            const int it = h * HI + u;
            const uint32_t i = wb + it * 64u + lane;
            if (i >= end) continue;
            const uint32_t li = wid * (64u * IT) + it * 64u + lane;
            const uint32_t o = obase + soff[li], v = pv[it];
            soff[li] = o;
            if ((v & (PV_MULTI | PV_LONG)) == (PV_MULTI | PV_LONG)) {
                tokoff[i] = o;
                continue;
            }
            out_ids[o] = f0[u];
            if (SPANS) out_spans[o] = st[it];
            const uint32_t c = (v & PV_MULTI) ? (v & PV_COUNT) : 1u;
            uint32_t sp = st[it], prev = f0[u];   // span and ID of the token before token j
            for (uint32_t j = 1; j < c; j += 4) {
                uint32_t x[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) x[t] = j + t < c ? scratch[st[it] + j + t] : 0u;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (j + t < c) out_ids[o + j + t] = x[t];
                if (SPANS) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if (j + t >= c) break;
                        sp += tok_len[prev];
                        out_spans[o + j + t] = sp;
                        prev = x[t];
                    }
                }
            }
        }
    }
    if (tid == 0) soff[end - first] = tbase + total;

    // documents whose first piece is in this tile: offsets in (start of the piece before the
    // tile, start of the tile's last piece]; the last tile also takes everything after it
    if (wid == 0) {
        const uint32_t dA = first ? wave_upper_bound(offsets, n_docs + 1, (uint64_t)pstart[first - 1]) : 0u;
        const uint32_t dB = last ? n_docs + 1 : wave_upper_bound(offsets, n_docs + 1, (uint64_t)pstart[end - 1]);
        if (lane == 0) { s_dA = dA; s_dB = dB; }
    }
    __syncthreads();
    for (uint32_t d = s_dA + wid; d < s_dB; d += NW) {
        // the first piece of the tile starting at or after the document's offset
        const uint32_t a = wave_lower_bound(pstart + first, end - first, (uint32_t)offsets[d]);
        if (lane == 0) out_offsets[d] = soff[a];
    }
}

// IDs of the pieces longer than 128 bytes: one workgroup per piece of the wave and block bins, and
// one per chunk of a giant piece (a chunk's IDs go to its place in the piece's output).  With spans,
// a workgroup scan of the token lengths gives each token's span from the piece's or chunk's start.
__global__ __launch_bounds__(256) void k_gather_long(uint8_t *ws, Layout L, uint32_t *__restrict__ out_ids,
                                                     uint32_t *__restrict__ out_spans,
                                                     const uint32_t *__restrict__ tok_len)
{
    __shared__ uint32_t swsum[4];
    __shared__ uint32_t s_carry;
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *pval = (const uint32_t *)(ws + L.pval);
    const uint32_t *tokoff = (const uint32_t *)(ws + L.tokoff);
    const uint32_t *scratch = (const uint32_t *)(ws + L.scratch);
    const uint32_t *cstart = (const uint32_t *)(ws + L.cstart), *cdest = (const uint32_t *)(ws + L.clen);
    const uint32_t *ccount = (const uint32_t *)(ws + L.ccount), *cpiece = (const uint32_t *)(ws + L.cpiece);
    const uint32_t c0 = ctrl->bin_count[0], c1 = ctrl->bin_count[1], nch = ctrl->n_chunks;
    const uint32_t *l0 = (const uint32_t *)(ws + L.bin_wave), *l1 = (const uint32_t *)(ws + L.bin_block);
    for (uint32_t q = blockIdx.x; q < c0 + c1 + nch; q += gridDim.x) {
        const uint32_t *src;
        uint32_t *dst;
        uint32_t c;
        if (q < c0 + c1) {
            const uint32_t p = q < c0 ? l0[q] : l1[q - c0];
            src = scratch + pstart[p];
            dst = out_ids + tokoff[p];
            c = pval[p] & PV_COUNT;
        } else {
            const uint32_t k = q - c0 - c1, p = cpiece[k];
            if (p == NO_PIECE) continue;   // reserved chunk slot not used
            src = scratch + cstart[k];
            dst = out_ids + tokoff[p] + cdest[k];
            c = ccount[k];
        }
        if (!out_spans) {
            for (uint32_t j = threadIdx.x; j < c; j += blockDim.x) dst[j] = src[j];
            continue;
        }
        uint32_t *sdst = out_spans + (dst - out_ids);
        const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
        if (threadIdx.x == 0) s_carry = q < c0 + c1 ? pstart[q < c0 ? l0[q] : l1[q - c0]] : cstart[q - c0 - c1];
        __syncthreads();
        for (uint32_t j0 = 0; j0 < c; j0 += blockDim.x) {
            const uint32_t j = j0 + threadIdx.x;
            const uint32_t id = j < c ? src[j] : 0u;
            const uint32_t len = j < c ? tok_len[id] : 0u;
            const uint32_t inc = wave_incl_sum(len);
            if (lane == 63) swsum[wid] = inc;
            __syncthreads();
            uint32_t before = s_carry, tot = 0;
            for (uint32_t w = 0; w < 4; ++w) {
                if (w < wid) before += swsum[w];
                tot += swsum[w];
            }
            if (j < c) {
                dst[j] = id;
                sdst[j] = before + inc - len;
            }
            __syncthreads();
            if (threadIdx.x == 0) s_carry += tot;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void k_export_starts(uint8_t *ws, Layout L, uint64_t n, uint32_t *out)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t np = ctrl->n_pieces;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i <= np; i += gridDim.x * blockDim.x)
        out[i] = i == np ? (uint32_t)n : pstart[i];
}

hipError_t launch_compact(const DevVocab &v, const Batch &b, uint32_t *out_ids, uint64_t *out_offsets,
                          uint32_t *out_spans, hipStream_t s, const Events *ev)
{
    const Layout &L = b.L;
    {
        LaunchScope k(nullptr, 0, s);
        if (out_spans)
            hipLaunchKernelGGL(k_emit<true>, dim3(L.n_scan_tiles), dim3(SCAN_THREADS), 0, s, b.ws, L, b.offsets,
                               b.n_docs, b.n, out_ids, out_offsets, out_spans, v.tok_len);
        else
            hipLaunchKernelGGL(k_emit<false>, dim3(L.n_scan_tiles), dim3(SCAN_THREADS), 0, s, b.ws, L, b.offsets,
                               b.n_docs, b.n, out_ids, out_offsets, out_spans, v.tok_len);
    }
    if (b.n) {
        LaunchScope k(nullptr, 0, s);
        uint32_t gl = L.cap_wave + L.cap_chunks < 1024 ? L.cap_wave + L.cap_chunks : 1024;
        hipLaunchKernelGGL(k_gather_long, dim3(gl), dim3(256), 0, s, b.ws, L, out_ids, out_spans, v.tok_len);
    }
    return hipGetLastError();
}

hipError_t launch_export_starts(const Batch &b, uint32_t *out_starts, hipStream_t s)
{
    uint32_t g = (uint32_t)((b.n + 1 + 255) / 256);
    hipLaunchKernelGGL(k_export_starts, dim3(g > 4096 ? 4096 : g), dim3(256), 0, s, b.ws, b.L, b.n, out_starts);
    return hipGetLastError();
}

}  // namespace tt
