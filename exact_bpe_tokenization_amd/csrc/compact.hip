// compact.hip -- output compaction: per-piece ID runs -> one contiguous ID array per batch.
//
// TokTier (arXiv 2607.29678), GPU full-tokenization paragraph: the complete path ends with output
// compaction, and piece counts and output length stay in device memory (no host round trip between
// kernels).  k_emit does it in one pass per tile of 4096 pieces: coalesced loads of the per-piece
// token counts and starts, a workgroup scan plus a decoupled look-back for the tile's first token
// offset, the gather of each piece's IDs into out_ids (consecutive pieces write consecutive IDs),
// and the token offsets of the documents whose first piece lies in the tile.  Pieces longer than a
// lane's limit (a few, with many IDs each) are copied by k_gather_long, one workgroup per piece.
#include "internal.h"

namespace tt {

__global__ __launch_bounds__(SCAN_THREADS) void k_emit(uint8_t *ws, Layout L, const uint64_t *__restrict__ offsets,
                                                      uint32_t n_docs, uint64_t n, uint32_t *__restrict__ out_ids,
                                                      uint64_t *__restrict__ out_offsets)
{
    constexpr int NW = SCAN_THREADS / 64;
    __shared__ uint32_t soff[SCAN_TILE + 1];     // token counts, then token offsets
    __shared__ uint32_t sps[SCAN_TILE + 1];      // piece starts of the tile and the next one
    __shared__ uint32_t swsum[NW];
    __shared__ uint32_t s_tile, s_base, s_prev, s_dA, s_dB;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *ntok = (const uint32_t *)(ws + L.ntok);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *scratch = (const uint32_t *)(ws + L.scratch);
    uint32_t *tokoff = (uint32_t *)(ws + L.tokoff);
    uint64_t *flags = (uint64_t *)(ws + L.sflag);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    if (tid == 0) s_tile = atomicAdd(&ctrl->tile_ctr_scan, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t np = ctrl->n_pieces;
    const uint64_t first64 = (uint64_t)tile * SCAN_TILE;
    if (first64 > np) return;                          // nothing at or below P in this tile
    const uint32_t first = (uint32_t)first64;
    const uint32_t cnt_t = min((uint32_t)SCAN_TILE, np - first);
    const bool last = first + cnt_t == np;
    for (uint32_t i = tid; i < cnt_t; i += SCAN_THREADS) {
        soff[i] = ntok[first + i];
        sps[i] = pstart[first + i];
    }
    if (tid == 0) {
        sps[cnt_t] = np ? pstart[first + cnt_t] : (uint32_t)n;   // pstart[np] == n
        s_prev = first ? pstart[first - 1] : 0u;
    }
    __syncthreads();
    const uint32_t i0 = tid * SCAN_PER_THREAD;
    uint32_t x[SCAN_PER_THREAD], sum = 0;
#pragma unroll
    for (int k = 0; k < SCAN_PER_THREAD; ++k) {
        x[k] = i0 + k < cnt_t ? soff[i0 + k] : 0u;
        sum += x[k];
    }
    uint32_t inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(inc, d, 64);
        if (lane >= (uint32_t)d) inc += y;
    }
    if (lane == 63) swsum[wid] = inc;
    __syncthreads();
    uint32_t before = inc - sum, total = 0;
    for (uint32_t w = 0; w < (uint32_t)NW; ++w) {
        if (w < wid) before += swsum[w];
        total += swsum[w];
    }
    if (wid == 0) {
        if (lane == 0 && tile > 0) st_flag(flags + tile, (1ull << 62) | total);
        const uint64_t basev = tile == 0 ? 0 : lookback_sum(flags, tile);
        if (lane == 0) {
            st_flag(flags + tile, (2ull << 62) | (basev + total));
            s_base = (uint32_t)basev;
            if (last) ctrl->n_tokens = (uint32_t)(basev + total);
        }
    }
    __syncthreads();
    const uint32_t base = s_base, tile_end = base + total;
    uint32_t run = base + before;
#pragma unroll
    for (int k = 0; k < SCAN_PER_THREAD; ++k) {
        if (i0 + k < cnt_t) soff[i0 + k] = run;
        run += x[k];
    }
    if (tid == 0) soff[cnt_t] = tile_end;
    __syncthreads();
    // gather: piece i of the tile owns IDs [soff[i], soff[i+1]) at scratch[its start byte ...]
    for (uint32_t i = tid; i < cnt_t; i += SCAN_THREADS) {
        const uint32_t o = soff[i], c = soff[i + 1] - o, b0 = sps[i];
        if (sps[i + 1] - b0 > (uint32_t)LANE_MAX) {
            tokoff[first + i] = o;                      // binned piece: k_gather_long copies it
            continue;
        }
        const uint32_t *src = scratch + b0;
        for (uint32_t j = 0; j < c; ++j) out_ids[o + j] = src[j];
    }
    // documents whose first piece is in this tile: offsets in (start of the piece before the
    // tile, start of the tile's last piece]; the last tile also takes everything after it
    if (wid == 0) {
        const uint32_t dA = first ? wave_upper_bound(offsets, n_docs + 1, (uint64_t)s_prev) : 0u;
        const uint32_t dB = last ? n_docs + 1 : wave_upper_bound(offsets, n_docs + 1, (uint64_t)sps[cnt_t - 1]);
        if (lane == 0) { s_dA = dA; s_dB = dB; }
    }
    __syncthreads();
    for (uint32_t d = s_dA + tid; d < s_dB; d += SCAN_THREADS) {
        const uint64_t off = offsets[d];
        uint32_t a = 0, b = cnt_t;
        while (a < b) {
            uint32_t m = (a + b) >> 1;
            if ((uint64_t)sps[m] < off) a = m + 1; else b = m;
        }
        out_offsets[d] = soff[a];
    }
}

// one workgroup per binned (longer than a lane's limit) piece
__global__ __launch_bounds__(256) void k_gather_long(uint8_t *ws, Layout L, uint32_t *__restrict__ out_ids)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *ntok = (const uint32_t *)(ws + L.ntok);
    const uint32_t *tokoff = (const uint32_t *)(ws + L.tokoff);
    const uint32_t *scratch = (const uint32_t *)(ws + L.scratch);
    const uint32_t c0 = ctrl->bin_count[0], c1 = ctrl->bin_count[1], c2 = ctrl->bin_count[2];
    const uint32_t *l0 = (const uint32_t *)(ws + L.bin_wave), *l1 = (const uint32_t *)(ws + L.bin_block),
                   *l2 = (const uint32_t *)(ws + L.bin_giant);
    for (uint32_t q = blockIdx.x; q < c0 + c1 + c2; q += gridDim.x) {
        const uint32_t p = q < c0 ? l0[q] : (q < c0 + c1 ? l1[q - c0] : l2[q - c0 - c1]);
        const uint32_t *src = scratch + pstart[p];
        uint32_t *dst = out_ids + tokoff[p];
        const uint32_t c = ntok[p];
        for (uint32_t j = threadIdx.x; j < c; j += blockDim.x) dst[j] = src[j];
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

hipError_t launch_compact(const Batch &b, uint32_t *out_ids, uint64_t *out_offsets, hipStream_t s,
                          const Events *ev)
{
    const Layout &L = b.L;
    {
        LaunchScope k(ev, 8, s);
        hipLaunchKernelGGL(k_emit, dim3(L.n_scan_tiles), dim3(SCAN_THREADS), 0, s, b.ws, L, b.offsets, b.n_docs,
                           b.n, out_ids, out_offsets);
    }
    if (b.n) {
        LaunchScope k(ev, 9, s);
        uint32_t gl = L.cap_wave < 2048 ? L.cap_wave : 2048;
        hipLaunchKernelGGL(k_gather_long, dim3(gl), dim3(256), 0, s, b.ws, L, out_ids);
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
