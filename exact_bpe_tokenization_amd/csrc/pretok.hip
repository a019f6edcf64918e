// pretok.hip -- stage 1: regex-exact run decomposition of the pre-tokenizer on gfx950.
//
// TokTier (arXiv 2607.29678), GPU pre-tokenization paragraph and Figure 6: every character is
// classified (letter / number / whitespace / other), maximal same-class runs are formed, and
// whether a character starts a piece depends only on its offset in the run, a few characters of
// look-back and per-run aggregates -- so classification is parallel and run summaries come from
// prefix scans.  Here the per-character rule is a 15-state automaton (the state says what the
// running leftmost-first match expects next).  Each character's transition function is a 16-byte
// map (one byte per state), maps compose associatively with byte permutes, so the state before
// every character comes from a parallel scan of maps: within a thread, across the workgroup, and
// across tiles through a decoupled look-back.  The two facts that need the future -- "no CR/LF
// later in this whitespace run" (where `\s*[\r\n]+` stops) and "only uppercase letters left in this
// letter run" (where the o200k case rule backtracks) -- are carried right to left; each tile's
// carry comes from a summary of the tiles after it.
//
// Kernels:  k_summary  per tile: the leftmost character that decides each backward flag (an
//                      early-exit scan of the tile's first bytes), and the automaton state its last
//                      60 bytes fix for the next tile (a second wavefront); also clears the control
//                      block, the look-back flags and the tile counters
//           k_pieces   per 8 KiB tile: UTF-8 decode + validation, categories, backward flags,
//                      automaton scan, piece starts (one read of the input; per tile a count, its
//                      first start and 2 bytes per piece written at the tile's own place)
//           k_compact  (piece-start export only; the encode chain's tile encoder does the same) the
//                      starts at their global places, long pieces listed by length
#include "internal.h"

#define TT_UCAT_QUAL static __device__ const
#include "unicode_table.inc"

namespace tt {

// ---------------------------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ uint32_t utf8_len(uint32_t b)
{
    if (b < 0x80u) return 1;
    if (b >= 0xC2u && b <= 0xDFu) return 2;
    if (b >= 0xE0u && b <= 0xEFu) return 3;
    if (b >= 0xF0u && b <= 0xF4u) return 4;
    return 0;   // continuation byte or never-valid lead
}

__device__ __forceinline__ uint32_t ucat(uint32_t cp)
{
    if (cp < 0x80u) {
        // ASCII without a table load: letters, digits, the six whitespace characters, the rest
        const uint32_t lc = cp | 32u;
        if (lc >= 'a' && lc <= 'z') return cp >= 'a' ? CAT_LL : CAT_LU;
        if (cp >= '0' && cp <= '9') return CAT_N;
        if (cp == ' ' || (cp >= 9u && cp <= 13u)) return CAT_W;
        return (cp >= 0x21u && cp <= 0x7Eu) ? (uint32_t)(CAT_O | CC_PS) : (uint32_t)CAT_O;   // punctuation, symbols
    }
    return tt_ucat_stage2[((uint32_t)tt_ucat_stage1[cp >> 8] << 8) | (cp & 255u)];
}

// backward map of one character for a boolean carried right-to-left:
// 0 = pass the value of the next character through, 2 = constant false, 3 = constant true
enum : uint32_t { BK_KEEP = 0, BK_F = 2, BK_T = 3 };

// NA  = "no CR/LF from here to the end of this whitespace run"   (true outside whitespace)
// AU  = "only uppercase letters from here to the end of this letter run" (true outside letters)
__device__ __forceinline__ void backward_maps(uint32_t code, bool eof_next, uint32_t &na, uint32_t &au)
{
    const uint32_t cat = code & 7u;
    na = cat != CAT_W ? BK_T : ((code & CC_CRLF) ? BK_F : (eof_next ? BK_T : BK_KEEP));
    const bool lower = cat == CAT_LL || cat == CAT_LO || cat == CAT_M;
    au = cat == CAT_LU ? (eof_next ? BK_T : BK_KEEP) : (lower ? BK_F : BK_T);
}

// 16-byte transition maps: byte s (s < 15) is the image of state s in bits 0-3 (bit 4 is the
// piece-start flag, ignored when composing); byte 15 is never selected.  Composition is a byte
// gather done with v_perm: two 8-byte halves selected by the low 3 bits, then one of the two by bit 3.
struct M16 {
    uint32_t w[4];
};

__device__ __forceinline__ M16 m16_identity() { return M16{{0x03020100u, 0x07060504u, 0x0B0A0908u, 0x0F0E0D0Cu}}; }

__device__ __forceinline__ uint32_t gather16(const M16 &b, uint32_t sel)
{
    const uint32_t s7 = sel & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(b.w[1], b.w[0], s7);
    const uint32_t hi = __builtin_amdgcn_perm(b.w[3], b.w[2], s7);
    return __builtin_amdgcn_perm(hi, lo, ((sel >> 1) & 0x04040404u) | 0x03020100u);
}

// apply a first, then b
__device__ __forceinline__ M16 compose16(const M16 &a, const M16 &b)
{
    return M16{{gather16(b, a.w[0]), gather16(b, a.w[1]), gather16(b, a.w[2]), gather16(b, a.w[3])}};
}

__device__ __forceinline__ uint32_t byte16(const M16 &m, uint32_t s)
{
    const uint32_t q = s >> 2;
    const uint32_t w = q == 0 ? m.w[0] : (q == 1 ? m.w[1] : (q == 2 ? m.w[2] : m.w[3]));
    return (w >> (8u * (s & 3u))) & 255u;
}

__device__ __forceinline__ M16 shfl_up16(const M16 &m, int d)
{
    return M16{{(uint32_t)__shfl_up(m.w[0], d, 64), (uint32_t)__shfl_up(m.w[1], d, 64),
                (uint32_t)__shfl_up(m.w[2], d, 64), (uint32_t)__shfl_up(m.w[3], d, 64)}};
}

__device__ __forceinline__ M16 shfl16(const M16 &m, int src)
{
    return M16{{(uint32_t)__shfl(m.w[0], src, 64), (uint32_t)__shfl(m.w[1], src, 64),
                (uint32_t)__shfl(m.w[2], src, 64), (uint32_t)__shfl(m.w[3], src, 64)}};
}

__device__ __forceinline__ M16 shfl_down16(const M16 &m, int d)
{
    return M16{{(uint32_t)__shfl_down(m.w[0], d, 64), (uint32_t)__shfl_down(m.w[1], d, 64),
                (uint32_t)__shfl_down(m.w[2], d, 64), (uint32_t)__shfl_down(m.w[3], d, 64)}};
}

__device__ __forceinline__ M16 m16_const(uint32_t st) { const uint32_t c = st * 0x01010101u; return M16{{c, c, c, c}}; }

// every state maps to the same state (only the state nibbles of bytes 0..14 count)
__device__ __forceinline__ bool is_const16(const M16 &m)
{
    const uint32_t c = (m.w[0] & 15u) * 0x01010101u;
    return (m.w[0] & 0x0F0F0F0Fu) == c && (m.w[1] & 0x0F0F0F0Fu) == c && (m.w[2] & 0x0F0F0F0Fu) == c &&
           (m.w[3] & 0x000F0F0Fu) == (c & 0x000F0F0Fu);
}

// Tile look-back flags of the automaton state: one map per tile, 4 words, each word carrying the
// flag kind in its top two bits (bytes 3, 7, 11 and 15 of a map use only bits 0-4): 1 = the tile's
// map, 2 = the constant map of the state after the tile, 0 = nothing published yet.  Words are
// stored and loaded one by one, each atomically; a reader accepts a flag only when its four words
// carry the same kind, so it never combines words of the two stores.
constexpr uint32_t FLAG_AGG = 1, FLAG_PREFIX = 2;

__device__ __forceinline__ void st_flag16(uint32_t *p, const M16 &m, uint32_t kind)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __hip_atomic_store(p + i, (m.w[i] & 0x3FFFFFFFu) | (kind << 30), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Automaton state entering `tile`.  Wave 0 reads the flags of 64 predecessors per step.  The walk
// ends at the nearest predecessor whose flag fixes the state: a prefix, or a map that sends every
// state to one state (an 8 KiB tile of text nearly always has one); only the predecessors up to it
// must have published, and their maps are composed (farthest first) with byte permutes.  The batch
// starts in S_ST.
__device__ uint32_t lookback_state(const uint32_t *flags, uint32_t tile)
{
    const uint32_t lane = threadIdx.x & 63u;
    M16 acc = m16_identity();
    int64_t top = (int64_t)tile - 1;
    for (;;) {
        const int64_t pos = top - (int64_t)lane;
        uint32_t f[4];
        if (pos >= 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f[i] = __hip_atomic_load(flags + 4 * pos + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = (uint32_t)S_ST * 0x01010101u | (FLAG_PREFIX << 30);
        }
        const uint32_t k0 = f[0] >> 30;
        const uint32_t kind = ((f[1] >> 30) == k0 && (f[2] >> 30) == k0 && (f[3] >> 30) == k0) ? k0 : 0u;
        M16 x = M16{{f[0] & 0x0F0F0F0Fu, f[1] & 0x0F0F0F0Fu, f[2] & 0x0F0F0F0Fu, f[3] & 0x0F0F0F0Fu}};
        const bool fixes = kind == FLAG_PREFIX || (kind == FLAG_AGG && is_const16(x));
        const uint64_t st = __ballot(fixes), nr = __ballot(kind == 0);
        const uint32_t kp = st ? (uint32_t)__ffsll((unsigned long long)st) - 1u : 64u;
        const uint64_t need = kp >= 63 ? ~0ull : ((2ull << kp) - 1);
        if (nr & need) { __builtin_amdgcn_s_sleep(1); continue; }
        if (kp == 0) return byte16(acc, byte16(shfl16(x, 0), 0) & 15u) & 15u;
        if (lane > kp) x = m16_identity();
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const M16 y = shfl_down16(x, d);
            if ((lane & (2u * d - 1u)) == 0) x = compose16(y, x);
        }
        acc = compose16(shfl16(x, 0), acc);
        if (kp < 64 || is_const16(acc)) return byte16(acc, 0) & 15u;
        top -= 64;
    }
}

// Per-byte code of position p (index j into the LDS byte window, `docbit` over the same window).
// Continuation bytes get CAT_CONT; `bad` is set when p breaks UTF-8 (only when check is true).
template <typename DocBit>
__device__ __forceinline__ uint32_t byte_code(const uint8_t *sraw, DocBit docbit, int j, uint64_t p, uint64_t n,
                                              int family, bool check, bool &bad)
{
    const uint32_t c = sraw[j];
    const bool isdoc = docbit(j);
    if ((c & 0xC0u) == 0x80u) {
        if (check) {
            // a continuation byte must be covered by a lead byte 1..3 bytes back in the same doc
            bool ok = false;
            if (!isdoc) {
                for (int back = 1; back <= 3; ++back) {
                    if ((int64_t)p - back < 0) break;
                    uint32_t lead = sraw[j - back];
                    if ((lead & 0xC0u) != 0x80u) { ok = utf8_len(lead) > (uint32_t)back; break; }
                }
            }
            bad |= !ok;
        }
        return CAT_CONT;
    }
    uint32_t len = utf8_len(c), cp = c;
    bool ok = len != 0 && p + len <= n;
    if (ok && len > 1) {
        cp = c & (0x7Fu >> len);
        for (uint32_t t = 1; t < len; ++t) {
            uint32_t cb = sraw[j + t];
            ok &= ((cb & 0xC0u) == 0x80u) && !docbit(j + (int)t);
            cp = (cp << 6) | (cb & 0x3Fu);
        }
        ok &= !(len == 3 && cp < 0x800u) && !(len == 4 && (cp < 0x10000u || cp > 0x10FFFFu)) &&
              !(cp >= 0xD800u && cp <= 0xDFFFu);
    }
    if (check) bad |= !ok;
    if (!ok) cp = 0xFFFDu;
    uint32_t code = ucat(cp) | (isdoc ? CC_DOC : 0u);
    if (c == '\r' || c == '\n') code |= CC_CRLF;
    if (c == ' ') code |= CC_SP;
    if (family == FAMILY_DEEPSEEK) {
        code |= ds_bits(cp, code);
    } else if (c == '\'') {
        // 's 't 're 've 'm 'll 'd (ASCII; case-insensitive except for the GPT-2 family)
        auto letter = [&](uint32_t t) -> uint32_t {
            if (p + t >= n || docbit(j + (int)t)) return 0;
            uint32_t x = sraw[j + t];
            if (family != 1 && x >= 'A' && x <= 'Z') x += 32;
            return x;
        };
        uint32_t x1 = letter(1), x2 = letter(2), lc = 0;
        if (x1 == 's' || x1 == 't' || x1 == 'm' || x1 == 'd') lc = 1;
        else if ((x1 == 'r' && x2 == 'e') || (x1 == 'v' && x2 == 'e') || (x1 == 'l' && x2 == 'l')) lc = 2;
        code |= lc << CC_CONTR_SHIFT;
    }
    return code;
}

// ---------------------------------------------------------------------------------------------
// k_summary: one workgroup of two wavefronts per tile (one workgroup when the batch is empty); the
// second computes the states the tile's last bytes fix (above) beside the first.  It also clears what
// the later kernels count on: the control block, the tile's look-back flags and the per-tile token
// counters.  The tile's summary of a backward flag is the map of its leftmost character whose map
// is not "pass through" (for NA: the first character that is not whitespace-other-than-CR/LF, or
// the last of its document; for AU: the first that is not an uppercase letter, or the last of its
// document).  Usually found in the first 256 bytes.

template <int T>
struct StepBytes {
    static constexpr int value = T;
};

// The state that enters the next tile when the tile's last WIN_BYTES bytes fix it: their automaton
// maps composed, one composition for each value of the backward flags that enters them from the
// right (NA, and AU under the case rules; the next tile knows which applies).  A composition that
// sends every state to one state gives that state whatever came before (the usual case: a few
// characters of text synchronize the automaton), and the next tile's pieces kernel takes it
// instead of waiting for this tile's look-back flag.  One lane per byte: lanes 0..59 the window,
// lanes 60..63 the four bytes after the tile (the next characters).  Result byte v (flag value v =
// NA | AU << 1): 0x10 | state when fixed, else 0.
constexpr int WIN_BYTES = 60;

__device__ __forceinline__ uint32_t wave_or(uint32_t x)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x |= (uint32_t)__shfl_xor((int)x, d, 64);
    return x;
}

// inclusive scan of 16-byte maps over the wavefront with DPP (lane i: lanes 0..i composed, lane 0's
// map first): row shifts inside each row of 16 lanes, then the row broadcasts of lanes 15 and 31
__device__ __forceinline__ M16 wave_scan16(M16 x)
{
    const uint32_t lane = threadIdx.x & 63u, r = lane & 15u, row = lane >> 4;
#define TT_DPPX(ctrl, rmask) M16{{(uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.w[0], ctrl, rmask, 0xF, false), \
                                  (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.w[1], ctrl, rmask, 0xF, false), \
                                  (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.w[2], ctrl, rmask, 0xF, false), \
                                  (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.w[3], ctrl, rmask, 0xF, false)}}
    { const M16 y = TT_DPPX(0x111, 0xF); if (r >= 1) x = compose16(y, x); }
    { const M16 y = TT_DPPX(0x112, 0xF); if (r >= 2) x = compose16(y, x); }
    { const M16 y = TT_DPPX(0x114, 0xF); if (r >= 4) x = compose16(y, x); }
    { const M16 y = TT_DPPX(0x118, 0xF); if (r >= 8) x = compose16(y, x); }
    { const M16 y = TT_DPPX(0x142, 0xA); if (row & 1u) x = compose16(y, x); }   // row_bcast:15
    { const M16 y = TT_DPPX(0x143, 0xC); if (row >= 2) x = compose16(y, x); }   // row_bcast:31
#undef TT_DPPX
    return x;
}

template <typename DocBit>
__device__ uint32_t window_states(const DevVocab &v, const uint8_t *swin, DocBit docbit, uint64_t wb, uint64_t n)
{
    const uint32_t lane = threadIdx.x & 63u;
    const bool DS = v.family == FAMILY_DEEPSEEK, CASE = v.family == FAMILY_O200K;
    const uint32_t NX = DS ? DS_NNEXT : NNEXT, AUM = DS ? 1u : 2u, NCTXV = DS ? DS_NCTX : NCTX;
    const int j = (int)lane + (64 - WIN_BYTES);   // this lane's byte in swin (position wb + j)
    const uint64_t p = wb + (uint64_t)j;
    bool ignore = false;
    const uint32_t code = p < n ? byte_code(swin, docbit, j, p, n, v.family, false, ignore) : (uint32_t)CC_EOF;
    // the next character: the first later byte that is not a continuation byte
    const bool cont = (code & 7u) == CAT_CONT && code != CC_EOF;
    const uint64_t starts = __ballot(!cont) & (lane < 63 ? ~0ull << (lane + 1) : 0ull);
    const uint32_t nc = (uint32_t)__shfl((int)code, starts ? __ffsll((unsigned long long)starts) - 1 : 63, 64);
    // backward flags: decided here (D) and their value (T), as the pieces kernel forms them
    const uint32_t cat = code & 7u;
    const bool win = lane < (uint32_t)WIN_BYTES, isch = cat != CAT_CONT;
    const bool ws_ = isch && cat == CAT_W, crlf = ws_ && (code & CC_CRLF);
    const bool en = (((nc >> 7) | (0x80u >> (nc & 7u))) & 1u) != 0;
    const bool tna = (isch && !ws_) || (ws_ && !crlf && en), dna = tna || crlf;
    const bool up = isch && cat == CAT_LU, low = isch && (cat == CAT_LL || cat == CAT_LO || cat == CAT_M);
    const bool tau = (isch && !(up || low)) || (up && en), dau = tau || low;
    // first decided position at or after each byte of the window (0: none, else 2 | value)
    uint32_t xn = win && dna ? 2u | (tna ? 1u : 0u) : 0u, xa = win && dau ? 2u | (tau ? 1u : 0u) : 0u;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t yn = __shfl_down(xn, d, 64), ya = __shfl_down(xa, d, 64);
        if (lane + d < 64) {
            if (xn == 0) xn = yn;
            if (xa == 0) xa = ya;
        }
    }
    const uint32_t xa_next = lane < 63 ? __shfl_down(xa, 1, 64) : 0u;   // AU of the next byte
    const uint32_t selfc = DS ? self_code_ds(code) : self_code(code, false);
    const uint32_t nextc = DS ? next_code_ds(nc) : ((nc & 7u) == CAT_CONT ? 5u : next_code(nc));
    const uint32_t base = win && isch ? (selfc * 2u + ((code & CC_DOC) ? 1u : 0u)) * NX * AUM + nextc * AUM : 0xFFFFu;
    // one composition per flag value (the maps of all values loaded together; past NCTXV: identity)
    const uint32_t nvar = CASE ? 4u : 2u;
    uint4 t[4];
#pragma unroll
    for (uint32_t var = 0; var < 4; ++var) {
        const uint32_t na = xn ? (xn & 1u) : (var & 1u), aun = xa_next ? (xa_next & 1u) : ((var >> 1) & 1u);
        const uint32_t ctx = min(base + ((na && ws_ && !crlf) ? 2u * NX * AUM : 0u) + (CASE ? aun : 0u), NCTXV);
        t[var] = (var < nvar && ctx < NCTXV) ? v.fmap16[ctx] : make_uint4(0x03020100u, 0x07060504u, 0x0B0A0908u, 0x0F0E0D0Cu);
    }
    uint32_t res = 0;
#pragma unroll
    for (uint32_t var = 0; var < 4; ++var) {
        if (var >= nvar) break;
        const M16 x = wave_scan16(M16{{t[var].x, t[var].y, t[var].z, t[var].w}});
        if (is_const16(x)) res |= (0x10u | (x.w[0] & 15u)) << (8u * var);
    }
    return (uint32_t)__builtin_amdgcn_readlane((int)res, 63);
}

__global__ __launch_bounds__(128) void k_summary(DevVocab v, const uint8_t *__restrict__ bytes,
                                                 const uint64_t *__restrict__ offsets, uint32_t n_docs,
                                                 uint64_t n, uint8_t *ws, Layout L)
{
    __shared__ uint8_t swin[72];
    bool bad_size = false;
    const uint32_t n_tiles = request_sizes(L, n, n_docs, &bad_size);
    const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
    if (wid == 0) {
        if (blockIdx.x == 0) ((uint32_t *)(ws + L.ctrl))[lane] = lane == 0 && bad_size ? (uint32_t)ST_BAD_OFFSETS : 0u;   // 64 words
        if (blockIdx.x < n_tiles && lane == 0) ((uint4 *)(ws + L.tflag_state))[blockIdx.x] = make_uint4(0u, 0u, 0u, 0u);
        for (uint32_t k = blockIdx.x * 64u + lane; k <= n_tiles / 64u; k += gridDim.x * 64u) {
            ((uint32_t *)(ws + L.tsb))[k] = 0;
            ((uint32_t *)(ws + L.gsum))[k] = 0;
        }
        for (uint32_t k = blockIdx.x * 64u + lane; k < L.cap_giant; k += gridDim.x * 64u) ((uint32_t *)(ws + L.gdone))[k] = 0;
    }
    if (blockIdx.x >= n_tiles) return;
    const uint64_t lo = (uint64_t)blockIdx.x * TILE;
    const uint64_t hi = min(lo + TILE, n);
    // wavefront 1: the window at the tile's end, bytes [hi - 64, hi + 8) and its document starts,
    // then the states the window fixes (beside wavefront 0's scan)
    if (wid == 1) {
        uint32_t wst = 0;
        if (blockIdx.x + 1 < n_tiles) {
            const uint64_t wb = hi - 64;
            const uint32_t wbyte0 = wb + lane < n ? bytes[wb + lane] : 0u;
            const uint32_t wbyte1 = lane < 8 && wb + 64 + lane < n ? bytes[wb + 64 + lane] : 0u;
            swin[lane] = (uint8_t)wbyte0;
            if (lane < 8) swin[64 + lane] = (uint8_t)wbyte1;
            // document starts in the window: narrow [lo, hi) of offsets down to at most 128 entries
            // that hold the first start >= wb, then read them (and the next 128 while they all lie
            // in the window)
            uint32_t dlo = 0, dhi = n_docs + 1;
            while (dhi - dlo > 128u) {
                const uint32_t step = (dhi - dlo + 63u) / 64u, idx = dlo + lane * step;
                const uint64_t t = __ballot(idx >= dhi || offsets[idx] >= wb);
                if (t == 0) { dlo = dlo + 63u * step; continue; }   // all probes before the window
                const uint32_t k = (uint32_t)__ffsll((unsigned long long)t) - 1u;
                const uint32_t nlo = k ? dlo + (k - 1u) * step : dlo, nhi = min(dhi, dlo + k * step + 1u);
                dlo = nlo;
                dhi = nhi;
            }
            uint32_t db0 = 0, db1 = 0, db2 = 0;
            for (;;) {
                uint64_t o[2];
                bool more = true;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t idx = dlo + 64u * h + lane;
                    o[h] = idx <= n_docs ? offsets[idx] : ~0ull;
                    if (o[h] >= wb && o[h] < wb + 72) {
                        const uint32_t j = (uint32_t)(o[h] - wb), bit = 1u << (j & 31u);
                        db0 |= j < 32u ? bit : 0u;
                        db1 |= j >= 32u && j < 64u ? bit : 0u;
                        db2 |= j >= 64u ? bit : 0u;
                    }
                }
                more = __builtin_amdgcn_readlane((int)(o[1] < wb + 72), 63) && dlo + 128u <= n_docs;
                if (!more) break;
                dlo += 128u;
            }
            db0 = wave_or(db0);
            db1 = wave_or(db1);
            db2 = wave_or(db2);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            wst = window_states(v, swin, [&](int j) -> bool {
                return (((j < 32 ? db0 : (j < 64 ? db1 : db2))) >> (j & 31)) & 1u;
            }, wb, n);
        }
        if (lane == 0) ((uint32_t *)(ws + L.twin))[blockIdx.x] = wst;
        return;
    }
    // wavefront 0: document starts in the pieces kernel's byte window of this tile, [lo - RAW_LEAD,
    // lo + TILE + RAW_TAIL): indices [d0, d1) of offsets (empty documents repeat one), kept for that
    // kernel; the window holds [lo, hi + 4), which the search below needs
    // (d1 and the first two starts from the 64 offsets after d0, read in one step; more steps only
    // for windows with more than 64 document starts)
    const uint64_t lo_w = lo >= (uint64_t)RAW_LEAD ? lo - RAW_LEAD : 0, hi_w = lo + TILE + RAW_TAIL;
    // the first scan step's bytes (4 per lane and the three after them, clamped to the batch; the
    // values past it unused), loaded with the document search's first offsets
    uint32_t pre[7];
#pragma unroll
    for (int t = 0; t < 7; ++t) pre[t] = bytes[min(lo + (uint64_t)(4u * lane + t), n - 1)];
    const uint32_t d0 = wave_lower_bound(offsets, n_docs + 1, lo_w);
    uint32_t d1 = d0, o0 = 0, o1 = 0;
    for (uint32_t b = d0;; b += 64u) {
        const uint32_t i = b + lane;
        const uint64_t o = i <= n_docs ? offsets[i] : ~0ull;
        if (b == d0) {
            o0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)o, 0);
            o1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)o, 1);
        }
        const uint64_t past = __ballot(o >= hi_w);
        if (past) {
            d1 = b + (uint32_t)__ffsll((unsigned long long)past) - 1u;
            break;
        }
    }
    if (lane == 0) {   // and the first two of those starts, so that the pieces kernel seldom reads offsets
        ((uint4 *)(ws + L.tdoc))[blockIdx.x] = make_uint4(d0, d1, d0 < d1 ? o0 : 0u, d0 + 1 < d1 ? o1 : 0u);
    }
    uint32_t na = BK_KEEP, au = BK_KEEP;
    // 64 T bytes per step, T per lane: the first step 256 bytes (where a flag is usually decided),
    // then 2 KiB steps (a tile inside a long whitespace or uppercase run decides nothing: 4 steps
    // instead of 31 dependent rounds of loads)
    auto scan = [&](uint64_t w, auto tc) {
        constexpr int T = decltype(tc)::value;
        // (the first step, 4 bytes per lane, from the bytes loaded above; the others byte by byte)
        constexpr int PRE = T == 4 ? 7 : 1;
        auto byte_at = [&](int t, uint64_t p) -> uint32_t { return T == 4 ? pre[t] : (uint32_t)bytes[p]; };
        uint32_t mna = BK_KEEP, mau = BK_KEEP;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint64_t p = w + (uint64_t)T * lane + t;
            if (p >= hi) continue;
            const uint32_t c = byte_at(t, p);
            if ((c & 0xC0u) == 0x80u) continue;
            uint32_t len = utf8_len(c), cp = c;
            const bool ok = len != 0 && p + len <= n;
            if (ok && len > 1) {
                cp = c & (0x7Fu >> len);
#pragma unroll
                for (uint32_t u = 1; u < 4; ++u)
                    if (u < len) cp = (cp << 6) | (byte_at(t + (int)u < PRE ? t + (int)u : 0, p + u) & 0x3Fu);
            }
            if (!ok) { len = 1; cp = 0xFFFDu; }
            const uint32_t code = ucat(cp) | ((c == '\r' || c == '\n') ? CC_CRLF : 0u);
            const uint64_t pn = p + len;
            bool eof_next = pn >= n;
            if (!eof_next) {
                uint32_t a = d0, b = d1;   // lower bound of pn among the tile's document starts
                while (a < b) {
                    const uint32_t m = (a + b) >> 1;
                    if (offsets[m] < pn) a = m + 1; else b = m;
                }
                eof_next = a < d1 && offsets[a] == pn;
            }
            uint32_t xna, xau;
            backward_maps(code, eof_next, xna, xau);
            if (mna == BK_KEEP) mna = xna;
            if (mau == BK_KEEP) mau = xau;
        }
        const uint64_t bna = __ballot(mna != BK_KEEP), bau = __ballot(mau != BK_KEEP);
        const uint32_t xna = (uint32_t)__builtin_amdgcn_readlane((int)mna, bna ? __ffsll((unsigned long long)bna) - 1 : 0);
        const uint32_t xau = (uint32_t)__builtin_amdgcn_readlane((int)mau, bau ? __ffsll((unsigned long long)bau) - 1 : 0);
        if (na == BK_KEEP && bna) na = xna;
        if (au == BK_KEEP && bau) au = xau;
    };
    uint64_t w = lo;
    if (w < hi) scan(w, StepBytes<4>{});   // (lo: the bytes in pre)
    for (w += 256; w < hi && (na == BK_KEEP || au == BK_KEEP); w += 64 * 32) scan(w, StepBytes<32>{});
    if (lane == 0) (ws + L.tbwd)[blockIdx.x] = (uint8_t)(na | (au << 2));

}

// The same per-byte code from registers: rw holds 24 bytes (4 before the thread's chunk, its 16, 4
// after), dm bit i says a document starts at window byte i, and window byte i is position
// p0 + i.  i is a compile-time index in the unrolled callers, so everything stays in registers.
__device__ __forceinline__ uint32_t wbyte(const uint32_t (&rw)[6], int i)
{
    return (rw[i >> 2] >> (8 * (i & 3))) & 255u;
}

__device__ __forceinline__ uint32_t reg_byte_code(const uint32_t (&rw)[6], uint32_t dm, int i, uint64_t p, uint64_t n,
                                                  int family, bool &bad)
{
    const uint32_t c = wbyte(rw, i);
    const bool isdoc = (dm >> i) & 1u;
    if ((c & 0xC0u) == 0x80u) {
        // a continuation byte must be covered by a lead byte 1..3 bytes back in the same doc
        bool ok = false, found = false;
#pragma unroll
        for (int back = 1; back <= 3; ++back) {
            if (found || (int64_t)p - back < 0) { found = true; continue; }
            const uint32_t lead = wbyte(rw, i - back);
            if ((lead & 0xC0u) != 0x80u) {
                ok = utf8_len(lead) > (uint32_t)back;
                found = true;
            }
        }
        bad |= !ok || isdoc;
        return CAT_CONT;
    }
    const uint32_t len = utf8_len(c);
    uint32_t cp = c;
    bool ok = len != 0 && p + len <= n;
    if (len > 1) {
        cp = c & (0x7Fu >> len);
#pragma unroll
        for (int t = 1; t < 4; ++t) {
            if ((uint32_t)t < len) {
                const uint32_t cb = wbyte(rw, i + t);
                ok &= ((cb & 0xC0u) == 0x80u) && !((dm >> (i + t)) & 1u);
                cp = (cp << 6) | (cb & 0x3Fu);
            }
        }
        ok &= !(len == 3 && cp < 0x800u) && !(len == 4 && (cp < 0x10000u || cp > 0x10FFFFu)) &&
              !(cp >= 0xD800u && cp <= 0xDFFFu);
    }
    bad |= !ok;
    if (!ok) cp = 0xFFFDu;
    uint32_t code = ucat(cp) | (isdoc ? CC_DOC : 0u);
    if (c == '\r' || c == '\n') code |= CC_CRLF;
    if (c == ' ') code |= CC_SP;
    if (family == FAMILY_DEEPSEEK) {
        code |= ds_bits(cp, code);
    } else if (c == '\'') {
        auto letter = [&](int t) -> uint32_t {
            if (p + t >= n || ((dm >> (i + t)) & 1u)) return 0;
            uint32_t x = wbyte(rw, i + t);
            if (family != 1 && x >= 'A' && x <= 'Z') x += 32;
            return x;
        };
        const uint32_t x1 = letter(1), x2 = letter(2);
        uint32_t lc = 0;
        if (x1 == 's' || x1 == 't' || x1 == 'm' || x1 == 'd') lc = 1;
        else if ((x1 == 'r' && x2 == 'e') || (x1 == 'v' && x2 == 'e') || (x1 == 'l' && x2 == 'l')) lc = 2;
        code |= lc << CC_CONTR_SHIFT;
    }
    return code;
}

// ---------------------------------------------------------------------------------------------
// k_pieces: dynamic tile ids; decode, automaton context, scans, look-backs, piece starts


// A backward flag of all 16 characters of a chunk at once.  Bit k of D: character k decides the
// flag (bit k of T: its value); other positions pass on the value of the position after them, and
// position 16 holds `carry`.  The result's bit k is the value of the first deciding position j >= k.
// On the bit-reversed masks the value moves upward through each run of pass-through positions; an
// addition carries it across the run.
__device__ __forceinline__ uint32_t fill_down16(uint32_t T, uint32_t D, uint32_t carry)
{
    const uint32_t Pr = __builtin_bitreverse32(~D & 0xFFFFu) >> 16, Tr = __builtin_bitreverse32(T) >> 16;
    const uint32_t s = ((Tr << 1) | carry) & Pr;
    const uint32_t filled = ((Pr + s) ^ Pr) & Pr;
    return __builtin_bitreverse32(Tr | filled) >> 16;
}

// first deciding value of a chunk from the left (the chunk's summary for the right-to-left scan)
__device__ __forceinline__ uint32_t first_decided(uint32_t T, uint32_t D)
{
    return D ? (((T >> (__ffs(D) - 1)) & 1u) ? (uint32_t)BK_T : (uint32_t)BK_F) : (uint32_t)BK_KEEP;
}

// contraction length code of an apostrophe at window index j of sraw (position p): 1 for 's 't 'm
// 'd, 2 for 're 've 'll (ASCII; case-insensitive except for the GPT-2 family), else 0
template <typename DocBit>
__device__ __forceinline__ uint32_t contraction_code(const uint8_t *sraw, DocBit docbit, int j, uint64_t p, uint64_t n,
                                                     int family)
{
    auto letter = [&](int t) -> uint32_t {
        if (p + t >= n || docbit(j + t)) return 0;
        uint32_t x = sraw[j + t];
        if (family != 1 && x >= 'A' && x <= 'Z') x += 32;
        return x;
    };
    const uint32_t x1 = letter(1), x2 = letter(2);
    if (x1 == 's' || x1 == 't' || x1 == 'm' || x1 == 'd') return 1;
    if ((x1 == 'r' && x2 == 'e') || (x1 == 'v' && x2 == 'e') || (x1 == 'l' && x2 == 'l')) return 2;
    return 0;
}

// VAR_CASE: the family has the case-boundary letter rule (the only one that reads the AU flag; for
// the others the flag changes no transition between reachable states and is left at zero).
// VAR_DS: the DeepSeek-style family (its own character bits and contexts, no contractions).
// Eight wavefronts per SIMD (at most 64 VGPRs): four tiles per CU, whose LDS (40 KB each) fits too;
// the tiles spend much of their time waiting on look-backs, which the fourth tile helps to hide.
enum : int { VAR_PLAIN = 0, VAR_CASE = 1, VAR_DS = 2 };

template <int VAR>
__global__ __launch_bounds__(PRE_THREADS) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_pieces(DevVocab v, const uint8_t *__restrict__ bytes, const uint64_t *__restrict__ offsets, uint32_t n_docs,
              uint64_t n, uint8_t *ws, Layout L)
{
    constexpr bool CASE = VAR == VAR_CASE, DS = VAR == VAR_DS;
    // context = ((self * 2 + doc) * NX + next) * AUM + au
    constexpr uint32_t NX = DS ? DS_NNEXT : NNEXT, AUM = DS ? 1u : 2u, NCTXV = DS ? DS_NCTX : NCTX;
    constexpr uint32_t NA_STEP = 2u * NX * AUM;   // NA set: the next self code (W0 -> W1, SP0 -> SP1)
    constexpr int NW = PRE_THREADS / 64;
    constexpr int SPAN = RAW_LEAD + TILE + RAW_TAIL;
    __shared__ __align__(16) uint8_t sraw[SPAN];
    __shared__ uint32_t sdoc[(SPAN + 31) / 32];
    __shared__ __align__(16) uint8_t scc[TILE + HALO];
    __shared__ uint16_t spiece[TILE];
    __shared__ uint4 smap16[NCTX_MAX + 1];      // [NCTXV]: identity (continuation bytes)
    __shared__ uint16_t sasc[128];              // ASCII character: byte code (no doc bit) | W, LU, LL, ' bits 8-11
    __shared__ uint16_t sctxa[256];             // byte code -> its part of the context (0xFFFF: not a character)
    __shared__ uint8_t sctxb[256];              // next character's byte code -> its part of the context
    __shared__ uint32_t sbkw[NW];
    __shared__ uint4 swmap[NW];
    __shared__ uint32_t swcnt[NW], swstate[NW];
    __shared__ uint32_t s_tile, s_carry, s_d0, s_d1, s_o0, s_o1, s_win, s_bk;

    const uint32_t n_tiles = request_sizes(L, n, n_docs);
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint8_t *tbwd = ws + L.tbwd;
    uint32_t *tfs = (uint32_t *)(ws + L.tflag_state);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;

    if (tid == 0) s_tile = atomicAdd(&ctrl->tile_ctr_pre, 1u);
    for (int i = tid; i < (int)NCTXV; i += PRE_THREADS) smap16[i] = v.fmap16[i];
    if (tid == 0) smap16[NCTXV] = make_uint4(0x03020100u, 0x07060504u, 0x0B0A0908u, 0x0F0E0D0Cu);
    if (tid < 128) {
        const uint32_t u = ucat(tid), cat = u & 7u;
        sasc[tid] = (uint16_t)(u | ((tid == '\r' || tid == '\n') ? CC_CRLF : 0u) | (tid == ' ' ? CC_SP : 0u) |
                               (DS ? ds_bits(tid, u) : 0u) |
                               (cat == CAT_W ? 0x100u : 0u) | (cat == CAT_LU ? 0x200u : 0u) |
                               (cat == CAT_LL ? 0x400u : 0u) | (tid == '\'' ? 0x800u : 0u));
    }
    if (tid < 256) {
        // the self / doc part of the context (self code with NA clear) and the next-character part
        const uint32_t selfc = DS ? self_code_ds(tid) : self_code(tid, false);
        const uint32_t nextc = DS ? next_code_ds(tid) : ((tid & 7u) == CAT_CONT ? 5u : next_code(tid));
        sctxa[tid] = (tid & 7u) == CAT_CONT ? (uint16_t)0xFFFFu
                                             : (uint16_t)((selfc * 2u + ((tid & CC_DOC) ? 1u : 0u)) * NX * AUM);
        sctxb[tid] = (uint8_t)(nextc * AUM);
    }
    for (int j = tid; j < (SPAN + 31) / 32; j += PRE_THREADS) sdoc[j] = 0;
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile >= n_tiles) return;   // (a request smaller than the plan's size bucket)
    const uint64_t lo = (uint64_t)tile * TILE;
    const int64_t base = (int64_t)lo - RAW_LEAD;
    // summaries of the next 64 tiles for the backward carry (wave 0), loaded now so that the load
    // overlaps the decode
    uint32_t bk_first = BK_T | (BK_T << 2);
    if (wid == 0 && tile + 1 + lane < n_tiles) bk_first = (ws + L.tbwd)[tile + 1 + lane];

    // raw bytes [lo - 4, lo + TILE + 24), as 32-bit words
    // (interior words from two aligned 4-byte loads, which never leave the pages of the bytes they
    // hold; the words at the batch edges byte by byte).  Inside the batch every thread issues all of
    // its loads before storing any, so that they are in flight together.
    if (base >= 0 && (uint64_t)base + SPAN <= n) {
        constexpr int RW = (SPAN / 4 + PRE_THREADS - 1) / PRE_THREADS;
        const uintptr_t a0 = (uintptr_t)(bytes + base);
        const uint32_t *al = (const uint32_t *)(a0 & ~(uintptr_t)3);
        const uint32_t sh = (uint32_t)(a0 & 3u);
        uint32_t x0[RW], x1[RW];
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            const uint32_t j = min((uint32_t)(tid + k * PRE_THREADS), (uint32_t)(SPAN / 4 - 1));
            x0[k] = al[j];
            x1[k] = sh ? al[j + 1] : 0u;
        }
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            const uint32_t j = tid + k * PRE_THREADS;
            if (j < (uint32_t)(SPAN / 4)) ((uint32_t *)sraw)[j] = sh ? __builtin_amdgcn_alignbyte(x1[k], x0[k], sh) : x0[k];
        }
    } else for (int j = tid; j < SPAN / 4; j += PRE_THREADS) {
        const int64_t p = base + 4 * j;
        uint32_t w = 0;
        if (p >= 0 && (uint64_t)p + 4 <= n) {
            const uintptr_t a = (uintptr_t)(bytes + p);
            const uint32_t *al = (const uint32_t *)(a & ~(uintptr_t)3);
            const uint32_t sh = 8u * (uint32_t)(a & 3u);
            const uint32_t w0 = al[0];
            w = sh ? __builtin_amdgcn_alignbyte(al[1], w0, sh >> 3) : w0;
        } else {
            for (int t = 0; t < 4; ++t)
                if (p + t >= 0 && (uint64_t)(p + t) < n) w |= (uint32_t)bytes[p + t] << (8 * t);
        }
        ((uint32_t *)sraw)[j] = w;
    }
    if (tid == 0) {   // documents starting in [base, base + SPAN), found by k_summary
        const uint4 dd = ((const uint4 *)(ws + L.tdoc))[tile];
        s_d0 = dd.x;
        s_d1 = dd.y;
        s_o0 = dd.z;
        s_o1 = dd.w;
    } else if (tid == 64) {
        // the previous tile's window states and this tile's own backward summary (which of those
        // states applies)
        s_win = tile > 0 ? ((const uint32_t *)(ws + L.twin))[tile - 1] : 0u;
        s_bk = (ws + L.tbwd)[tile];
    }
    // document offsets must start at 0, never decrease and end at n
    bool bad_offs = false;
    for (uint64_t d = (uint64_t)tile * PRE_THREADS + tid; d < n_docs; d += (uint64_t)n_tiles * PRE_THREADS)
        if (offsets[d] > offsets[d + 1]) bad_offs = true;
    if (tile == 0 && tid == 0 && (offsets[0] != 0 || offsets[n_docs] != n)) bad_offs = true;
    if (bad_offs) atomicOr(&ctrl->status, ST_BAD_OFFSETS);
    __syncthreads();
    for (uint32_t d = s_d0 + tid; d < s_d1; d += PRE_THREADS) {
        const uint64_t od = d == s_d0 ? s_o0 : d == s_d0 + 1 ? s_o1 : offsets[d];
        int64_t j = (int64_t)od - base;
        if (j >= 0 && j < SPAN) atomicOr(&sdoc[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    auto docbit = [&](int j) -> bool { return (sdoc[j >> 5] >> (j & 31)) & 1u; };

    // per-byte codes of the tile (validated) and of the halo after it, and per-chunk masks of the
    // characters (bit k: byte k of the chunk).  A wavefront whose bytes are all ASCII takes its codes
    // and masks from a table; the others decode UTF-8.
    const int c0 = tid * PRE_CHUNK;
    const uint64_t pos0 = lo + (uint64_t)c0;
    // bytes 0..16 of the chunk at or past the end of the batch
    const uint32_t rem = pos0 >= n ? 0u : (n - pos0 > 17u ? 17u : (uint32_t)(n - pos0));
    const uint32_t xeof = (0x1FFFFu << rem) & 0x1FFFFu;
    uint32_t dm = 0, mW = 0, mC = 0, mU = 0, mL = 0, mX = xeof & 0xFFFFu;
    bool ascii = false;
    {
        bool bad = false;
        // window: sraw[c0 .. c0 + 24) = positions lo + c0 - 4 ...; 16-byte aligned LDS reads
        static_assert(RAW_LEAD == 4 && PRE_CHUNK == 16, "window layout");
        const uint4 r0 = *(const uint4 *)(sraw + c0);
        const uint2 r1 = *(const uint2 *)(sraw + c0 + 16);
        const uint32_t rw[6] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y};
        const uint32_t dw = (uint32_t)c0 >> 5;
        dm = (uint32_t)((((uint64_t)sdoc[dw + 1] << 32) | sdoc[dw]) >> (c0 & 31));
        uint32_t w[PRE_CHUNK / 4] = {0, 0, 0, 0};
        const uint32_t hibits = (rw[0] | rw[1] | rw[2] | rw[3] | rw[4] | rw[5]) & 0x80808080u;
        ascii = __ballot(hibits != 0) == 0;
        if (ascii) {
            // every byte the wavefront looks at is ASCII: a table lookup per byte; the few document
            // starts, positions past the end of the batch (byte 0: no mask bit) and apostrophes are
            // applied afterwards, bit by bit
            uint32_t apos = 0;
#pragma unroll
            for (int k = 0; k < PRE_CHUNK; ++k) {
                const uint32_t f = sasc[wbyte(rw, k + RAW_LEAD)];
                w[k >> 2] |= (f & 0xFFu) << (8 * (k & 3));
                mW |= ((f >> 8) & 1u) << k;
                mC |= ((f >> 3) & 1u) << k;
                if (!DS) apos |= ((f >> 11) & 1u) << k;
                if (CASE) {
                    mU |= ((f >> 9) & 1u) << k;
                    mL |= ((f >> 10) & 1u) << k;
                }
            }
            apos &= ~xeof;
            auto or_code = [&](int k, uint32_t add) {   // add to the code of byte k (k not uniform)
                const int q = k >> 2;
                add <<= 8 * (k & 3);
                w[0] |= q == 0 ? add : 0u;
                w[1] |= q == 1 ? add : 0u;
                w[2] |= q == 2 ? add : 0u;
                w[3] |= q == 3 ? add : 0u;
            };
            for (uint32_t m = (dm >> RAW_LEAD) & 0xFFFFu; m; m &= m - 1) or_code(__ffs(m) - 1, CC_DOC);
            for (uint32_t m = xeof & 0xFFFFu; m; m &= m - 1) or_code(__ffs(m) - 1, CC_EOF);
            while (apos) {
                const int k = __ffs(apos) - 1;
                apos &= apos - 1;
                or_code(k, contraction_code(sraw, docbit, RAW_LEAD + c0 + k, lo + c0 + k, n, v.family) << CC_CONTR_SHIFT);
            }
        } else {
#pragma unroll
            for (int k = 0; k < PRE_CHUNK; ++k) {
                const uint32_t code = ((xeof >> k) & 1u) ? (uint32_t)CC_EOF
                                                         : reg_byte_code(rw, dm, k + RAW_LEAD, pos0 + k, n, v.family, bad);
                w[k >> 2] |= code << (8 * (k & 3));
                const uint32_t cat = code & 7u;
                mW |= ((0x10u >> cat) & 1u) << k;                   // whitespace
                mC |= ((code >> 3) & (0x10u >> cat) & 1u) << k;     // CR/LF
                mX |= ((0x80u >> cat) & 1u) << k;                   // continuation byte or past the end
                if (CASE) {
                    mU |= ((0x01u >> cat) & 1u) << k;               // uppercase letter
                    mL |= ((0x26u >> cat) & 1u) << k;               // lowercase or other letter, mark
                }
            }
        }
        *(uint4 *)(scc + c0) = make_uint4(w[0], w[1], w[2], w[3]);
        if (tid < HALO) {
            const uint64_t p = lo + TILE + tid;
            bool ignore = false;
            scc[TILE + tid] = p < n ? (uint8_t)byte_code(sraw, docbit, RAW_LEAD + TILE + tid, p, n, v.family, false,
                                                         ignore)
                                    : CC_EOF;
        }
        if (bad) atomicOr(&ctrl->status, ST_BAD_UTF8);
    }

    // backward carry into this tile: first non-pass-through summary of a later tile
    if (wid == 0) {
        uint32_t na = BK_KEEP, au = BK_KEEP;
        for (uint32_t t0 = tile + 1; na == BK_KEEP || au == BK_KEEP; t0 += 64) {
            uint32_t t = t0 + lane;
            uint32_t x = t0 == tile + 1 ? bk_first : t < n_tiles ? (uint32_t)tbwd[t] : (BK_T | (BK_T << 2));
            uint64_t mna = __ballot((x & 3u) != 0), mau = __ballot((x >> 2) != 0);
            uint32_t xna = (uint32_t)__builtin_amdgcn_readlane((int)x, mna ? __ffsll((unsigned long long)mna) - 1 : 0);
            uint32_t xau = (uint32_t)__builtin_amdgcn_readlane((int)x, mau ? __ffsll((unsigned long long)mau) - 1 : 0);
            if (na == BK_KEEP && mna) na = xna & 3u;
            if (au == BK_KEEP && mau) au = xau >> 2;
        }
        if (lane == 0) s_carry = (na & 1u) | ((au & 1u) << 1);
    }
    __syncthreads();

    // codes of the chunk's 16 bytes and the 4 after it
    uint32_t cw[5];
    {
        const uint4 a = *(const uint4 *)(scc + c0);
        cw[0] = a.x; cw[1] = a.y; cw[2] = a.z; cw[3] = a.w;
        cw[4] = *(const uint32_t *)(scc + c0 + PRE_CHUNK);
    }
    auto code_at = [&](int k) -> uint32_t { return (cw[k >> 2] >> (8 * (k & 3))) & 255u; };
    // code of the character after each byte (packed like cw) and the mask of bytes whose next
    // character starts a document or lies past the end of the batch
    uint32_t ncw[PRE_CHUNK / 4], en;
    if (ascii) {
#pragma unroll
        for (int j = 0; j < PRE_CHUNK / 4; ++j) ncw[j] = __builtin_amdgcn_alignbyte(cw[j + 1], cw[j], 1);
        en = ((dm >> (RAW_LEAD + 1)) | (xeof >> 1)) & 0xFFFFu;
    } else {
        // right to left: the first byte after j that is not a continuation byte (byte 19 at the latest)
        uint32_t nxt = code_at(PRE_CHUNK + 3);
        ncw[0] = ncw[1] = ncw[2] = ncw[3] = 0;
        en = 0;
#pragma unroll
        for (int j = PRE_CHUNK + 2; j >= 0; --j) {
            if (j < PRE_CHUNK) {
                ncw[j >> 2] |= nxt << (8 * (j & 3));
                en |= ((nxt >> 7) | ((0x80u >> (nxt & 7u)) & 1u)) << j;
            }
            const uint32_t cj = code_at(j);
            nxt = ((cj & 7u) == CAT_CONT && cj != CC_EOF) ? nxt : cj;
        }
    }

    // The two backward flags of the chunk's characters.  NA is decided by a character that is not
    // whitespace (true), a CR/LF (false) or whitespace whose next character starts a document (true);
    // AU by a character that is not a letter or mark (true), a lowercase or other letter or a mark
    // (false) or an uppercase letter whose next character starts a document (true).  Continuation
    // bytes and the other characters pass on the value of the position after them.
    const uint32_t isch = ~mX & 0xFFFFu;
    uint32_t tna, dna, tau = 0, dau = 0;
    {
        const uint32_t ws_ = mW & isch, crlf = mC & isch;
        tna = (isch & ~ws_) | (ws_ & ~crlf & en);
        dna = tna | crlf;
        if (CASE) {
            const uint32_t up = mU & isch, low = mL & isch;
            tau = (isch & ~(up | low)) | (up & en);
            dau = tau | low;
        }
    }
    // value entering each chunk from its right: that of the first chunk to the right whose flag is
    // decided -- in the wavefront, the first deciding lane after this one (two ballots per flag: the
    // deciding lanes and their values); then the wavefronts to the right, then the tile carry
    auto bk_comb = [](uint32_t x, uint32_t r) -> uint32_t {
        if ((x & 3u) == BK_KEEP) x = (x & ~3u) | (r & 3u);
        if ((x >> 2) == BK_KEEP) x = (x & 3u) | (r & ~3u);
        return x;
    };
    const uint32_t agg_na = first_decided(tna, dna), agg_au = CASE ? first_decided(tau, dau) : (uint32_t)BK_KEEP;
    const uint64_t d_na = __ballot(agg_na != BK_KEEP), t_na = __ballot(agg_na == BK_T);
    const uint64_t d_au = CASE ? __ballot(agg_au != BK_KEEP) : 0ull, t_au = CASE ? __ballot(agg_au == BK_T) : 0ull;
    auto first_of = [](uint64_t d, uint64_t t) -> uint32_t {   // first deciding lane of d, BK_KEEP if none
        return d ? (((t >> (__ffsll((unsigned long long)d) - 1)) & 1ull) ? (uint32_t)BK_T : (uint32_t)BK_F)
                 : (uint32_t)BK_KEEP;
    };
    if (lane == 0) sbkw[wid] = first_of(d_na, t_na) | (first_of(d_au, t_au) << 2);
    const uint64_t after = ~((2ull << lane) - 1ull);   // the lanes after this one (none for lane 63)
    __syncthreads();
    uint32_t right = first_of(d_na & after, t_na) | (first_of(d_au & after, t_au) << 2);
    for (uint32_t w = wid + 1; w < (uint32_t)NW; ++w) right = bk_comb(right, sbkw[w]);
    const uint32_t na_in = ((right & 3u) == BK_KEEP) ? (s_carry & 1u) : (right & 1u);
    const uint32_t au_in = ((right >> 2) == BK_KEEP) ? ((s_carry >> 1) & 1u) : ((right >> 2) & 1u);

    // each character's automaton context (packed 16 bits per character): the sum of two table
    // entries (the character's code, the next character's code) and the two flags; continuation
    // bytes and positions past the end saturate to the identity map
    uint32_t pk_ctx[PRE_CHUNK / 2] = {0, 0, 0, 0, 0, 0, 0, 0};
    {
        const uint32_t naw = fill_down16(tna, dna, na_in) & mW & ~mC;   // whitespace (not CR/LF) with NA set
        uint32_t aun = 0;
        if (CASE) aun = (fill_down16(tau, dau, au_in) >> 1) | (au_in << 15);   // AU of the next character
#pragma unroll
        for (int k = 0; k < PRE_CHUNK; ++k) {
            const uint32_t nc = (ncw[k >> 2] >> (8 * (k & 3))) & 255u;
            uint32_t ctx = (uint32_t)sctxa[code_at(k)] + (uint32_t)sctxb[nc] + NA_STEP * ((naw >> k) & 1u);
            if (CASE) ctx += (aun >> k) & 1u;
            ctx = min(ctx, NCTXV);
            pk_ctx[k >> 1] |= ctx << (16 * (k & 1));
        }
    }
    auto ctx_at = [&](int k) -> uint32_t { return (pk_ctx[k >> 1] >> (16 * (k & 1))) & 0xFFFFu; };

    // The chunk's map, composed from the left until the map of every chunk of the wavefront sends
    // all states to one state (a few characters of text nearly always do: only runs of digits and
    // the first characters of a contraction keep states apart).  From there on each lane follows
    // its one state, and the piece-start bits of those bytes no longer depend on the state that
    // enters the chunk.  `kconv` (uniform) is the number of bytes composed.
    const uint8_t *smb = (const uint8_t *)smap16;
    M16 acc = m16_identity();
    uint32_t kconv = PRE_CHUNK, s_run = 0, tail_mask = 0;
#pragma unroll
    for (int k = 0; k < PRE_CHUNK; ++k) {
        if (kconv == PRE_CHUNK) {
            const uint4 m = smap16[ctx_at(k)];
            acc = compose16(acc, M16{{m.x, m.y, m.z, m.w}});
            if ((k & 1) && k + 1 < PRE_CHUNK && __ballot(!is_const16(acc)) == 0) {
                kconv = k + 1;
                s_run = acc.w[0] & 15u;
            }
        } else {
            const uint32_t b = smb[ctx_at(k) * 16u + s_run];
            tail_mask |= ((b >> 4) & 1u) << k;
            s_run = b & 15u;
        }
    }
    const bool wave_const = kconv < PRE_CHUNK;
    if (wave_const) acc = m16_const(s_run);

    // wavefront scan of the chunk maps (a shift of one state when every map is constant); the
    // wavefronts' maps are scanned by wave 0, which also takes the state entering the tile from the
    // look-back
    M16 incl = acc;
    const uint32_t prev_run = __shfl_up(s_run, 1, 64);   // (constant maps: the state entering the chunk)
    if (!wave_const) {
        // inside each row of 16 lanes (DPP row shifts), then across rows (row broadcasts of lanes 15
        // and 31), composing the farther map first
        const uint32_t r = lane & 15u, row = lane >> 4;
#define TT_DPP4(ctrl, rmask) M16{{(uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl.w[0], ctrl, rmask, 0xF, false), \
                                  (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl.w[1], ctrl, rmask, 0xF, false), \
                                  (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl.w[2], ctrl, rmask, 0xF, false), \
                                  (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl.w[3], ctrl, rmask, 0xF, false)}}
        { const M16 y = TT_DPP4(0x111, 0xF); if (r >= 1) incl = compose16(y, incl); }
        { const M16 y = TT_DPP4(0x112, 0xF); if (r >= 2) incl = compose16(y, incl); }
        { const M16 y = TT_DPP4(0x114, 0xF); if (r >= 4) incl = compose16(y, incl); }
        { const M16 y = TT_DPP4(0x118, 0xF); if (r >= 8) incl = compose16(y, incl); }
        { const M16 y = TT_DPP4(0x142, 0xA); if (row & 1u) incl = compose16(y, incl); }   // row_bcast:15
        { const M16 y = TT_DPP4(0x143, 0xC); if (row >= 2) incl = compose16(y, incl); }   // row_bcast:31
#undef TT_DPP4
    }
    M16 excl = m16_identity();
    if (!wave_const) {
        excl = shfl_up16(incl, 1);
        if (lane == 0) excl = m16_identity();
    }
    if (lane == 63) swmap[wid] = make_uint4(incl.w[0], incl.w[1], incl.w[2], incl.w[3]);
    __syncthreads();
    if (wid == 0) {
        M16 wm = m16_identity();
        if (lane < (uint32_t)NW) {
            const uint4 t = swmap[lane];
            wm = M16{{t.x, t.y, t.z, t.w}};
        }
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            const M16 y = shfl_up16(wm, d);
            if (lane >= (uint32_t)d) wm = compose16(y, wm);
        }
        M16 wex = shfl_up16(wm, 1);
        if (lane == 0) wex = m16_identity();
        const M16 tile_map = shfl16(wm, NW - 1);
        // automaton state entering this tile: fixed by the previous tile's last bytes, else from the
        // look-back (this tile's flags: its map, then the state after it)
        const uint32_t bk_self = s_bk;
        const uint32_t na_prev = (bk_self & 3u) != BK_KEEP ? (bk_self & 1u) : (s_carry & 1u);
        const uint32_t au_prev = (bk_self >> 2) != BK_KEEP ? ((bk_self >> 2) & 1u) : ((s_carry >> 1) & 1u);
        const uint32_t wv = (s_win >> (8u * (na_prev | (CASE ? au_prev << 1 : 0u)))) & 0xFFu;
        uint32_t entry = S_ST;
        if (tile > 0) {
            if (wv & 0x10u) {
                entry = wv & 15u;
            } else {
                if (lane == 0) st_flag16(tfs + 4 * tile, tile_map, FLAG_AGG);
                entry = lookback_state(tfs, tile);
            }
        }
        if (lane == 0) st_flag16(tfs + 4 * tile, m16_const(byte16(tile_map, entry) & 15u), FLAG_PREFIX);
        if (lane < (uint32_t)NW) swstate[lane] = byte16(wex, entry) & 15u;
    }
    __syncthreads();

    // piece starts of this chunk: the bytes before kconv from the state entering the chunk (those
    // after it were found by the single-state run)
    uint32_t s = (wave_const && lane > 0) ? prev_run : byte16(excl, swstate[wid]) & 15u, mask = tail_mask;
#pragma unroll
    for (int k = 0; k < PRE_CHUNK; ++k) {
        if ((uint32_t)k < kconv) {
            const uint32_t b = smb[ctx_at(k) * 16u + s];
            mask |= ((b >> 4) & 1u) << k;
            s = b & 15u;
        }
    }
    const uint32_t cnt = __popc(mask), icnt = wave_incl_sum(cnt);
    if (lane == 63) swcnt[wid] = icnt;
    __syncthreads();
    uint32_t before = icnt - cnt, total = 0;
    for (uint32_t w = 0; w < (uint32_t)NW; ++w) {
        if (w < wid) before += swcnt[w];
        total += swcnt[w];
    }
    // stage this tile's starts in LDS for a coalesced write
    {
        uint32_t o = before, m = mask;
        while (m) {
            int k = __ffs(m) - 1;
            m &= m - 1;
            spiece[o++] = (uint16_t)(c0 + k);
        }
    }

    __syncthreads();
    // the tile's piece count and first start, and its starts as offsets at the tile's own place;
    // the compaction kernel gives them their global places once every tile has its count
    if (tid == 0) {
        ((uint32_t *)(ws + L.tcnt))[tile] = total;
        ((uint32_t *)(ws + L.tfirst))[tile] = total ? (uint32_t)lo + spiece[0] : NO_START;
        if (total) atomicAdd((uint32_t *)(ws + L.gsum) + tile / 64u, total);
    }
    uint16_t *prs = (uint16_t *)(ws + L.prs) + lo;
    for (uint32_t i = tid; i < total; i += PRE_THREADS) prs[i] = spiece[i];
}

// k_compact: one workgroup per tile puts the tile's piece starts at their global places (the pieces
// before the tile: the 64-tile group sums before its group, then the tiles of its group before
// it), records the tile's first piece index, and lists the pieces longer than SHORT_MAX by length.
// The last piece of a tile ends at the first start of the next tile that has one, else at the end
// of the batch.
__global__ __launch_bounds__(256) void k_compact(uint8_t *ws, Layout L, uint64_t n)
{
    __shared__ __align__(16) uint16_t sps[TILE];
    __shared__ uint32_t s_base, s_next;
    uint32_t n_docs = 0;
    const uint32_t n_tiles = request_sizes(L, n, n_docs);
    const uint32_t tile = blockIdx.x;
    if (tile >= n_tiles) return;
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *tcnt = (const uint32_t *)(ws + L.tcnt), *tfirst = (const uint32_t *)(ws + L.tfirst);
    const uint32_t *gsum = (const uint32_t *)(ws + L.gsum);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    const uint32_t cnt = tcnt[tile], lo = tile * (uint32_t)TILE;
    // every load at once: the tile's start offsets (16 bytes per load, into LDS; the last vector may
    // run past the count, inside the tile's part of the array), the pieces before the tile (wave 0)
    // and the first start after it (wave 1)
    {
        const uint4 *src = (const uint4 *)((const uint16_t *)(ws + L.prs) + lo);
        const uint32_t nv = (cnt + 7u) / 8u;   // <= TILE / 8 = 4 per thread
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t v = tid + 256u * k;
            if (v < nv) ((uint4 *)sps)[v] = src[v];
        }
    }
    if (wid == 0) {
        const uint32_t g = tile / 64u;
        uint32_t x = 0;
        for (uint32_t k = lane; k < g; k += 64u) x += gsum[k];
        if (64u * g + lane < tile) x += tcnt[64u * g + lane];
        x = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(x), 63);
        if (lane == 0) s_base = x;
    } else if (wid == 1) {
        uint32_t nx = (uint32_t)n;
        for (uint32_t t0 = tile + 1; t0 < n_tiles; t0 += 64u) {
            const uint32_t t = t0 + lane;
            const uint32_t f = t < n_tiles ? tfirst[t] : NO_START;
            const uint64_t has = __ballot(f != NO_START);
            if (has) {
                nx = (uint32_t)__builtin_amdgcn_readlane((int)f, __ffsll((unsigned long long)has) - 1);
                break;
            }
        }
        if (lane == 0) s_next = nx;
    }
    __syncthreads();
    const uint32_t base = s_base, next = s_next;
    uint32_t *pstart = (uint32_t *)(ws + L.pstart);
    for (uint32_t i = tid; i < cnt; i += 256u) {
        const uint32_t a = lo + sps[i], e = i + 1 < cnt ? lo + sps[i + 1] : next;
        pstart[base + i] = a;
        if (e - a > (uint32_t)SHORT_MAX) list_long(ws, L, ctrl, base + i, e - a);
    }
    if (tid == 0) {
        ((uint32_t *)(ws + L.tbase))[tile] = base;
        if (tile == n_tiles - 1) {
            ctrl->n_pieces = base + cnt;
            pstart[base + cnt] = (uint32_t)n;
            ((uint32_t *)(ws + L.tbase))[n_tiles] = base + cnt;
        }
    }
}

// ---------------------------------------------------------------------------------------------

hipError_t launch_pretokenize(const DevVocab &v, const Batch &b, hipStream_t s, const Events *ev, bool compact)
{
    const Layout &L = b.L;
    {
        LaunchScope k(ev, TK_SUMMARY, s);
        hipLaunchKernelGGL(k_summary, dim3(L.n_tiles ? L.n_tiles : 1u), dim3(128), 0, s, v, b.bytes, b.offsets, b.n_docs,
                           b.n, b.ws, L);
    }
    if (L.n_tiles == 0) return hipGetLastError();
    {
        LaunchScope k(ev, TK_PIECES, s);
        const dim3 grid(L.n_tiles);
        if (v.family == FAMILY_O200K)
            hipLaunchKernelGGL(k_pieces<VAR_CASE>, grid, dim3(PRE_THREADS), 0, s, v, b.bytes, b.offsets, b.n_docs,
                               b.n, b.ws, L);
        else if (v.family == FAMILY_DEEPSEEK)
            hipLaunchKernelGGL(k_pieces<VAR_DS>, grid, dim3(PRE_THREADS), 0, s, v, b.bytes, b.offsets, b.n_docs,
                               b.n, b.ws, L);
        else
            hipLaunchKernelGGL(k_pieces<VAR_PLAIN>, grid, dim3(PRE_THREADS), 0, s, v, b.bytes, b.offsets, b.n_docs,
                               b.n, b.ws, L);
        if (compact) hipLaunchKernelGGL(k_compact, grid, dim3(256), 0, s, b.ws, L, b.n);
    }
    return hipGetLastError();
}

// the piece starts as one array (pretokenize-only calls): n_pieces starts, then the batch end
__global__ __launch_bounds__(256) void k_export_starts(uint8_t *ws, Layout L, uint64_t n, uint32_t *out)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t np = ctrl->n_pieces;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i <= np; i += gridDim.x * blockDim.x)
        out[i] = i == np ? (uint32_t)n : pstart[i];
}

hipError_t launch_export_starts(const Batch &b, uint32_t *out_starts, hipStream_t s)
{
    uint32_t g = (uint32_t)((b.n + 1 + 255) / 256);
    hipLaunchKernelGGL(k_export_starts, dim3(g > 4096 ? 4096 : g), dim3(256), 0, s, b.ws, b.L, b.n, out_starts);
    return hipGetLastError();
}

}  // namespace tt
