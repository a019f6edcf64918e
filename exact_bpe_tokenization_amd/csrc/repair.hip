// repair.hip -- incremental repair of an appended request, on top of the GPU encoder.
//
// TokTier (arXiv 2607.29678), incremental repair section and Figure 5: a session holds the records
// (token ID, source byte offset) of its text A; the next request is A || B.  The last w characters
// of A (w = 512, doubled at most five times) and B are encoded as a window; the longest run of
// records on which the cached and the window's records agree in position and ID is searched, and a
// splice in that run is accepted only under a certificate; otherwise the window grows, and after
// the last window the whole text is encoded.  A miss costs work, never exactness: the result always
// equals the full encoding of A || B.
//
// The certificate, derived here in terms of this library's pre-tokenizer automaton (the pages' own
// proof is in terms of synchronizing character-class transitions).  Let s be the window's first
// character and e a character of A.
//  (R) If the composition of the transition maps of characters s+1 .. e-1 sends every state to one
//      state, the full text and the window enter e in the same state.  Their contexts from s+1 on
//      are the same (a context reads the character, the next two bytes and backward flags, all
//      from the right), so from e on they have the same piece starts.
//  (L) If every context up to e is the same for A alone as for A || B, the two have the same piece
//      starts up to e.  A context can read past the end of A only within A's last two characters,
//      within A's trailing whitespace other than CR/LF (the "no CR/LF ahead" flag), and for the
//      o200k family within its trailing uppercase letters (the "only uppercase ahead" flag); e must
//      lie before all three.
//  If moreover e starts a piece in the window, it starts a piece in the full text and in A alone,
//  and since BPE encodes each piece on its own, the full encoding is A's records before e followed
//  by the window's records from e.  The pages' other two conditions -- the equal run holds at least
//  two tokens and covers more bytes than the longest token -- are kept as stated; e is the last
//  record boundary of the equal run that passes the certificate.
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/toktier.h"
#include "internal.h"
#include "vocab.h"
#include "unicode_table.inc"

using namespace tt;

namespace {

constexpr uint32_t REPAIR_W0 = 512;      // first window, characters of A
constexpr uint32_t REPAIR_DOUBLINGS = 5;

uint32_t ucat_host(uint32_t cp)
{
    if (cp < 0x80u) {
        const uint32_t lc = cp | 32u;
        if (lc >= 'a' && lc <= 'z') return cp >= 'a' ? CAT_LL : CAT_LU;
        if (cp >= '0' && cp <= '9') return CAT_N;
        if (cp == ' ' || (cp >= 9u && cp <= 13u)) return CAT_W;
        return (cp >= 0x21u && cp <= 0x7Eu) ? (uint32_t)(CAT_O | CC_PS) : (uint32_t)CAT_O;
    }
    return tt_ucat_stage2[((uint32_t)tt_ucat_stage1[cp >> 8] << 8) | (cp & 255u)];
}

// character starts of valid UTF-8 text (pos[k] = byte offset of character k, pos[nc] = n) and the
// code points; false on invalid UTF-8
bool decode(const uint8_t *s, uint64_t n, std::vector<uint64_t> &pos, std::vector<uint32_t> &cps)
{
    pos.clear();
    cps.clear();
    for (uint64_t i = 0; i < n;) {
        const uint32_t c = s[i];
        const uint32_t len = c < 0x80 ? 1 : (c >> 5) == 6 ? 2 : (c >> 4) == 14 ? 3 : (c >> 3) == 30 ? 4 : 0;
        if (!len || i + len > n) return false;
        uint32_t cp = len == 1 ? c : c & (0x7Fu >> len);
        for (uint32_t k = 1; k < len; ++k) {
            if ((s[i + k] & 0xC0) != 0x80) return false;
            cp = (cp << 6) | (s[i + k] & 0x3Fu);
        }
        static const uint32_t min_cp[5] = {0, 0, 0x80, 0x800, 0x10000};
        if (cp < min_cp[len] || cp > 0x10FFFF || (cp >= 0xD800 && cp <= 0xDFFF)) return false;
        pos.push_back(i);
        cps.push_back(cp);
        i += len;
    }
    pos.push_back(n);
    return true;
}

// The byte code of character k of the text [0, n) (one document), as the pieces kernel forms it.
uint32_t char_code(int family, const uint8_t *s, uint64_t n, const std::vector<uint64_t> &pos,
                   const std::vector<uint32_t> &cps, uint64_t k, bool doc)
{
    const uint64_t p = pos[k];
    const uint32_t c = s[p], cp = cps[k];
    uint32_t code = ucat_host(cp) | (doc ? CC_DOC : 0u);
    if (c == '\r' || c == '\n') code |= CC_CRLF;
    if (c == ' ') code |= CC_SP;
    if (family == FAMILY_DEEPSEEK) {
        code |= ds_bits(cp, code);
    } else if (c == '\'') {
        auto letter = [&](uint64_t t) -> uint32_t {
            if (p + t >= n) return 0;
            uint32_t x = s[p + t];
            if (family != FAMILY_GPT2 && x >= 'A' && x <= 'Z') x += 32;
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

// Automaton contexts of characters [k0, nc) of the text [0, n), one document starting at character
// k0 when doc0 is set (a window), else inside a document that started earlier.
void contexts(int family, const uint8_t *s, uint64_t n, const std::vector<uint64_t> &pos,
              const std::vector<uint32_t> &cps, uint64_t k0, bool doc0, std::vector<uint32_t> &ctx)
{
    const uint64_t nc = cps.size();
    const uint64_t m = nc - k0;
    std::vector<uint32_t> code(m);
    for (uint64_t i = 0; i < m; ++i) code[i] = char_code(family, s, n, pos, cps, k0 + i, doc0 && i == 0);
    // backward flags: NA = no CR/LF from here to the end of this whitespace run; AU = only uppercase
    // letters from here to the end of this letter run (each true past the end of the text)
    std::vector<uint8_t> na(m + 1, 1), au(m + 1, 1);
    for (uint64_t i = m; i-- > 0;) {
        const uint32_t cat = code[i] & 7u;
        const bool last = i + 1 == m;
        na[i] = cat != CAT_W ? 1 : ((code[i] & CC_CRLF) ? 0 : (last ? 1 : na[i + 1]));
        const bool low = cat == CAT_LL || cat == CAT_LO || cat == CAT_M;
        au[i] = cat == CAT_LU ? (last ? 1 : au[i + 1]) : (low ? 0 : 1);
    }
    ctx.assign(m, 0);
    for (uint64_t i = 0; i < m; ++i) {
        const uint32_t c = code[i], cat = c & 7u;
        const uint32_t nxc = i + 1 < m ? code[i + 1] : (uint32_t)CC_EOF;
        const bool naw = na[i] && cat == CAT_W && !(c & CC_CRLF);
        const uint32_t doc = (c & CC_DOC) ? 1u : 0u;
        if (family == FAMILY_DEEPSEEK) {
            ctx[i] = (self_code_ds(c) * 2u + doc) * DS_NNEXT + next_code_ds(nxc) + (naw ? 2u * DS_NNEXT : 0u);
        } else {
            ctx[i] = (self_code(c, false) * 2u + doc) * (2u * NNEXT) + 2u * next_code(nxc) + (naw ? 4u * NNEXT : 0u);
            if (family == FAMILY_O200K) ctx[i] += au[i + 1];
        }
    }
}

struct Scratch {
    uint8_t *bytes;
    uint64_t *offs, *oo;
    uint32_t *ids, *spans;
    void *ws;
    uint64_t ws_bytes;
};

uint64_t a256(uint64_t x) { return (x + 255) & ~255ull; }

int scratch_layout(const toktier_vocab *v, uint64_t total, void *base, uint64_t bytes, Scratch *sc, uint64_t *need)
{
    uint64_t ws = 0;
    int rc = toktier_workspace_bytes_ex(v, total, 1, &ws);
    if (rc) return rc;
    const uint64_t cap = total ? total : 1;
    const uint64_t o_offs = a256(total + 1), o_oo = o_offs + 256, o_ids = o_oo + 256;
    const uint64_t o_spans = o_ids + a256(4 * cap), o_ws = o_spans + a256(4 * cap);
    *need = o_ws + ws;
    if (!sc) return TOKTIER_OK;
    if (!base || bytes < *need) return TOKTIER_E_INVALID_ARG;
    uint8_t *b = (uint8_t *)base;
    sc->bytes = b;
    sc->offs = (uint64_t *)(b + o_offs);
    sc->oo = (uint64_t *)(b + o_oo);
    sc->ids = (uint32_t *)(b + o_ids);
    sc->spans = (uint32_t *)(b + o_spans);
    sc->ws = b + o_ws;
    sc->ws_bytes = ws;
    return TOKTIER_OK;
}

// Encode text[a, b) as one document on the GPU; records (ID, byte offset relative to a) to the host.
int encode_range(const toktier_vocab *v, const uint8_t *text, uint64_t a, uint64_t b, const Scratch &sc,
                 hipStream_t st, std::vector<uint32_t> &ids, std::vector<uint32_t> &spans)
{
    const uint64_t m = b - a;
    const uint64_t offs[2] = {0, m};
    if (m && hipMemcpyAsync(sc.bytes, text + a, m, hipMemcpyHostToDevice, st) != hipSuccess) return TOKTIER_E_HIP;
    if (hipMemcpyAsync(sc.offs, offs, sizeof(offs), hipMemcpyHostToDevice, st) != hipSuccess) return TOKTIER_E_HIP;
    uint64_t nt = 0;
    int rc = toktier_encode_batch_spans(v, sc.bytes, sc.offs, 1, m, sc.ids, m ? sc.spans : nullptr, m ? m : 1, sc.oo,
                                        sc.ws, sc.ws_bytes, st, &nt);
    if (rc) return rc;
    ids.resize(nt);
    spans.resize(nt);
    if (nt && (hipMemcpyAsync(ids.data(), sc.ids, 4 * nt, hipMemcpyDeviceToHost, st) != hipSuccess ||
               hipMemcpyAsync(spans.data(), sc.spans, 4 * nt, hipMemcpyDeviceToHost, st) != hipSuccess))
        return TOKTIER_E_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return TOKTIER_E_HIP;
    return TOKTIER_OK;
}

}  // namespace

extern "C" int toktier_repair_scratch_bytes(const toktier_vocab *v, uint64_t total_bytes, uint64_t *out_bytes)
{
    if (!v || !out_bytes) return TOKTIER_E_INVALID_ARG;
    return scratch_layout(v, total_bytes, nullptr, 0, nullptr, out_bytes);
}

extern "C" int toktier_repair_append(const toktier_vocab *v, const uint8_t *text, uint64_t len_a, uint64_t len_total,
                                     const uint32_t *cached_ids, const uint32_t *cached_spans, uint64_t n_cached,
                                     uint32_t *out_ids, uint32_t *out_spans, uint64_t capacity, uint64_t *out_n,
                                     void *scratch, uint64_t scratch_bytes, void *stream, toktier_repair_info *info)
{
    if (!v || !out_n || len_a > len_total || (len_total && !text) || (n_cached && (!cached_ids || !cached_spans)))
        return TOKTIER_E_INVALID_ARG;
    if (v->da.n) return TOKTIER_E_INVALID_ARG;   // added tokens: the literal pass is not repaired
    if (len_total >= 0xFFFFFFFFull) return TOKTIER_E_INVALID_ARG;
    if (capacity < len_total || (len_total && (!out_ids || !out_spans))) return TOKTIER_E_CAPACITY;
    if (n_cached > len_a || (n_cached && cached_spans[0] != 0) || (len_a && !n_cached)) return TOKTIER_E_INVALID_ARG;
    if (n_cached && cached_spans[n_cached - 1] >= len_a) return TOKTIER_E_INVALID_ARG;
    // the records are repaired in place when the output arrays are the cached ones; otherwise no
    // output array may overlap an input array or the other output array
    const bool in_place = n_cached && out_ids == cached_ids && out_spans == cached_spans;
    {
        auto apart = [](const void *a, uint64_t na_, const void *b, uint64_t nb_) {
            const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
            return !na_ || !nb_ || x + na_ <= y || y + nb_ <= x;
        };
        const uint64_t oc = len_total ? 4 * capacity : 0, cc = 4 * n_cached;
        if (!apart(out_ids, oc, out_spans, oc)) return TOKTIER_E_INVALID_ARG;
        if (!in_place && (!apart(out_ids, oc, cached_ids, cc) || !apart(out_ids, oc, cached_spans, cc) ||
                          !apart(out_spans, oc, cached_ids, cc) || !apart(out_spans, oc, cached_spans, cc)))
            return TOKTIER_E_INVALID_ARG;
    }
    if (len_a < len_total && (text[len_a] & 0xC0u) == 0x80u) return TOKTIER_E_INVALID_UTF8;   // A ends inside a character
    Scratch sc;
    uint64_t need = 0;
    int rc = scratch_layout(v, len_total, scratch, scratch_bytes, &sc, &need);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    toktier_repair_info inf;
    memset(&inf, 0, sizeof(inf));
    const int fam = v->family;

    // Each attempt reads only its window: A's last w characters and B, decoded and checked here, with
    // character indices counted from the window's first character (the pages price a repair at
    // O(append + window), whatever the length of A).  The rest of A is read only by the full-text
    // encode after every window missed, and the cached records only from the window's start on.
    std::vector<uint64_t> pos;
    std::vector<uint32_t> cps;
    std::vector<uint32_t> wids, wspans, ctxw;
    for (uint32_t att = 0; att <= REPAIR_DOUBLINGS; ++att) {
        const uint64_t w = (uint64_t)REPAIR_W0 << att;
        // byte offset of A's w-th character from its end; A must hold more than w characters
        uint64_t bs = len_a, found = 0;
        while (bs > 0 && found < w) {
            --bs;
            if ((text[bs] & 0xC0u) != 0x80u) ++found;
        }
        if (found < w || bs == 0) break;   // the window would hold all of A
        if (!decode(text + bs, len_total - bs, pos, cps)) return TOKTIER_E_INVALID_UTF8;
        const uint64_t nc = cps.size();
        const uint64_t na = (uint64_t)(std::lower_bound(pos.begin(), pos.end(), len_a - bs) - pos.begin());
        if (pos[na] != len_a - bs) return TOKTIER_E_INVALID_UTF8;
        // (L): the first character whose context may differ between A alone and A || B (0 when the
        // run that decides it reaches the window's start: then no splice point qualifies)
        uint64_t dl = na - 2;
        {
            uint64_t k = na;
            while (k > 0 && (ucat_host(cps[k - 1]) & 7u) == CAT_W && cps[k - 1] != '\r' && cps[k - 1] != '\n') --k;
            dl = std::min(dl, k ? k - 1 : 0);
            if (fam == FAMILY_O200K) {
                k = na;
                while (k > 0 && (ucat_host(cps[k - 1]) & 7u) == CAT_LU) --k;
                dl = std::min(dl, k ? k - 1 : 0);
            }
        }
        inf.attempts = att + 1;
        inf.window_chars = (uint32_t)w;
        rc = encode_range(v, text, bs, len_total, sc, st, wids, wspans);
        if (rc) return rc;
        // window contexts (a document from its first character) and piece starts
        contexts(fam, text + bs, len_total - bs, pos, cps, 0, true, ctxw);
        std::vector<uint8_t> wstart(nc, 0);
        uint32_t state = S_ST;
        for (uint64_t i = 0; i < nc; ++i) {
            const uint8_t c = v->hmap[ctxw[i]][state];
            wstart[i] = (c >> 4) & 1u;
            state = c & 15u;
        }
        // (R): the first character after which the maps of the window's characters 1.. send every
        // state to one
        uint64_t sync = UINT64_MAX;
        {
            uint8_t img[NSTATES];
            for (int q = 0; q < NSTATES; ++q) img[q] = (uint8_t)q;
            for (uint64_t k = 1; k < na; ++k) {
                bool same = true;
                for (int q = 0; q < NSTATES; ++q) {
                    img[q] = v->hmap[ctxw[k]][img[q]] & 15u;
                    same &= img[q] == img[0];
                }
                if (same) { sync = k; break; }
            }
        }
        // the longest run of records equal in position and ID, among cached records at or after the
        // window start and window records that start inside A
        const uint64_t i0 = (uint64_t)(std::lower_bound(cached_spans, cached_spans + n_cached, (uint32_t)bs) -
                                       cached_spans);
        for (uint64_t t = i0 ? i0 : 1; t < n_cached; ++t)   // the records read below must increase
            if (cached_spans[t] <= cached_spans[t - 1]) return TOKTIER_E_INVALID_ARG;
        uint64_t i = i0, j = 0, best_len = 0, best_i = 0, cur_len = 0, cur_i = 0;
        while (i < n_cached && j < wids.size()) {
            const uint64_t pc = cached_spans[i], pw = bs + wspans[j];
            if (pw >= len_a) break;
            if (pc == pw) {
                if (cached_ids[i] == wids[j]) {
                    if (!cur_len) cur_i = i;
                    ++cur_len;
                    if (cur_len > best_len) { best_len = cur_len; best_i = cur_i; }
                } else {
                    cur_len = 0;
                }
                ++i;
                ++j;
            } else {
                cur_len = 0;
                if (pc < pw) ++i; else ++j;
            }
        }
        if (best_len < 2) continue;
        const uint64_t run_a = cached_spans[best_i];
        const uint64_t last = best_i + best_len - 1;
        const uint64_t run_b = last + 1 < n_cached ? cached_spans[last + 1] : len_a;
        if (run_b - run_a <= v->dv.lmax) continue;
        // splice point: the last record boundary of the run that passes the certificate
        uint64_t e_byte = UINT64_MAX;
        for (uint64_t r1 = best_i + best_len + 1; r1 > best_i && e_byte == UINT64_MAX; --r1) {
            const uint64_t r = r1 - 1;                                     // boundary before record r
            const uint64_t b = (r < n_cached ? cached_spans[r] : len_a) - bs;
            const uint64_t k = (uint64_t)(std::lower_bound(pos.begin(), pos.end(), b) - pos.begin());
            if (pos[k] != b || k >= nc) continue;                          // inside a character
            if (sync == UINT64_MAX || k <= sync || k >= dl) continue;
            if (!wstart[k]) continue;
            e_byte = bs + b;
        }
        if (e_byte == UINT64_MAX) continue;
        // cached records before e, then the window's records from e
        const uint64_t nl = (uint64_t)(std::lower_bound(cached_spans + i0, cached_spans + n_cached, (uint32_t)e_byte) -
                                       cached_spans);
        uint64_t jr = 0;
        while (jr < wids.size() && bs + wspans[jr] < e_byte) ++jr;
        const uint64_t total = nl + (wids.size() - jr);
        if (total > capacity) return TOKTIER_E_CAPACITY;
        if (!in_place) {
            memcpy(out_ids, cached_ids, 4 * nl);
            memcpy(out_spans, cached_spans, 4 * nl);
        }
        for (uint64_t t = jr; t < wids.size(); ++t) {
            out_ids[nl + t - jr] = wids[t];
            out_spans[nl + t - jr] = (uint32_t)(bs + wspans[t]);
        }
        inf.spliced = 1;
        inf.splice_byte = e_byte;
        inf.fresh_tokens = wids.size() - jr;
        *out_n = total;
        if (info) *info = inf;
        return TOKTIER_OK;
    }
    // every window missed (or A is shorter than the first window): the whole text
    rc = encode_range(v, text, 0, len_total, sc, st, wids, wspans);
    if (rc) return rc;
    if (wids.size() > capacity) return TOKTIER_E_CAPACITY;
    if (!wids.empty()) {
        memcpy(out_ids, wids.data(), 4 * wids.size());
        memcpy(out_spans, wspans.data(), 4 * wspans.size());
    }
    inf.spliced = 0;
    inf.fresh_tokens = wids.size();
    *out_n = wids.size();
    if (info) *info = inf;
    return TOKTIER_OK;
}
