// toktier.hip -- host side of the C ABI (include/toktier.h): vocabulary load and validation,
// device tables, argument checks and the stream-ordered launch chain.
#include <stdio.h>
#include <stdlib.h>
#include <stddef.h>
#include <string.h>

#include <string>
#include <vector>
#include <algorithm>
#include <mutex>
#include <array>

#include "../../include/toktier.h"
#include "internal.h"

static_assert(tt::FAMILY_GPT2 == TOKTIER_GPT2 && tt::FAMILY_O200K == TOKTIER_O200K &&
              tt::FAMILY_DEEPSEEK == TOKTIER_DEEPSEEK, "family codes");
#include "unicode_table.inc"
#include "vocab.h"

using namespace tt;


static thread_local std::string g_hip_err;

static int hip_fail(hipError_t e)
{
    g_hip_err = hipGetErrorString(e);
    (void)hipGetLastError();   // clear the sticky error
    return TOKTIER_E_HIP;
}

#define HIP_TRY(x)                                 \
    do {                                           \
        hipError_t e_ = (x);                       \
        if (e_ != hipSuccess) return hip_fail(e_); \
    } while (0)

// ---------------------------------------------------------------------------------------------
// Library-owned scratch of toktier_encode_batch_static: one fixed array per device, used in place of
// a caller workspace by callers that cannot allocate.  In host code `scratch` is only a handle for
// the runtime; its device address on each device comes from hipGetSymbolAddress (taken once per
// device, with that device current, when the first vocabulary is loaded there) and only that
// address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[TOKTIER_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device; NULL until set up

// Called with device `dev` current.  Idempotent.
int setup_static_scratch(int dev)
{
    if (dev < 0 || dev >= MAX_DEVICES) return TOKTIER_E_INVALID_ARG;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (g_scratch_ptr[dev]) return TOKTIER_OK;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr || ((uintptr_t)ptr & 255u)) return TOKTIER_E_HIP;
    g_scratch_ptr[dev] = ptr;
    return TOKTIER_OK;
}

void *static_scratch(int dev)
{
    if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    return g_scratch_ptr[dev];
}
}  // namespace

// ---------------------------------------------------------------------------------------------
// pre-tokenizer automaton tables.
//
// The per-character rule of each family (paper, derivation paragraph: one run rule per regex
// alternative) as a deterministic automaton over character contexts.  A context is: the
// character's own code (13 kinds), whether it is the first character of a document, the kind of the
// next character (6, incl. end of text) and one backward flag.  For each context and each state
// the table gives the next state and whether a piece starts at the character.  The state before a
// character is what the running leftmost-first match expects there; at a match start the first
// alternative that can match (in the family's order) decides the new state.

namespace {

enum Self { SF_LU = 0, SF_LL, SF_LO, SF_N, SF_M, SF_O, SF_AP2, SF_AP3, SF_W0, SF_W1, SF_SP0, SF_SP1,
            SF_CRLF };
enum Next { NX_L = 0, NX_N, NX_W, NX_M, NX_O, NX_EOF };
constexpr int STOP = -1;

struct Ctx {
    int self, nx;
    bool allu;   // only uppercase letters from the next character to the end of its letter run
    bool L() const { return self <= SF_LO; }
    bool N() const { return self == SF_N; }
    bool M() const { return self == SF_M; }
    bool Oany() const { return self >= SF_M && self <= SF_AP3; }      // [^\s\p{L}\p{N}]
    bool Oprime() const { return self >= SF_O && self <= SF_AP3; }    // other, not a mark
    bool W() const { return self >= SF_W0; }
    bool SP() const { return self == SF_SP0 || self == SF_SP1; }
    bool CRLF() const { return self == SF_CRLF; }
    bool NA() const { return self == SF_W1 || self == SF_SP1; }       // no CR/LF ahead in the run
    bool X() const { return !CRLF() && !L() && !N(); }                // [^\r\n\p{L}\p{N}]
    bool LM() const { return L() || M(); }
    int contr() const { return self == SF_AP2 ? 2 : (self == SF_AP3 ? 3 : 0); }
    bool nxL() const { return nx == NX_L; }
    bool nxLM() const { return nx == NX_L || nx == NX_M; }
    bool nxOany() const { return nx == NX_M || nx == NX_O; }
    bool nxW_or_eof() const { return nx == NX_W || nx == NX_EOF; }
};

int contraction_state(int len) { return len == 2 ? S_C1 : S_C2; }

// whitespace alternatives shared by cl100k and o200k: \s*[\r\n]+ | \s+(?!\S) | \s+
int ws_dispatch(const Ctx &c)
{
    if (!c.NA()) return S_WNL;           // a CR/LF lies ahead in this run (or is this char)
    return c.nxW_or_eof() ? S_WNS : S_ST;
}

// o200k letter phases: A = upper|other-letter|mark run, B = lower|other-letter|mark run
int letter_step(const Ctx &c)
{
    if (c.self == SF_LL) return S_LB;
    if (c.self == SF_LO || c.self == SF_M) return c.allu ? S_LEND : S_LA;
    return S_LA;   // uppercase
}

int dispatch(int fam, const Ctx &c)
{
    if (fam == TOKTIER_GPT2) {
        if (c.contr()) return contraction_state(c.contr());
        if (c.SP() && c.nxL()) return S_LRUN;
        if (c.SP() && c.nx == NX_N) return S_NALL;
        if (c.SP() && c.nxOany()) return S_ORUN;
        if (c.L()) return S_LRUN;
        if (c.N()) return S_NALL;
        if (c.Oany()) return S_ORUN;
        return c.nxW_or_eof() ? S_WNS : S_ST;
    }
    if (fam == TOKTIER_CL100K) {
        if (c.contr()) return contraction_state(c.contr());
        if (c.X() && c.nxL()) return S_LRUN;
        if (c.L()) return S_LRUN;
        if (c.N()) return S_N1;
        if (c.SP() && c.nxOany()) return S_ORNL;
        if (c.Oany()) return S_ORNL;
        return ws_dispatch(c);
    }
    // o200k
    if (c.LM()) return letter_step(c);
    if (c.X() && c.nxLM()) return S_LA;
    if (c.N()) return S_N1;
    if (c.SP() && c.nx == NX_O) return S_ORNL;
    if (c.Oprime()) return S_ORNL;
    return ws_dispatch(c);
}

int cont(int fam, int st, const Ctx &c)
{
    switch (st) {
    case S_ST: return STOP;
    case S_C1: return S_ST;
    case S_C2: return S_C1;
    case S_LRUN: return c.L() ? S_LRUN : STOP;
    case S_NALL: return c.N() ? S_NALL : STOP;
    case S_N1: return c.N() ? S_N2 : STOP;
    case S_N2: return c.N() ? S_ST : STOP;
    case S_ORUN: return c.Oany() ? S_ORUN : STOP;
    case S_ORNL: return c.Oany() ? S_ORNL : (c.CRLF() ? S_ONL : STOP);
    case S_ONL: return c.CRLF() ? S_ONL : STOP;
    case S_WNL: return (c.W() && !c.NA()) ? S_WNL : STOP;
    case S_WNS: return (c.W() && c.nxW_or_eof()) ? S_WNS : STOP;
    case S_LA:
    case S_LB:
    case S_LEND:
        if (c.LM()) {
            if (st == S_LA) return letter_step(c);
            if (st == S_LB) return c.self == SF_LU ? STOP : S_LB;
            return STOP;
        }
        // the letter match ends at the end of its run: an optional contraction suffix follows
        if (c.contr()) return contraction_state(c.contr());
        return STOP;
    }
    (void)fam;
    return STOP;
}

// ---- DeepSeek style: three splitters in sequence (paper, derivation paragraph on the DeepSeek
// family: the composition is one per-character rule when every splitter re-splits each earlier
// piece and the unmatched stretches stay pieces).  Splitter 1 isolates digit groups of 1-3,
// splitter 2 runs of CJK ideographs and kana, splitter 3 applies the body alternatives
//   A  one ASCII punctuation / symbol character, then ASCII letters
//   B  one optional character that is not CR/LF, a letter, punctuation or a symbol, then letters
//      and marks
//   C  an optional space, punctuation / symbols, then any CR/LF
//   D-F  the whitespace alternatives of cl100k
// to each piece left by the first two, whose ends are the ends of the text for it.  Between
// characters i and i+1 the first two splitters cut where the document ends, where a digit meets a
// non-digit, and (between non-digits) where the CJK ranges begin or end: the character before such
// a cut sees "end of text" next, and its transition ends every match (state DS_ST).  Digit groups
// count in states DS_N1 and DS_N2.  Characters that no body alternative can start are passed over
// by the splitter and form a piece of their own (state DS_GAP), which ends where a match can start.

enum DsState { DS_ST = 0, DS_N1, DS_N2, DS_AL, DS_LM, DS_PSR, DS_PNL, DS_WNL, DS_WNS, DS_GAP, DS_NSTATES };
static_assert(DS_NSTATES <= NSTATES, "DeepSeek-style states fit the maps");

// self codes 0..15 and next codes 0..9 as defined by the pieces kernel (self_code_ds, next_code_ds)
struct DsCtx {
    int self, nx;   // nx: the next character as the body splitter sees it (9 = end of text)
    bool cut;       // the first two splitters cut after this character
    bool N() const { return self == 10; }
    bool LA() const { return self == 0; }
    bool LM() const { return self <= 4; }
    bool PSa() const { return self == 5; }
    bool PS() const { return self >= 5 && self <= 7; }
    bool X() const { return self == 8 || self == 9; }
    bool W() const { return self >= 11; }
    bool SP() const { return self == 13 || self == 14; }
    bool CRLF() const { return self == 15; }
    bool NA() const { return self == 12 || self == 14; }   // no CR/LF ahead in this whitespace run
    bool nxLA() const { return nx == 0; }
    bool nxLM() const { return nx <= 2; }
    bool nxPS() const { return nx == 3 || nx == 4; }
    bool nxW_or_eof() const { return nx == 5 || nx == 9; }
};

DsCtx ds_ctx(int self, int next)
{
    auto self_cjk = [](int x) { return x == 2 || x == 4 || x == 7 || x == 9; };
    auto next_cjk = [](int x) { return x == 2 || x == 4 || x == 7; };
    const bool sn = self == 10, nn = next == 8;
    const bool cut = next == 9 || sn != nn || (!sn && !nn && self_cjk(self) != next_cjk(next));
    return DsCtx{self, cut ? 9 : next, cut};
}

int ds_dispatch(const DsCtx &c)
{
    if (c.N()) return DS_N1;
    if (c.PSa() && c.nxLA()) return DS_AL;
    if (c.LM()) return DS_LM;
    if (((c.W() && !c.CRLF()) || c.X()) && c.nxLM()) return DS_LM;
    if (c.SP() && c.nxPS()) return DS_PSR;
    if (c.PS()) return DS_PSR;
    if (c.W()) {
        if (!c.NA()) return DS_WNL;
        return c.nxW_or_eof() ? DS_WNS : DS_ST;
    }
    return DS_GAP;
}

int ds_cont(int st, const DsCtx &c)
{
    switch (st) {
    case DS_N1: return c.N() ? DS_N2 : STOP;
    case DS_N2: return c.N() ? DS_ST : STOP;
    case DS_AL: return c.LA() ? DS_AL : STOP;
    case DS_LM: return c.LM() ? DS_LM : STOP;
    case DS_PSR: return c.PS() ? DS_PSR : (c.CRLF() ? DS_PNL : STOP);
    case DS_PNL: return c.CRLF() ? DS_PNL : STOP;
    case DS_WNL: return (c.W() && !c.NA()) ? DS_WNL : STOP;
    case DS_WNS: return (c.W() && c.nxW_or_eof()) ? DS_WNS : STOP;
    case DS_GAP: return ds_dispatch(c) == DS_GAP ? DS_GAP : STOP;
    default: return STOP;   // DS_ST and the unused states
    }
}

void build_tables_ds(uint64_t *fmap, uint32_t *fstart)
{
    for (int self = 0; self < DS_NSELF; ++self)
        for (int doc = 0; doc < 2; ++doc)
            for (int nx = 0; nx < DS_NNEXT; ++nx) {
                const DsCtx c = ds_ctx(self, nx);
                const int idx = (self * 2 + doc) * DS_NNEXT + nx;
                const int d = ds_dispatch(c);
                uint64_t m = 0;
                uint32_t st = 0;
                for (int s = 0; s < NSTATES; ++s) {
                    int r = doc ? STOP : ds_cont(s, c);
                    if (r == STOP) { r = d; st |= 1u << s; }
                    if (c.cut) r = DS_ST;
                    m |= (uint64_t)r << (4 * s);
                }
                fmap[idx] = m;
                fstart[idx] = st;
            }
}

void build_tables(int fam, uint64_t *fmap, uint32_t *fstart)
{
    if (fam == TOKTIER_DEEPSEEK) {
        build_tables_ds(fmap, fstart);
        return;
    }
    for (int self = 0; self < NSELF; ++self)
        for (int doc = 0; doc < 2; ++doc)
            for (int nx = 0; nx < NNEXT; ++nx)
                for (int au = 0; au < 2; ++au) {
                    Ctx c{self, nx, au != 0};
                    int idx = ((self * 2 + doc) * NNEXT + nx) * 2 + au;
                    int d = dispatch(fam, c);
                    uint64_t m = 0;
                    uint32_t st = 0;
                    for (int s = 0; s < NSTATES; ++s) {
                        int r = doc ? STOP : cont(fam, s, c);
                        if (r == STOP) { r = d; st |= 1u << s; }
                        m |= (uint64_t)r << (4 * s);
                    }
                    fmap[idx] = m;
                    fstart[idx] = st;
                }
}

// Two-choice cuckoo placement of n items into `cap` slots (candidate slots from ck_slots with `seed`):
// an item goes to a free candidate slot, else it takes one and the item there moves to its other
// candidate, and so on.  where[slot] = item + 1 (0: free).  False when an eviction chain runs too long
// (the caller retries with another seed, then a larger table).
template <typename Digest>
bool cuckoo_place(uint32_t n, uint32_t cap, uint64_t seed, Digest digest, std::vector<uint32_t> &where)
{
    where.assign(cap, 0);
    for (uint32_t it = 0; it < n; ++it) {
        uint32_t cur = it, i, j;
        ck_slots(digest(cur), seed, cap, i, j);
        uint32_t pos = where[i] == 0 ? i : (where[j] == 0 ? j : i);
        for (int kick = 0;; ++kick) {
            if (where[pos] == 0) {
                where[pos] = cur + 1;
                break;
            }
            if (kick >= 1000) return false;
            const uint32_t out = where[pos] - 1;
            where[pos] = cur + 1;
            cur = out;
            ck_slots(digest(cur), seed, cap, i, j);
            if (i == j) return false;
            pos = pos == i ? j : i;
        }
    }
    return true;
}

// a table of at most about 45 % load for n items, placed; returns its capacity and seed
template <typename Digest>
void cuckoo_build(uint32_t n, uint64_t salt, Digest digest, std::vector<uint32_t> &where, uint32_t &cap, uint64_t &seed)
{
    cap = (uint32_t)std::max<uint64_t>(64, (uint64_t)n * 20 / 9 + 1);
    for (uint32_t attempt = 1;; ++attempt) {
        seed = ck_mix(salt + 0x9E3779B97F4A7C15ull * attempt);
        if (cuckoo_place(n, cap, seed, digest, where)) return;
        if (attempt % 4 == 0) cap = (uint32_t)((uint64_t)cap * 9 / 8 + 1);
    }
}

// valid UTF-8 in the sense the pre-tokenizer checks: no overlong forms, surrogates or code points
// above U+10FFFF, no truncated or stray sequences
bool valid_utf8(const uint8_t *s, uint32_t n)
{
    for (uint32_t i = 0; i < n;) {
        const uint32_t c = s[i];
        uint32_t len = c < 0x80 ? 1 : (c >> 5) == 6 ? 2 : (c >> 4) == 14 ? 3 : (c >> 3) == 30 ? 4 : 0;
        if (!len || i + len > n) return false;
        uint32_t cp = len == 1 ? c : c & (0x7Fu >> len);
        for (uint32_t k = 1; k < len; ++k) {
            if ((s[i + k] & 0xC0) != 0x80) return false;
            cp = (cp << 6) | (s[i + k] & 0x3Fu);
        }
        static const uint32_t min_cp[5] = {0, 0, 0x80, 0x800, 0x10000};
        if (cp < min_cp[len] || cp > 0x10FFFF || (cp >= 0xD800 && cp <= 0xDFFF)) return false;
        i += len;
    }
    return true;
}

// the added-token tables: literals, IDs, the first-two-bytes map and lists (longest first), the
// one-byte literals
int build_added_tables(toktier_vocab *v, const uint8_t *bytes, const uint32_t *offs, const uint32_t *ids,
                       uint32_t n)
{
    const uint32_t total = offs[n];
    std::vector<uint32_t> pmap(2048, 0), pre(65537, 0), list, one(256, NO_LIT);
    std::vector<std::vector<uint32_t>> by2(65536);
    uint32_t lmin = ~0u, lmax = 0;
    for (uint32_t k = 0; k < n; ++k) {
        const uint32_t len = offs[k + 1] - offs[k];
        lmin = std::min(lmin, len);
        lmax = std::max(lmax, len);
        const uint8_t *s = bytes + offs[k];
        if (len == 1) { one[s[0]] = k; continue; }
        const uint32_t x = s[0] | ((uint32_t)s[1] << 8);
        by2[x].push_back(k);
        pmap[x >> 5] |= 1u << (x & 31);
    }
    for (uint32_t x = 0; x < 65536; ++x) {
        std::vector<uint32_t> &l = by2[x];
        std::sort(l.begin(), l.end(), [&](uint32_t a, uint32_t b) {
            const uint32_t la = offs[a + 1] - offs[a], lb = offs[b + 1] - offs[b];
            return la != lb ? la > lb : a < b;
        });
        pre[x] = (uint32_t)list.size();
        list.insert(list.end(), l.begin(), l.end());
    }
    pre[65536] = (uint32_t)list.size();
    const uint64_t o_bytes = 0, o_off = align256(total + 1), o_id = o_off + align256(4ull * (n + 1));
    const uint64_t o_pmap = o_id + align256(4ull * n), o_pre = o_pmap + align256(4ull * pmap.size());
    const uint64_t o_list = o_pre + align256(4ull * pre.size()), o_one = o_list + align256(4ull * list.size() + 4);
    const uint64_t size = o_one + align256(4ull * 256);
    void *d = nullptr;
    hipError_t e = hipMalloc(&d, size);
    if (e != hipSuccess) {
        hip_fail(e);
        return TOKTIER_E_OOM;
    }
    uint8_t *base = (uint8_t *)d;
    e = hipMemcpy(base + o_bytes, bytes, total, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_off, offs, 4ull * (n + 1), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_id, ids, 4ull * n, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_pmap, pmap.data(), 4ull * pmap.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_pre, pre.data(), 4ull * pre.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess && !list.empty())
        e = hipMemcpy(base + o_list, list.data(), 4ull * list.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_one, one.data(), 4ull * 256, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e);
    }
    v->dadded = d;
    v->da.bytes = base + o_bytes;
    v->da.off = (const uint32_t *)(base + o_off);
    v->da.id = (const uint32_t *)(base + o_id);
    v->da.pmap = (const uint32_t *)(base + o_pmap);
    v->da.pre = (const uint32_t *)(base + o_pre);
    v->da.list = (const uint32_t *)(base + o_list);
    v->da.one = (const uint32_t *)(base + o_one);
    v->da.n = n;
    v->da.lmin = lmin;
    v->da.lmax = lmax;
    return TOKTIER_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// whole-piece tables.  A piece whose bytes equal the bytes of token t encodes to [t] exactly when t
// is "self-reachable": BPE of t's own byte string ends in t.  That is decided here, once per
// vocabulary, by running the library's GPU BPE kernels over every token's byte string (2..32
// bytes) with the tables still empty; the tables then hold exactly those tokens.

namespace {

// byte string of every token: len[t], off[t] into tb
struct TokenStrings {
    std::vector<uint32_t> len, off;
    std::vector<uint8_t> tb;
};

int token_strings(const uint32_t *merges, uint32_t n_merges, TokenStrings &ts)
{
    const uint32_t ntok_all = 256 + n_merges;
    ts.len.resize(ntok_all);
    ts.off.resize(ntok_all + 1);
    uint64_t total = 0;
    for (uint32_t t = 0; t < ntok_all; ++t) {
        ts.len[t] = t < 256 ? 1u : ts.len[merges[2 * (t - 256)]] + ts.len[merges[2 * (t - 256) + 1]];
        ts.off[t] = (uint32_t)total;
        total += ts.len[t];
        if (total > 0xFFFFFFF0ull) return TOKTIER_E_BAD_MERGES;
    }
    ts.off[ntok_all] = (uint32_t)total;
    ts.tb.resize(total);
    for (uint32_t t = 0; t < ntok_all; ++t) {
        if (t < 256) { ts.tb[ts.off[t]] = (uint8_t)t; continue; }
        uint32_t a = merges[2 * (t - 256)], b = merges[2 * (t - 256) + 1];
        memcpy(&ts.tb[ts.off[t]], &ts.tb[ts.off[a]], ts.len[a]);
        memcpy(&ts.tb[ts.off[t] + ts.len[a]], &ts.tb[ts.off[b]], ts.len[b]);
    }
    return TOKTIER_OK;
}

// The token-string hash (every token, duplicates of one string included) and the strings, on the
// device.  Skipped (pointers stay NULL) when some token is longer than STR_LMAX bytes.
int build_string_table(toktier_vocab *v, const TokenStrings &ts)
{
    const uint32_t ntok_all = (uint32_t)ts.len.size();
    uint32_t lmax = 0;
    for (uint32_t t = 0; t < ntok_all; ++t) lmax = std::max(lmax, ts.len[t]);
    if (lmax > STR_LMAX) return TOKTIER_OK;
    uint32_t lc = 10;
    while ((1ull << lc) < 2ull * ntok_all) ++lc;
    const uint64_t cap = 1ull << lc;
    std::vector<uint32_t> tab(4 * cap, 0);
    for (uint32_t t = 0; t < ntok_all; ++t) {
        uint64_t h = 0;
        for (uint32_t k = 0; k < ts.len[t]; ++k) h = h * STR_P + ts.tb[ts.off[t] + k];
        const uint64_t key = str_key(h, ts.len[t]);
        uint64_t i = str_slot(key, 64 - lc);
        while (tab[4 * i + 3]) i = (i + 1) & (cap - 1);
        tab[4 * i] = (uint32_t)key;
        tab[4 * i + 1] = (uint32_t)(key >> 32);
        tab[4 * i + 2] = t;
        tab[4 * i + 3] = ts.len[t];
    }
    const uint64_t o_tab = 0, o_off = align256(16 * cap), o_bytes = o_off + align256(4ull * (ntok_all + 1));
    const uint64_t total = o_bytes + align256(ts.tb.size());
    void *d = nullptr;
    hipError_t e = hipMalloc(&d, total);
    if (e != hipSuccess) {
        hip_fail(e);
        return TOKTIER_E_OOM;
    }
    uint8_t *base = (uint8_t *)d;
    e = hipMemcpy(base + o_tab, tab.data(), 16 * cap, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_off, ts.off.data(), 4ull * (ntok_all + 1), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(base + o_bytes, ts.tb.data(), ts.tb.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e);
    }
    v->dstr = d;
    v->dv.str = (const uint4 *)(base + o_tab);
    v->dv.tok_off = (const uint32_t *)(base + o_off);
    v->dv.tok_bytes = base + o_bytes;
    v->dv.str_mask = (uint32_t)(cap - 1);
    v->dv.str_shift = 64 - lc;
    v->dv.lmax = lmax;
    return TOKTIER_OK;
}

int fill_whole_piece_tables(toktier_vocab *v, const TokenStrings &ts, const std::vector<uint32_t> &cand,
                            const std::vector<uint32_t> &pv);

int build_whole_piece_tables(toktier_vocab *v, const TokenStrings &ts)
{
    const uint32_t ntok_all = (uint32_t)ts.len.size();
    const std::vector<uint32_t> &len = ts.len, &off = ts.off;
    const std::vector<uint8_t> &tb = ts.tb;
    std::vector<uint32_t> cand, starts;
    std::vector<uint8_t> batch;
    for (uint32_t t = 256; t < ntok_all; ++t) {
        if (len[t] < 2 || len[t] > (uint32_t)TABLE_MAX) continue;
        cand.push_back(t);
        starts.push_back((uint32_t)batch.size());
        batch.insert(batch.end(), tb.begin() + off[t], tb.begin() + off[t] + len[t]);
    }
    if (cand.empty()) return TOKTIER_OK;
    const uint32_t npc = (uint32_t)cand.size();
    std::vector<uint32_t> pv(npc);
    if (v->dv.flags & VF_IGNORE_MERGES) {
        // every token string is its own piece's result: the smallest ID of each string
        std::vector<std::pair<std::string, uint32_t>> keyed;
        keyed.reserve(npc);
        for (uint32_t i = 0; i < npc; ++i)
            keyed.emplace_back(std::string((const char *)&tb[off[cand[i]]], len[cand[i]]), cand[i]);
        std::sort(keyed.begin(), keyed.end());
        std::vector<uint32_t> first(ntok_all, 0);
        for (size_t i = 0; i < keyed.size(); ++i)
            if (i == 0 || keyed[i].first != keyed[i - 1].first) first[keyed[i].second] = 1;
        for (uint32_t i = 0; i < npc; ++i) pv[i] = first[cand[i]] ? cand[i] : NO_PIECE;
        return fill_whole_piece_tables(v, ts, cand, pv);
    }
    starts.push_back((uint32_t)batch.size());
    const uint64_t N = batch.size();
    const Layout L = make_layout(N);
    uint8_t *dbytes = nullptr, *dws = nullptr;
    hipError_t e = hipMalloc((void **)&dbytes, N);
    if (e == hipSuccess) e = hipMalloc((void **)&dws, L.total);
    if (e == hipSuccess) e = hipMemcpy(dbytes, batch.data(), N, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(dws + L.ctrl, 0, sizeof(Ctrl));
    if (e == hipSuccess) e = hipMemset(dws + L.gdone, 0, 4ull * L.cap_giant);
    if (e == hipSuccess) e = hipMemcpy(dws + L.ctrl + offsetof(Ctrl, n_pieces), &npc, 4, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(dws + L.pstart, starts.data(), 4ull * starts.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess) {
        Batch b{dbytes, nullptr, 1, N, dws, L};
        e = launch_route(v->dv, b, 0, nullptr);
        if (e == hipSuccess) e = launch_giant_prep(v->dv, b, 0, nullptr);
        if (e == hipSuccess) e = launch_bpe(v->dv, b, 0, nullptr);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(0);
    if (e == hipSuccess) e = hipMemcpy(pv.data(), dws + L.pval, 4ull * npc, hipMemcpyDeviceToHost);
    if (dbytes) (void)hipFree(dbytes);
    if (dws) (void)hipFree(dws);
    if (e != hipSuccess) return hip_fail(e);
    return fill_whole_piece_tables(v, ts, cand, pv);
}

// the tables from the candidates whose result word pv[i] is the candidate itself
int fill_whole_piece_tables(toktier_vocab *v, const TokenStrings &ts, const std::vector<uint32_t> &cand,
                            const std::vector<uint32_t> &pv)
{
    const std::vector<uint32_t> &len = ts.len, &off = ts.off;
    const std::vector<uint8_t> &tb = ts.tb;
    const uint32_t npc = (uint32_t)cand.size();
    std::vector<uint32_t> short_t, long_t;
    for (uint32_t i = 0; i < npc; ++i) {
        if (pv[i] != cand[i]) continue;   // not self-reachable: BPE of its bytes is not [token]
        (len[cand[i]] <= WA_MAX ? short_t : long_t).push_back(cand[i]);
    }
    // two-choice cuckoo tables, under half full (both candidate slots are read in one round trip)
    std::vector<uint64_t> akeys(short_t.size());
    for (size_t i = 0; i < short_t.size(); ++i) {
        const uint32_t t = short_t[i];
        uint64_t key = (uint64_t)len[t] << 56;
        for (uint32_t k = 0; k < len[t]; ++k) key |= (uint64_t)tb[off[t] + k] << (8 * k);
        akeys[i] = key;
    }
    std::vector<std::array<uint64_t, 4>> bkeys(long_t.size());
    for (size_t i = 0; i < long_t.size(); ++i) {
        const uint32_t t = long_t[i];
        std::array<uint64_t, 4> k4 = {0, 0, 0, 0};
        for (uint32_t k = 0; k < len[t]; ++k) k4[k >> 3] |= (uint64_t)tb[off[t] + k] << (8 * (k & 7));
        bkeys[i] = k4;
    }
    std::vector<uint32_t> wa_where, wb_where;
    uint32_t ca = 0, cb = 0;
    uint64_t sa = 0, sb = 0;
    cuckoo_build((uint32_t)short_t.size(), 0x5A17ull, [&](uint32_t i) { return akeys[i]; }, wa_where, ca, sa);
    cuckoo_build((uint32_t)long_t.size(), 0xB16Bull,
                 [&](uint32_t i) { return wb_digest(bkeys[i][0], bkeys[i][1], bkeys[i][2], bkeys[i][3], len[long_t[i]]); },
                 wb_where, cb, sb);
    std::vector<uint32_t> wa(4ull * ca, 0), wb(12ull * cb, 0);
    for (uint32_t h = 0; h < ca; ++h) {
        if (!wa_where[h]) continue;
        const uint32_t i = wa_where[h] - 1;
        wa[4 * h] = (uint32_t)akeys[i];
        wa[4 * h + 1] = (uint32_t)(akeys[i] >> 32);
        wa[4 * h + 2] = short_t[i];
    }
    for (uint32_t h = 0; h < cb; ++h) {
        if (!wb_where[h]) continue;
        const uint32_t i = wb_where[h] - 1;
        for (int w = 0; w < 4; ++w) {
            wb[12ull * h + 2 * w] = (uint32_t)bkeys[i][w];
            wb[12ull * h + 2 * w + 1] = (uint32_t)(bkeys[i][w] >> 32);
        }
        wb[12ull * h + 8] = len[long_t[i]];
        wb[12ull * h + 9] = long_t[i];
    }
    // the hot sets: the short entries in ID order, each into a free way of its set
    std::vector<uint32_t> hot(4ull * HOT_SLOTS, 0);
    for (size_t i = 0; i < short_t.size(); ++i) {
        const uint32_t set = hot_set(akeys[i]);
        for (uint32_t w = 0; w < 2; ++w) {
            uint32_t *e = &hot[4ull * (2 * set + w)];
            if (e[0] | e[1]) continue;
            e[0] = (uint32_t)akeys[i];
            e[1] = (uint32_t)(akeys[i] >> 32);
            e[2] = short_t[i];
            break;
        }
    }
    void *d = nullptr;
    const uint64_t bytes_a = 16ull * ca, bytes_b = 48ull * cb, bytes_h = 16ull * HOT_SLOTS;
    hipError_t e = hipMalloc(&d, bytes_a + bytes_b + bytes_h);
    if (e != hipSuccess) {
        hip_fail(e);
        return TOKTIER_E_OOM;
    }
    e = hipMemcpy(d, wa.data(), bytes_a, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy((uint8_t *)d + bytes_a, wb.data(), bytes_b, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy((uint8_t *)d + bytes_a + bytes_b, hot.data(), bytes_h, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e);
    }
    v->dwords = d;
    v->dv.wa = (const uint4 *)d;
    v->dv.wb = (const uint4 *)((uint8_t *)d + bytes_a);
    v->dv.hot = (const uint4 *)((uint8_t *)d + bytes_a + bytes_b);
    v->dv.wa_cap = ca;
    v->dv.wseed = sa;
    v->dv.wb_cap = cb;
    v->dv.bseed = sb;
    return TOKTIER_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------

extern "C" const char *toktier_status_string(int status)
{
    switch (status) {
    case TOKTIER_OK: return "ok";
    case TOKTIER_E_INVALID_ARG: return "invalid argument";
    case TOKTIER_E_BAD_FAMILY: return "unknown pre-tokenizer family";
    case TOKTIER_E_BAD_MERGES: return "merge list is not rank-consistent, has duplicates or is too large";
    case TOKTIER_E_INVALID_UTF8: return "input is not valid UTF-8";
    case TOKTIER_E_CAPACITY: return "output or workspace capacity too small";
    case TOKTIER_E_HIP: return "HIP runtime error";
    case TOKTIER_E_OOM: return "out of memory";
    default: return "unknown status";
    }
}

extern "C" const char *toktier_last_hip_error(void) { return g_hip_err.c_str(); }

extern "C" const char *toktier_unicode_table_sha256(void) { return TT_UNICODE_TABLE_SHA256; }

extern "C" int toktier_load_vocab(const uint32_t *merges, uint32_t n_merges, int family, toktier_vocab **out)
{
    return toktier_load_vocab_ex(merges, n_merges, family, 0, nullptr, nullptr, nullptr, 0, out);
}

extern "C" int toktier_load_vocab_ex(const uint32_t *merges, uint32_t n_merges, int family, uint32_t flags,
                                     const uint8_t *added_bytes, const uint32_t *added_offsets,
                                     const uint32_t *added_ids, uint32_t n_added, toktier_vocab **out)
{
    if (!out || (n_merges && !merges)) return TOKTIER_E_INVALID_ARG;
    if ((flags & ~(uint32_t)TOKTIER_IGNORE_MERGES) || n_added > TOKTIER_MAX_ADDED) return TOKTIER_E_INVALID_ARG;
    if (n_added) {
        if (!added_bytes || !added_offsets || !added_ids || added_offsets[0] != 0) return TOKTIER_E_INVALID_ARG;
        std::vector<std::string> seen;
        for (uint32_t k = 0; k < n_added; ++k) {
            if (added_offsets[k + 1] <= added_offsets[k]) return TOKTIER_E_INVALID_ARG;
            const uint32_t len = added_offsets[k + 1] - added_offsets[k];
            if (len > TOKTIER_MAX_ADDED_BYTES || !valid_utf8(added_bytes + added_offsets[k], len))
                return TOKTIER_E_INVALID_ARG;
            seen.emplace_back((const char *)added_bytes + added_offsets[k], len);
        }
        std::sort(seen.begin(), seen.end());
        if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return TOKTIER_E_INVALID_ARG;
    }
    if (family != TOKTIER_GPT2 && family != TOKTIER_CL100K && family != TOKTIER_O200K && family != TOKTIER_DEEPSEEK)
        return TOKTIER_E_BAD_FAMILY;
    if (n_merges > TOKTIER_MAX_MERGES) return TOKTIER_E_BAD_MERGES;

    // operand flags of every token: bit 1 = the left operand of some merge, bit 0 = the right one
    std::vector<uint8_t> lr(256ull + n_merges, 0);
    for (uint32_t r = 0; r < n_merges; ++r) {
        const uint32_t a = merges[2 * r], b = merges[2 * r + 1];
        if (a >= 256u + r || b >= 256u + r) return TOKTIER_E_BAD_MERGES;   // rank-inconsistent
        lr[a] |= 2u;
        lr[b] |= 1u;
    }
    auto rkx = [&](uint32_t r) { return (r << 2) | lr[256u + r]; };
    std::vector<uint32_t> r2(65536, NO_RANK);
    uint32_t n_general = 0;
    for (uint32_t r = 0; r < n_merges; ++r) {
        uint32_t a = merges[2 * r], b = merges[2 * r + 1];
        if ((a | b) < 256u) {
            if (r2[(a << 8) | b] != NO_RANK) return TOKTIER_E_BAD_MERGES;   // duplicate pair
            r2[(a << 8) | b] = rkx(r);
        } else {
            ++n_general;
        }
    }
    // pair table: two-choice cuckoo, under half full (both candidate slots read in one round trip)
    std::vector<uint64_t> pkeys;
    pkeys.reserve(n_general);
    for (uint32_t r = 0; r < n_merges; ++r) {
        const uint32_t a = merges[2 * r], b = merges[2 * r + 1];
        if ((a | b) >= 256u) pkeys.push_back((((uint64_t)a << 21) | b) << 22 | rkx(r));
    }
    {
        std::vector<uint64_t> ks(pkeys.size());
        for (size_t i = 0; i < pkeys.size(); ++i) ks[i] = pkeys[i] >> 22;
        std::sort(ks.begin(), ks.end());
        if (std::adjacent_find(ks.begin(), ks.end()) != ks.end()) return TOKTIER_E_BAD_MERGES;   // duplicate pair
    }
    std::vector<uint32_t> pwhere;
    uint32_t pcap = 0;
    uint64_t pseed = 0;
    cuckoo_build((uint32_t)pkeys.size(), 0x7A1Bull, [&](uint32_t i) { return pkeys[i] >> 22; }, pwhere, pcap, pseed);
    const uint64_t cap = pcap;
    std::vector<uint64_t> slots(cap, EMPTY_SLOT);
    for (uint32_t h = 0; h < pcap; ++h)
        if (pwhere[h]) slots[h] = pkeys[pwhere[h] - 1];
    uint64_t fmap[NCTX_MAX] = {};
    uint32_t fstart[NCTX_MAX] = {};
    build_tables(family, fmap, fstart);
    uint8_t fmap16[NCTX_MAX][16];
    for (int c = 0; c < NCTX_MAX; ++c) {
        for (int st = 0; st < 16; ++st)
            fmap16[c][st] = st < NSTATES ? (uint8_t)(((fmap[c] >> (4 * st)) & 15u) | (((fstart[c] >> st) & 1u) << 4)) : 0;
    }

    // one device allocation: r2 | slots | merges | byte transition maps
    const uint64_t o_r2 = 0, o_slots = align256(65536 * 4), o_merges = o_slots + align256(cap * 8);
    const uint64_t o_fmap = o_merges + align256(8ull * n_merges + 8);
    const uint64_t total = o_fmap + align256(sizeof(fmap16));

    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    {
        const int rs = setup_static_scratch(dev);
        if (rs != TOKTIER_OK) return rs;
    }
    void *d = nullptr;
    hipError_t e = hipMalloc(&d, total);
    if (e != hipSuccess) {
        hip_fail(e);
        return TOKTIER_E_OOM;
    }
    uint8_t *base = (uint8_t *)d;
    hipError_t c1 = hipMemcpy(base + o_r2, r2.data(), 65536 * 4, hipMemcpyHostToDevice);
    hipError_t c2 = hipMemcpy(base + o_slots, slots.data(), cap * 8, hipMemcpyHostToDevice);
    hipError_t c3 = n_merges ? hipMemcpy(base + o_merges, merges, 8ull * n_merges, hipMemcpyHostToDevice)
                             : hipSuccess;
    hipError_t c4 = hipMemcpy(base + o_fmap, fmap16, sizeof(fmap16), hipMemcpyHostToDevice);
    for (hipError_t ci : {c1, c2, c3, c4})
        if (ci != hipSuccess) {
            (void)hipFree(d);
            return hip_fail(ci);
        }
    toktier_vocab *v = (toktier_vocab *)calloc(1, sizeof(toktier_vocab));
    if (!v) {
        (void)hipFree(d);
        return TOKTIER_E_OOM;
    }
    v->device = dev;
    v->family = family;
    memcpy(v->hmap, fmap16, sizeof(fmap16));
    v->n_merges = n_merges;
    v->dmem = d;
    v->dv.r2 = (const uint32_t *)(base + o_r2);
    v->dv.slots = (const uint64_t *)(base + o_slots);
    v->dv.merges = (const uint32_t *)(base + o_merges);
    v->dv.fmap16 = (const uint4 *)(base + o_fmap);
    v->dv.slot_cap = pcap;
    v->dv.pseed = pseed;
    v->dv.n_merges = n_merges;
    v->dv.family = family;
    v->dv.flags = (flags & TOKTIER_IGNORE_MERGES) ? VF_IGNORE_MERGES : 0u;
    v->dv.wa = nullptr;
    v->dv.wb = nullptr;
    v->dv.hot = nullptr;
    v->dv.str = nullptr;
    v->dv.tok_off = nullptr;
    v->dv.tok_bytes = nullptr;
    TokenStrings ts;
    int rc = token_strings(merges, n_merges, ts);
    if (rc == TOKTIER_OK) {
        hipError_t el = hipMalloc(&v->dlen, 4ull * ts.len.size());
        if (el == hipSuccess) el = hipMemcpy(v->dlen, ts.len.data(), 4ull * ts.len.size(), hipMemcpyHostToDevice);
        if (el != hipSuccess) rc = hip_fail(el);
        v->dv.tok_len = (const uint32_t *)v->dlen;
    }
    if (rc == TOKTIER_OK) rc = build_string_table(v, ts);
    // ignore_merges looks long pieces up in the token string hash, which needs tokens <= STR_LMAX bytes
    if (rc == TOKTIER_OK && (v->dv.flags & VF_IGNORE_MERGES) && !v->dv.str) rc = TOKTIER_E_INVALID_ARG;
    if (rc == TOKTIER_OK) rc = build_whole_piece_tables(v, ts);
    if (rc == TOKTIER_OK && n_added) rc = build_added_tables(v, added_bytes, added_offsets, added_ids, n_added);
    if (rc != TOKTIER_OK) {
        if (v->dadded) (void)hipFree(v->dadded);
        if (v->dwords) (void)hipFree(v->dwords);
        if (v->dstr) (void)hipFree(v->dstr);
        if (v->dlen) (void)hipFree(v->dlen);
        (void)hipFree(v->dmem);
        free(v);
        return rc;
    }
    *out = v;
    return TOKTIER_OK;
}

extern "C" int toktier_free_vocab(toktier_vocab *v)
{
    if (!v) return TOKTIER_OK;
    hipError_t e = hipDeviceSynchronize();
    hipError_t f = hipFree(v->dmem);
    for (void *extra : {v->dwords, v->dstr, v->dlen, v->dadded}) {
        if (!extra) continue;
        hipError_t g = hipFree(extra);
        if (f == hipSuccess) f = g;
    }
    free(v);
    if (e != hipSuccess) return hip_fail(e);
    if (f != hipSuccess) return hip_fail(f);
    return TOKTIER_OK;
}

extern "C" int toktier_vocab_info(const toktier_vocab *v, uint32_t *n_merges, int *family)
{
    if (!v) return TOKTIER_E_INVALID_ARG;
    if (n_merges) *n_merges = v->n_merges;
    if (family) *family = v->family;
    return TOKTIER_OK;
}

extern "C" int toktier_workspace_bytes(uint64_t total_bytes, uint32_t n_docs, uint64_t *out_bytes)
{
    if (!out_bytes || total_bytes >= 0xFFFFFFFFull || n_docs == 0xFFFFFFFFu) return TOKTIER_E_INVALID_ARG;
    *out_bytes = make_layout(total_bytes).total;
    return TOKTIER_OK;
}

extern "C" int toktier_workspace_bytes_ex(const toktier_vocab *v, uint64_t total_bytes, uint32_t n_docs,
                                          uint64_t *out_bytes)
{
    if (!v) return TOKTIER_E_INVALID_ARG;
    int rc = toktier_workspace_bytes(total_bytes, n_docs, out_bytes);
    if (rc || !v->da.n) return rc;
    *out_bytes = make_add_layout(*out_bytes, total_bytes, n_docs, v->da.lmin).total;
    return TOKTIER_OK;
}

namespace {

int check_batch(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets, uint32_t n_docs,
                uint64_t total_bytes, void *workspace, uint64_t workspace_bytes, Batch *b)
{
    if (!v || !offsets || !workspace || n_docs == 0 || n_docs == 0xFFFFFFFFu) return TOKTIER_E_INVALID_ARG;
    if (total_bytes >= 0xFFFFFFFFull || (total_bytes && !bytes)) return TOKTIER_E_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return TOKTIER_E_INVALID_ARG;
    Layout L = make_layout(total_bytes);
    if (workspace_bytes < L.total) return TOKTIER_E_CAPACITY;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev != v->device) return TOKTIER_E_INVALID_ARG;
    b->bytes = bytes;
    b->offsets = offsets;
    b->n_docs = n_docs;
    b->n = total_bytes;
    b->ws = (uint8_t *)workspace;
    b->L = L;
    return TOKTIER_OK;
}

// read the control block back (one device-to-host copy) and map device-detected errors
int read_ctrl(void *workspace, hipStream_t s, Ctrl *out)
{
    static thread_local Ctrl *pinned = nullptr;
    if (!pinned) {
        hipError_t e = hipHostMalloc((void **)&pinned, sizeof(Ctrl), hipHostMallocDefault);
        if (e != hipSuccess) {
            pinned = nullptr;
            return hip_fail(e);
        }
    }
    HIP_TRY(hipMemcpyAsync(pinned, workspace, sizeof(Ctrl), hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    *out = *pinned;
    if (out->status & ST_BAD_OFFSETS) return TOKTIER_E_INVALID_ARG;
    if (out->status & ST_BAD_UTF8) return TOKTIER_E_INVALID_UTF8;
    return TOKTIER_OK;
}

}  // namespace

namespace {

// the encode chain: pre-tokenizer (with the long-piece lists), seams and chunks of giant pieces, the
// tile encoder (with the short-piece lists), BPE of every listed piece, the output writer
hipError_t launch_chain(const DevVocab &v, const Batch &b, uint32_t *out_ids, uint64_t *out_offsets,
                        uint32_t *out_spans, hipStream_t s, const Events *ev)
{
    hipError_t e = launch_pretokenize(v, b, s, ev, false);   // (the tile encoder places the starts)
    if (e == hipSuccess) e = launch_tiles(v, b, s, ev);
    if (e == hipSuccess) e = launch_giant_prep(v, b, s, ev);
    if (e == hipSuccess) e = launch_bpe(v, b, s, ev);
    if (e == hipSuccess) e = launch_emit(v, b, out_ids, out_offsets, out_spans, s, ev);
    return e;
}

int encode_impl(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets, uint32_t n_docs,
                uint64_t total_bytes, uint32_t *out_ids, uint64_t ids_capacity, uint64_t *out_offsets,
                uint32_t *out_spans, void *workspace, uint64_t workspace_bytes, void *stream,
                uint64_t *out_n_tokens, const Events *ev)
{
    Batch b;
    int rc = check_batch(v, bytes, offsets, n_docs, total_bytes, workspace, workspace_bytes, &b);
    if (rc) return rc;
    if (!out_offsets || (total_bytes && !out_ids)) return TOKTIER_E_INVALID_ARG;
    if (ids_capacity < total_bytes) return TOKTIER_E_CAPACITY;
    hipStream_t s = (hipStream_t)stream;
    if (v->da.n && total_bytes) {
        // added tokens: literal pass, one read of the literal count, then the pipeline on the
        // documents cut at the literals and the final merge
        const AddLayout A = make_add_layout(b.L.total, total_bytes, n_docs, v->da.lmin);
        if (workspace_bytes < A.total) return TOKTIER_E_CAPACITY;
        HIP_TRY(launch_literals(v->da, b, A, s));
        LitCtrl lc;
        HIP_TRY(hipMemcpyAsync(&lc, b.ws + A.lctrl, sizeof(LitCtrl), hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        if (lc.status & ST_BAD_OFFSETS) return TOKTIER_E_INVALID_ARG;
        if (lc.n_lit) {
            if ((uint64_t)n_docs + 2ull * lc.n_lit >= 0xFFFFFFFFull || lc.n_lit > A.k_cap) return TOKTIER_E_CAPACITY;
            HIP_TRY(launch_literal_docs(b, A, lc.n_lit, s));
            Batch b2 = b;
            b2.offsets = (const uint64_t *)(b.ws + A.offs2);
            b2.n_docs = n_docs + 2 * lc.n_lit;
            HIP_TRY(launch_chain(v->dv, b2, (uint32_t *)(b.ws + A.ids2), (uint64_t *)(b.ws + A.oo2),
                                 out_spans ? (uint32_t *)(b.ws + A.spans2) : nullptr, s, ev));
            HIP_TRY(launch_literal_merge(v->da, b, A, lc.n_lit, out_ids, out_offsets, out_spans, s));
            if (!out_n_tokens) return TOKTIER_OK;
            Ctrl c;
            rc = read_ctrl(workspace, s, &c);
            if (rc) return rc;
            *out_n_tokens = c.n_tokens;
            return TOKTIER_OK;
        }
    }
    HIP_TRY(launch_chain(v->dv, b, out_ids, out_offsets, out_spans, s, ev));
    if (!out_n_tokens) return TOKTIER_OK;
    Ctrl c;
    rc = read_ctrl(workspace, s, &c);
    if (rc) return rc;
    *out_n_tokens = c.n_tokens;
    return TOKTIER_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// plans: the kernel chain of one encode captured once as a HIP graph for fixed buffers and sizes
// (paper, latency paragraph: device-resident counts and a CUDA graph take the host out of the
// chain).  The chain holds kernels only -- every counter and flag is cleared by its first kernel --
// so a replay recomputes everything from the input buffer's current contents.

struct toktier_plan {
    const toktier_vocab *v;
    void *workspace;
    hipGraph_t graph;
    hipGraphExec_t exec;
};

namespace {

// capture the chain of batch b as a graph, instantiate and upload it
int plan_capture(const toktier_vocab *v, const Batch &b, uint32_t *out_ids, uint64_t *out_offsets,
                 uint32_t *out_spans, void *workspace, void *stream, toktier_plan **out)
{
    hipStream_t s = (hipStream_t)stream;
    hipStream_t cap = nullptr;
    HIP_TRY(hipStreamCreateWithFlags(&cap, hipStreamNonBlocking));
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        hipError_t e1 = launch_chain(v->dv, b, out_ids, out_offsets, out_spans, cap, nullptr);
        e = hipStreamEndCapture(cap, &g);
        if (e == hipSuccess) e = e1;
    }
    hipGraphExec_t x = nullptr;
    if (e == hipSuccess) e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e == hipSuccess) e = hipGraphUpload(x, s);
    (void)hipStreamDestroy(cap);
    if (e != hipSuccess) {
        if (x) (void)hipGraphExecDestroy(x);
        if (g) (void)hipGraphDestroy(g);
        return hip_fail(e);
    }
    toktier_plan *p = (toktier_plan *)calloc(1, sizeof(toktier_plan));
    if (!p) {
        (void)hipGraphExecDestroy(x);
        (void)hipGraphDestroy(g);
        return TOKTIER_E_OOM;
    }
    p->v = v;
    p->workspace = workspace;
    p->graph = g;
    p->exec = x;
    *out = p;
    return TOKTIER_OK;
}

}  // namespace

extern "C" int toktier_plan_create(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                   uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids, uint64_t ids_capacity,
                                   uint64_t *out_offsets, uint32_t *out_spans, void *workspace,
                                   uint64_t workspace_bytes, void *stream, toktier_plan **out)
{
    if (!out) return TOKTIER_E_INVALID_ARG;
    *out = nullptr;
    Batch b;
    int rc = check_batch(v, bytes, offsets, n_docs, total_bytes, workspace, workspace_bytes, &b);
    if (rc) return rc;
    if (v->da.n) return TOKTIER_E_INVALID_ARG;   // the literal pass reads a count on the host
    if (!out_offsets || (total_bytes && !out_ids)) return TOKTIER_E_INVALID_ARG;
    if (ids_capacity < total_bytes) return TOKTIER_E_CAPACITY;
    return plan_capture(v, b, out_ids, out_offsets, out_spans, workspace, stream, out);
}

extern "C" int toktier_plan_create_bucket(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                          uint32_t max_docs, uint64_t max_bytes, const uint64_t *sizes,
                                          uint32_t *out_ids, uint64_t ids_capacity, uint64_t *out_offsets,
                                          uint32_t *out_spans, void *workspace, uint64_t workspace_bytes,
                                          void *stream, toktier_plan **out)
{
    if (!out) return TOKTIER_E_INVALID_ARG;
    *out = nullptr;
    if (!sizes || max_bytes == 0 || !out_ids) return TOKTIER_E_INVALID_ARG;
    Batch b;
    int rc = check_batch(v, bytes, offsets, max_docs, max_bytes, workspace, workspace_bytes, &b);
    if (rc) return rc;
    if (v->da.n) return TOKTIER_E_INVALID_ARG;   // the literal pass reads a count on the host
    if (!out_offsets) return TOKTIER_E_INVALID_ARG;
    if (ids_capacity < max_bytes) return TOKTIER_E_CAPACITY;
    b.L.dsz = sizes;
    b.L.cap_n = max_bytes;
    b.L.cap_docs = max_docs;
    return plan_capture(v, b, out_ids, out_offsets, out_spans, workspace, stream, out);
}

extern "C" int toktier_plan_launch(toktier_plan *p, void *stream, uint64_t *out_n_tokens)
{
    if (!p) return TOKTIER_E_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(hipGraphLaunch(p->exec, s));
    if (!out_n_tokens) return TOKTIER_OK;
    Ctrl c;
    int rc = read_ctrl(p->workspace, s, &c);
    if (rc) return rc;
    *out_n_tokens = c.n_tokens;
    return TOKTIER_OK;
}

extern "C" int toktier_plan_free(toktier_plan *p)
{
    if (!p) return TOKTIER_OK;
    hipError_t e1 = hipGraphExecDestroy(p->exec), e2 = hipGraphDestroy(p->graph);
    free(p);
    if (e1 != hipSuccess) return hip_fail(e1);
    if (e2 != hipSuccess) return hip_fail(e2);
    return TOKTIER_OK;
}

extern "C" int toktier_encode_batch(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                    uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                                    uint64_t ids_capacity, uint64_t *out_offsets, void *workspace,
                                    uint64_t workspace_bytes, void *stream, uint64_t *out_n_tokens)
{
    return encode_impl(v, bytes, offsets, n_docs, total_bytes, out_ids, ids_capacity, out_offsets, nullptr,
                       workspace, workspace_bytes, stream, out_n_tokens, nullptr);
}

// The encode chain on the library-owned scratch of the current device (for callers that cannot
// allocate): no allocation of any kind, the same kernels as toktier_encode_batch.
extern "C" int toktier_encode_batch_static(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                           uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                                           uint64_t ids_capacity, uint64_t *out_offsets, void *stream,
                                           uint64_t *out_n_tokens)
{
    if (!v || v->da.n) return TOKTIER_E_INVALID_ARG;   // added tokens read a count on the host
    uint64_t need = 0;
    int rc = toktier_workspace_bytes(total_bytes, n_docs, &need);
    if (rc) return rc;
    if (need > (uint64_t)TOKTIER_STATIC_SCRATCH_BYTES) return TOKTIER_E_CAPACITY;
    void *ws = static_scratch(v->device);
    if (!ws) return TOKTIER_E_HIP;   // set up when the vocabulary was loaded on its device
    Batch b;
    rc = check_batch(v, bytes, offsets, n_docs, total_bytes, ws, TOKTIER_STATIC_SCRATCH_BYTES, &b);
    if (rc) return rc;
    if (!out_offsets || (total_bytes && !out_ids)) return TOKTIER_E_INVALID_ARG;
    if (ids_capacity < total_bytes) return TOKTIER_E_CAPACITY;
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(launch_chain(v->dv, b, out_ids, out_offsets, nullptr, s, nullptr));
    if (!out_n_tokens) return TOKTIER_OK;
    Ctrl c;   // one blocking copy of the control block into this frame
    HIP_TRY(hipMemcpyAsync(&c, ws, sizeof(Ctrl), hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    if (c.status & ST_BAD_OFFSETS) return TOKTIER_E_INVALID_ARG;
    if (c.status & ST_BAD_UTF8) return TOKTIER_E_INVALID_UTF8;
    *out_n_tokens = c.n_tokens;
    return TOKTIER_OK;
}

extern "C" int toktier_encode_batch_spans(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                          uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                                          uint32_t *out_spans, uint64_t ids_capacity, uint64_t *out_offsets,
                                          void *workspace, uint64_t workspace_bytes, void *stream,
                                          uint64_t *out_n_tokens)
{
    if (total_bytes && !out_spans) return TOKTIER_E_INVALID_ARG;
    return encode_impl(v, bytes, offsets, n_docs, total_bytes, out_ids, ids_capacity, out_offsets, out_spans,
                       workspace, workspace_bytes, stream, out_n_tokens, nullptr);
}

extern "C" int toktier_encode_batch_timed(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                          uint32_t n_docs, uint64_t total_bytes, uint32_t *out_ids,
                                          uint64_t ids_capacity, uint64_t *out_offsets, void *workspace,
                                          uint64_t workspace_bytes, void *stream, uint64_t *out_n_tokens,
                                          void *const *events_before, void *const *events_after)
{
    Events ev{events_before, events_after};
    return encode_impl(v, bytes, offsets, n_docs, total_bytes, out_ids, ids_capacity, out_offsets, nullptr,
                       workspace, workspace_bytes, stream, out_n_tokens, &ev);
}

extern "C" int toktier_pretokenize_batch(const toktier_vocab *v, const uint8_t *bytes, const uint64_t *offsets,
                                         uint32_t n_docs, uint64_t total_bytes, uint32_t *out_piece_starts,
                                         uint64_t starts_capacity, void *workspace, uint64_t workspace_bytes,
                                         void *stream, uint64_t *out_n_pieces)
{
    Batch b;
    int rc = check_batch(v, bytes, offsets, n_docs, total_bytes, workspace, workspace_bytes, &b);
    if (rc) return rc;
    if (!out_piece_starts || !out_n_pieces) return TOKTIER_E_INVALID_ARG;
    if (starts_capacity < total_bytes + 1) return TOKTIER_E_CAPACITY;
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(launch_pretokenize(v->dv, b, s, nullptr, true));
    HIP_TRY(launch_export_starts(b, out_piece_starts, s));
    Ctrl c;
    rc = read_ctrl(workspace, s, &c);
    if (rc) return rc;
    *out_n_pieces = c.n_pieces;
    return TOKTIER_OK;
}

extern "C" int toktier_last_status(void *workspace, void *stream, uint64_t *out_n_tokens)
{
    if (!workspace) return TOKTIER_E_INVALID_ARG;
    Ctrl c;
    int rc = read_ctrl(workspace, (hipStream_t)stream, &c);
    if (rc) return rc;
    if (out_n_tokens) *out_n_tokens = c.n_tokens;
    return TOKTIER_OK;
}
