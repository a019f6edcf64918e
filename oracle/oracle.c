/*
 * oracle.c -- plain, serial CPU reference for exact byte-level BPE tokenization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU path must compute; it is linked only by
 * the tests, the smoke check and the benchmark's CPU-baseline leg.  It shares no code, table or
 * header with the GPU library.
 *
 * What it computes (TokTier, arXiv 2607.29678; "background" section and the summary page's §2.2
 * equation F = E* o G):  for each document, G splits the text into pieces with a leftmost-first
 * alternation regex, E encodes each piece independently with byte-level BPE, and the document's IDs
 * are the concatenation of the pieces' IDs.
 *
 *  G  (paper, GPU pre-tokenization paragraph: "leftmost-first alternation regex with backtracking";
 *     each match begins where the previous one ended).  Implemented here without a regex engine: one
 *     hand-written matcher per alternative, tried in the family's order at each match start; each
 *     matcher returns the end that a backtracking engine with greedy quantifiers would report.
 *  E  (paper, GPU BPE paragraph; summary page §2.3): the textbook loop -- repeatedly merge the
 *     leftmost adjacent pair of lowest rank -- run with a priority queue keyed (rank, position)
 *     over a linked list, with lazy invalidation of stale queue entries.
 *  T  The BPE trainer that produces the merge lists used as inputs (most frequent pair, ties to the
 *     smallest (left, right); merges creating a token longer than max_token_bytes are skipped).
 *
 * The rule families are this project's own wording of the GPT-2-, cl100k-, o200k- and
 * DeepSeek-style patterns the paper evaluates (paper, derivation paragraph: the cl100k and o200k
 * lineages, and the DeepSeek family's three splitters applied in sequence).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* character classes (table probed out of the `regex` engine by unicode_classes.py)            */

enum { C_LU = 1, C_LL = 2, C_LO = 3, C_N = 4, C_W = 5, C_M = 6, C_O = 7, C_PS = 8 };   /* PS: \p{P} or \p{S} */
static uint8_t *g_cls = NULL;

int orc_set_classes(const uint8_t *table, uint64_t n)
{
    if (n != 0x110000) return -1;
    if (!g_cls) g_cls = (uint8_t *)malloc(n);
    if (!g_cls) return -2;
    memcpy(g_cls, table, n);
    return 0;
}

static inline int klass(uint32_t c) { return g_cls[c]; }
static inline int is_L(uint32_t c) { int k = klass(c); return k == C_LU || k == C_LL || k == C_LO; }
static inline int is_N(uint32_t c) { return klass(c) == C_N; }
static inline int is_W(uint32_t c) { return klass(c) == C_W; }
/* [^\s\p{L}\p{N}] -- includes marks */
static inline int is_O(uint32_t c) { return !is_L(c) && !is_N(c) && !is_W(c); }
static inline int is_crlf(uint32_t c) { return c == '\r' || c == '\n'; }
/* [^\r\n\p{L}\p{N}] */
static inline int is_X(uint32_t c) { return !is_crlf(c) && !is_L(c) && !is_N(c); }
/* o200k-style letter sets: A = [\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}], B = [\p{Ll}\p{Lm}\p{Lo}\p{M}] */
static inline int is_A(uint32_t c) { int k = klass(c); return k == C_LU || k == C_LO || k == C_M; }
static inline int is_B(uint32_t c) { int k = klass(c); return k == C_LL || k == C_LO || k == C_M; }

/* DeepSeek-style sets */
static inline int is_PS(uint32_t c) { return klass(c) == C_PS; }
static inline int is_LM(uint32_t c) { return is_L(c) || klass(c) == C_M; }
static inline int is_ascii_alpha(uint32_t c) { return (c >= 'a' && c <= 'z') || (c >= 'A' && c <= 'Z'); }
/* the 32 ASCII punctuation and symbol characters: ! through /, : through @, [ through `, { through ~ */
static inline int is_ascii_punct(uint32_t c)
{
    return (c >= 0x21 && c <= 0x2F) || (c >= 0x3A && c <= 0x40) || (c >= 0x5B && c <= 0x60) || (c >= 0x7B && c <= 0x7E);
}
/* CJK unified ideographs U+4E00..U+9FA5, hiragana and katakana blocks U+3040..U+30FF */
static inline int is_cjk(uint32_t c) { return (c >= 0x4E00 && c <= 0x9FA5) || (c >= 0x3040 && c <= 0x30FF); }
/* [^\r\n\p{L}\p{P}\p{S}] */
static inline int is_ds_prefix(uint32_t c) { return !is_crlf(c) && !is_L(c) && !is_PS(c); }

/* ------------------------------------------------------------------------------------------ */
/* UTF-8 decode with validation (RFC 3629: no overlongs, no surrogates, nothing above U+10FFFF)  */

/* Decodes bytes [0,n) into code points; pos[k] = byte offset of char k, pos[nc] = n.
 * Returns the number of chars, or -1 if the bytes are not valid UTF-8. */
static int64_t utf8_decode(const uint8_t *s, uint64_t n, uint32_t *cp, uint64_t *pos)
{
    uint64_t i = 0;
    int64_t k = 0;
    while (i < n) {
        uint32_t b0 = s[i], c;
        int len;
        if (b0 < 0x80) { c = b0; len = 1; }
        else if (b0 >= 0xC2 && b0 <= 0xDF) { c = b0 & 0x1F; len = 2; }
        else if (b0 >= 0xE0 && b0 <= 0xEF) { c = b0 & 0x0F; len = 3; }
        else if (b0 >= 0xF0 && b0 <= 0xF4) { c = b0 & 0x07; len = 4; }
        else return -1;
        if (i + len > n) return -1;
        for (int j = 1; j < len; j++) {
            uint32_t b = s[i + j];
            if ((b & 0xC0) != 0x80) return -1;
            c = (c << 6) | (b & 0x3F);
        }
        if (len == 3 && c < 0x800) return -1;               /* overlong */
        if (len == 4 && (c < 0x10000 || c > 0x10FFFF)) return -1;
        if (c >= 0xD800 && c <= 0xDFFF) return -1;          /* surrogate */
        cp[k] = c;
        pos[k] = i;
        k++;
        i += len;
    }
    pos[k] = n;
    return k;
}

/* ------------------------------------------------------------------------------------------ */
/* matchers: each returns the end of the match starting at p, or -1 (no match)                  */

typedef struct { const uint32_t *c; int64_t n; } Doc;   /* one document, n chars; n is its EOF */

static int64_t run_end(const Doc *d, int64_t p, int (*pred)(uint32_t))
{
    while (p < d->n && pred(d->c[p])) p++;
    return p;
}

static int lower_eq(uint32_t c, char want) { return c == (uint32_t)want; }
static int ci_eq(uint32_t c, char want) { return c == (uint32_t)want || c == (uint32_t)(want - 32); }

/* 's|'t|'re|'ve|'m|'ll|'d at p, tried in that order; returns the match length or 0. */
static int contraction_len(const Doc *d, int64_t p, int (*eq)(uint32_t, char))
{
    static const char *alts[] = { "s", "t", "re", "ve", "m", "ll", "d" };
    if (p >= d->n || d->c[p] != '\'') return 0;
    for (int a = 0; a < 7; a++) {
        const char *t = alts[a];
        int64_t q = p + 1;
        int ok = 1;
        for (; *t; t++, q++)
            if (q >= d->n || !eq(d->c[q], *t)) { ok = 0; break; }
        if (ok) return (int)(q - p);
    }
    return 0;
}

/* ' ?' followed by 1+ chars of a class: the optional space is tried first (greedy). */
static int64_t sp_opt_run(const Doc *d, int64_t p, int (*pred)(uint32_t))
{
    if (d->c[p] == ' ' && p + 1 < d->n && pred(d->c[p + 1])) return run_end(d, p + 1, pred);
    if (pred(d->c[p])) return run_end(d, p, pred);
    return -1;
}

/* \s+(?!\S): greedy whitespace run, then give back chars until the next char is not \S. */
static int64_t ws_not_before_nonws(const Doc *d, int64_t p)
{
    if (!is_W(d->c[p])) return -1;
    int64_t e = run_end(d, p, is_W);
    for (int64_t k = e; k > p; k--)
        if (k == d->n || is_W(d->c[k])) return k;
    return -1;
}

/* \s+ */
static int64_t ws_all(const Doc *d, int64_t p)
{
    return is_W(d->c[p]) ? run_end(d, p, is_W) : -1;
}

/* \s*[\r\n]+ : \s* takes the whole run, then backs off until [\r\n]+ can match (greedily). */
static int64_t ws_to_last_newline(const Doc *d, int64_t p)
{
    int64_t e = run_end(d, p, is_W);
    for (int64_t k = e; k >= p; k--) {
        if (k < d->n && is_crlf(d->c[k])) {
            int64_t q = k;
            while (q < d->n && is_crlf(d->c[q])) q++;
            return q;
        }
    }
    return -1;
}

/* ' ?[^\s\p{L}\p{N}]+[\r\n]*' */
static int64_t sp_opt_other_newlines(const Doc *d, int64_t p)
{
    int64_t q = sp_opt_run(d, p, is_O);
    if (q < 0) return -1;
    while (q < d->n && is_crlf(d->c[q])) q++;
    return q;
}

/* \p{N}{1,3} */
static int64_t num_upto3(const Doc *d, int64_t p)
{
    int64_t q = p;
    while (q < d->n && q - p < 3 && is_N(d->c[q])) q++;
    return q > p ? q : -1;
}

/* ---- GPT-2 style ---- */
static int64_t g2_contraction(const Doc *d, int64_t p)
{
    int k = contraction_len(d, p, lower_eq);
    return k ? p + k : -1;
}
static int64_t g2_letters(const Doc *d, int64_t p) { return sp_opt_run(d, p, is_L); }
static int64_t g2_numbers(const Doc *d, int64_t p) { return sp_opt_run(d, p, is_N); }
static int64_t g2_other(const Doc *d, int64_t p) { return sp_opt_run(d, p, is_O); }

/* ---- cl100k style ---- */
static int64_t cl_contraction(const Doc *d, int64_t p)
{
    int k = contraction_len(d, p, ci_eq);
    return k ? p + k : -1;
}
/* [^\r\n\p{L}\p{N}]?\p{L}+ */
static int64_t cl_letters(const Doc *d, int64_t p)
{
    if (is_X(d->c[p]) && p + 1 < d->n && is_L(d->c[p + 1])) return run_end(d, p + 1, is_L);
    if (is_L(d->c[p])) return run_end(d, p, is_L);
    return -1;
}

/* ---- o200k style ---- */
/* X? then the word body, then an optional case-insensitive contraction.  The body for the first
 * alternative is A* B+ and for the second A+ B*; both quantifiers are greedy and backtrack. */
static int64_t ok_suffix(const Doc *d, int64_t q)
{
    return q + contraction_len(d, q, ci_eq);
}
static int64_t ok_word_lower(const Doc *d, int64_t p)       /* X? A* B+ C? */
{
    for (int take_x = 1; take_x >= 0; take_x--) {
        if (take_x && !is_X(d->c[p])) continue;
        int64_t q = p + take_x;
        int64_t aend = run_end(d, q, is_A);
        /* A* gives back chars one at a time until B+ can start */
        for (int64_t j = aend; j >= q; j--) {
            if (j < d->n && is_B(d->c[j])) return ok_suffix(d, run_end(d, j, is_B));
        }
    }
    return -1;
}
static int64_t ok_word_upper(const Doc *d, int64_t p)       /* X? A+ B* C? */
{
    for (int take_x = 1; take_x >= 0; take_x--) {
        if (take_x && !is_X(d->c[p])) continue;
        int64_t q = p + take_x;
        int64_t aend = run_end(d, q, is_A);
        if (aend == q) continue;
        return ok_suffix(d, run_end(d, aend, is_B));
    }
    return -1;
}

/* ---- DeepSeek style: three splitters applied one after the other ----
 * Stage 1 isolates digit groups (\p{N}{1,3}), stage 2 isolates runs of CJK ideographs and kana,
 * stage 3 splits with the body alternatives below.  Each stage re-splits every piece of the stage
 * before it on its own (the piece's ends are the text's ends for the stage's matcher), and the
 * characters between two matches of a stage form a piece too (paper, derivation paragraph on the
 * DeepSeek family: the splitters' composition is one per-character predicate provided every
 * splitter re-splits each earlier piece and unmatched spans survive as pieces). */

/* stage 2: [\u4E00-\u9FA5\u3040-\u30FF]+ */
static int64_t ds_cjk_run(const Doc *d, int64_t p) { return is_cjk(d->c[p]) ? run_end(d, p, is_cjk) : -1; }

/* stage 3, alternative 1: one ASCII punctuation or symbol character, then ASCII letters */
static int64_t ds_punct_word(const Doc *d, int64_t p)
{
    if (!is_ascii_punct(d->c[p]) || p + 1 >= d->n || !is_ascii_alpha(d->c[p + 1])) return -1;
    return run_end(d, p + 1, is_ascii_alpha);
}

/* alternative 2: [^\r\n\p{L}\p{P}\p{S}]?[\p{L}\p{M}]+ (the optional prefix is tried first) */
static int64_t ds_word(const Doc *d, int64_t p)
{
    if (is_ds_prefix(d->c[p]) && p + 1 < d->n && is_LM(d->c[p + 1])) return run_end(d, p + 1, is_LM);
    return is_LM(d->c[p]) ? run_end(d, p, is_LM) : -1;
}

/* alternative 3: ' ?[\p{P}\p{S}]+[\r\n]*' */
static int64_t ds_punct(const Doc *d, int64_t p)
{
    int64_t q = sp_opt_run(d, p, is_PS);
    if (q < 0) return -1;
    while (q < d->n && is_crlf(d->c[q])) q++;
    return q;
}

typedef int64_t (*alt_fn)(const Doc *, int64_t);

static const alt_fn DS_STAGE1[] = { num_upto3, NULL };
static const alt_fn DS_STAGE2[] = { ds_cjk_run, NULL };
static const alt_fn DS_STAGE3[] = { ds_punct_word, ds_word, ds_punct, ws_to_last_newline, ws_not_before_nonws,
                                    ws_all, NULL };

/* One splitter on chars [a, b) of doc: leftmost-first matching, each match starting where the last
 * one ended; a position where no alternative matches is passed over, and the passed-over characters
 * between two matches form one piece.  Appends the piece starts (document char indices) to out. */
static int64_t split_isolated(const uint32_t *cp, int64_t a, int64_t b, const alt_fn *alts, int64_t *out)
{
    Doc sub = { cp + a, b - a };
    int64_t np = 0, p = 0;
    int in_gap = 0;
    while (p < sub.n) {
        int64_t e = -1;
        for (int k = 0; alts[k]; k++) {
            e = alts[k](&sub, p);
            if (e > p) break;
        }
        if (e > p) {
            out[np++] = a + p;
            in_gap = 0;
            p = e;
        } else {
            if (!in_gap) out[np++] = a + p;
            in_gap = 1;
            p++;
        }
    }
    return np;
}

/* The three stages over one document of nc chars: returns the number of pieces, their starts (char
 * indices) in s3.  s1, s2, s3 hold nc + 1 entries each. */
static int64_t ds_split_doc(const uint32_t *cp, int64_t nc, int64_t *s1, int64_t *s2, int64_t *s3)
{
    int64_t n1 = split_isolated(cp, 0, nc, DS_STAGE1, s1), n2 = 0, n3 = 0;
    s1[n1] = nc;
    for (int64_t k = 0; k < n1; k++) n2 += split_isolated(cp, s1[k], s1[k + 1], DS_STAGE2, s2 + n2);
    s2[n2] = nc;
    for (int64_t k = 0; k < n2; k++) n3 += split_isolated(cp, s2[k], s2[k + 1], DS_STAGE3, s3 + n3);
    return n3;
}

static const alt_fn FAM_G2[] = { g2_contraction, g2_letters, g2_numbers, g2_other,
                                 ws_not_before_nonws, ws_all, NULL };
static const alt_fn FAM_CL[] = { cl_contraction, cl_letters, num_upto3, sp_opt_other_newlines,
                                 ws_to_last_newline, ws_not_before_nonws, ws_all, NULL };
static const alt_fn FAM_OK[] = { ok_word_lower, ok_word_upper, num_upto3, sp_opt_other_newlines,
                                 ws_to_last_newline, ws_not_before_nonws, ws_all, NULL };

static const alt_fn *family_alts(int family)
{
    switch (family) {
    case 1: return FAM_G2;
    case 2: return FAM_CL;
    case 3: return FAM_OK;
    case 4: return DS_STAGE3;   /* the DeepSeek style runs all three stages (ds_split_doc) */
    default: return NULL;
    }
}

/* Pre-tokenize a batch.  offsets[0..n_docs] are byte offsets (offsets[0] = 0, non-decreasing,
 * offsets[n_docs] = n).  Writes the byte offset of every piece start to piece_starts (document
 * order) and returns the number of pieces.  Errors: -1 invalid UTF-8, -2 capacity, -3 bad family,
 * -4 bad offsets, -5 out of memory, -6 no alternative matched (cannot happen for these families). */
int64_t orc_pretokenize(int family, const uint8_t *text, uint64_t n, const uint64_t *offsets,
                        uint32_t n_docs, uint64_t *piece_starts, uint64_t cap)
{
    const alt_fn *alts = family_alts(family);
    if (!alts) return -3;
    if (!g_cls) return -5;
    if (offsets[0] != 0 || offsets[n_docs] != n) return -4;
    uint64_t maxdoc = 0;
    for (uint32_t d = 0; d < n_docs; d++) {
        if (offsets[d + 1] < offsets[d]) return -4;
        if (offsets[d + 1] - offsets[d] > maxdoc) maxdoc = offsets[d + 1] - offsets[d];
    }
    uint32_t *cp = (uint32_t *)malloc((maxdoc + 1) * sizeof(uint32_t));
    uint64_t *pos = (uint64_t *)malloc((maxdoc + 1) * sizeof(uint64_t));
    int64_t *ds = family == 4 ? (int64_t *)malloc(3 * (maxdoc + 1) * sizeof(int64_t)) : NULL;
    if (!cp || !pos || (family == 4 && !ds)) { free(cp); free(pos); free(ds); return -5; }
    uint64_t np = 0;
    int64_t rc = 0;
    for (uint32_t d = 0; d < n_docs && rc == 0; d++) {
        uint64_t b0 = offsets[d];
        int64_t nc = utf8_decode(text + b0, offsets[d + 1] - b0, cp, pos);
        if (nc < 0) { rc = -1; break; }
        if (family == 4) {
            int64_t *s3 = ds + 2 * (maxdoc + 1);
            int64_t n3 = ds_split_doc(cp, nc, ds, ds + (maxdoc + 1), s3);
            if (np + (uint64_t)n3 > cap) { rc = -2; break; }
            for (int64_t k = 0; k < n3; k++) piece_starts[np++] = b0 + pos[s3[k]];
            continue;
        }
        Doc doc = { cp, nc };
        int64_t p = 0;
        while (p < nc) {
            int64_t e = -1;
            for (int a = 0; alts[a]; a++) {
                e = alts[a](&doc, p);
                if (e > p) break;
            }
            if (e <= p) { rc = -6; break; }
            if (np >= cap) { rc = -2; break; }
            piece_starts[np++] = b0 + pos[p];
            p = e;
        }
    }
    free(cp);
    free(pos);
    free(ds);
    return rc ? rc : (int64_t)np;
}

/* ------------------------------------------------------------------------------------------ */
/* merge-rank map: (left_id, right_id) -> rank, plain open addressing                            */

typedef struct {
    uint64_t *keys;     /* (left << 32 | right) + 1; 0 = empty */
    uint32_t *rank;
    uint64_t mask;
    uint32_t n_merges;
} RankMap;

static uint64_t mix64(uint64_t x)
{
    x ^= x >> 33; x *= 0xff51afd7ed558ccdULL; x ^= x >> 33; x *= 0xc4ceb9fe1a85ec53ULL; x ^= x >> 33;
    return x;
}

static RankMap *rankmap_new(const uint32_t *merges, uint32_t n_merges)
{
    RankMap *m = (RankMap *)calloc(1, sizeof(RankMap));
    uint64_t cap = 16;
    while (cap < 2ull * n_merges + 16) cap <<= 1;
    m->keys = (uint64_t *)calloc(cap, sizeof(uint64_t));
    m->rank = (uint32_t *)calloc(cap, sizeof(uint32_t));
    m->mask = cap - 1;
    m->n_merges = n_merges;
    for (uint32_t r = 0; r < n_merges; r++) {
        uint64_t key = (((uint64_t)merges[2 * r] << 32) | merges[2 * r + 1]) + 1;
        uint64_t h = mix64(key) & m->mask;
        while (m->keys[h] && m->keys[h] != key) h = (h + 1) & m->mask;
        if (!m->keys[h]) { m->keys[h] = key; m->rank[h] = r; }   /* first (lowest) rank wins */
    }
    return m;
}

static inline uint32_t rankmap_get(const RankMap *m, uint32_t l, uint32_t r)
{
    uint64_t key = (((uint64_t)l << 32) | r) + 1;
    uint64_t h = mix64(key) & m->mask;
    while (m->keys[h]) {
        if (m->keys[h] == key) return m->rank[h];
        h = (h + 1) & m->mask;
    }
    return UINT32_MAX;
}

static void rankmap_free(RankMap *m)
{
    if (!m) return;
    free(m->keys); free(m->rank); free(m);
}

void *orc_bpe_new(const uint32_t *merges, uint32_t n_merges) { return rankmap_new(merges, n_merges); }
void orc_bpe_free(void *h) { rankmap_free((RankMap *)h); }

/* ------------------------------------------------------------------------------------------ */
/* E: priority-queue BPE on one piece                                                            */

typedef struct { uint64_t *a; uint64_t n, cap; } Heap;   /* min-heap of (rank << 32 | pos) */

static int heap_push(Heap *h, uint64_t v)
{
    if (h->n == h->cap) {
        uint64_t nc = h->cap ? 2 * h->cap : 64;
        uint64_t *na = (uint64_t *)realloc(h->a, nc * sizeof(uint64_t));
        if (!na) return -1;
        h->a = na; h->cap = nc;
    }
    uint64_t i = h->n++;
    while (i > 0) {
        uint64_t par = (i - 1) / 2;
        if (h->a[par] <= v) break;
        h->a[i] = h->a[par];
        i = par;
    }
    h->a[i] = v;
    return 0;
}

static uint64_t heap_pop(Heap *h)
{
    uint64_t top = h->a[0], v = h->a[--h->n];
    uint64_t i = 0;
    for (;;) {
        uint64_t l = 2 * i + 1, r = l + 1, m = i;
        uint64_t best = v;
        if (l < h->n && h->a[l] < best) { m = l; best = h->a[l]; }
        if (r < h->n && h->a[r] < best) { m = r; best = h->a[r]; }
        if (m == i) break;
        h->a[i] = h->a[m];
        i = m;
    }
    if (h->n) h->a[i] = v;
    return top;
}

/* Encode one piece of len bytes; writes its IDs to out and returns the count (< 0 on OOM). */
static int64_t bpe_piece(const RankMap *m, const uint8_t *s, uint64_t len, uint32_t *out,
                         uint32_t *ids, int64_t *nxt, int64_t *prv, Heap *hp)
{
    if (len == 0) return 0;
    for (uint64_t i = 0; i < len; i++) {
        ids[i] = s[i];
        nxt[i] = (i + 1 < len) ? (int64_t)(i + 1) : -1;
        prv[i] = (int64_t)i - 1;
    }
    hp->n = 0;
    for (uint64_t i = 0; i + 1 < len; i++) {
        uint32_t r = rankmap_get(m, ids[i], ids[i + 1]);
        if (r != UINT32_MAX && heap_push(hp, ((uint64_t)r << 32) | i)) return -1;
    }
    while (hp->n) {
        uint64_t top = heap_pop(hp);
        uint32_t r = (uint32_t)(top >> 32);
        int64_t i = (int64_t)(top & 0xffffffffu);
        int64_t j = nxt[i];
        /* stale entry: node i was absorbed, or its current pair is no longer the one of rank r */
        if (prv[i] == -2 || j < 0 || rankmap_get(m, ids[i], ids[j]) != r) continue;
        ids[i] = 256u + r;
        nxt[i] = nxt[j];
        if (nxt[j] >= 0) prv[nxt[j]] = i;
        prv[j] = -2;                                   /* absorbed */
        if (prv[i] >= 0) {
            uint32_t rl = rankmap_get(m, ids[prv[i]], ids[i]);
            if (rl != UINT32_MAX && heap_push(hp, ((uint64_t)rl << 32) | (uint64_t)prv[i])) return -1;
        }
        if (nxt[i] >= 0) {
            uint32_t rr = rankmap_get(m, ids[i], ids[nxt[i]]);
            if (rr != UINT32_MAX && heap_push(hp, ((uint64_t)rr << 32) | (uint64_t)i)) return -1;
        }
    }
    int64_t k = 0;
    for (int64_t i = 0; i >= 0; i = nxt[i]) out[k++] = ids[i];
    return k;
}

/* Encode pieces [piece_starts[p], piece_starts[p+1]) (piece_starts[n_pieces] = end).  Writes the
 * concatenated IDs to out_ids and, if ntok is non-NULL, each piece's token count.  Returns the
 * number of IDs, -2 on capacity, -5 on out of memory. */
int64_t orc_bpe_encode(void *handle, const uint8_t *text, const uint64_t *piece_starts,
                       uint64_t n_pieces, uint32_t *out_ids, uint64_t cap, uint32_t *ntok)
{
    const RankMap *m = (const RankMap *)handle;
    uint64_t maxlen = 0;
    for (uint64_t p = 0; p < n_pieces; p++) {
        uint64_t l = piece_starts[p + 1] - piece_starts[p];
        if (l > maxlen) maxlen = l;
    }
    uint32_t *ids = (uint32_t *)malloc((maxlen + 1) * sizeof(uint32_t));
    int64_t *nxt = (int64_t *)malloc((maxlen + 1) * sizeof(int64_t));
    int64_t *prv = (int64_t *)malloc((maxlen + 1) * sizeof(int64_t));
    Heap hp = { 0, 0, 0 };
    int64_t rc = 0;
    uint64_t nt = 0;
    if (!ids || !nxt || !prv) rc = -5;
    for (uint64_t p = 0; p < n_pieces && rc == 0; p++) {
        uint64_t b = piece_starts[p], l = piece_starts[p + 1] - b;
        if (nt + l > cap) { rc = -2; break; }             /* a piece never has more IDs than bytes */
        int64_t k = bpe_piece(m, text + b, l, out_ids + nt, ids, nxt, prv, &hp);
        if (k < 0) { rc = -5; break; }
        if (ntok) ntok[p] = (uint32_t)k;
        nt += (uint64_t)k;
    }
    free(ids); free(nxt); free(prv); free(hp.a);
    return rc ? rc : (int64_t)nt;
}

/* ------------------------------------------------------------------------------------------ */
/* T: byte-level BPE trainer over the unique-piece multiset                                       */

typedef struct { uint32_t a, b; int64_t count; uint32_t *w; uint32_t nw, capw; int forbidden; uint32_t tstamp; } Pair;

typedef struct {
    uint64_t *keys;   /* (a << 32 | b) + 1, 0 = empty */
    uint32_t *idx;    /* index into pairs */
    uint64_t mask, used;
    Pair *pairs;
    uint64_t npairs, cappairs;
} PairMap;

static int pm_grow(PairMap *pm)
{
    uint64_t ncap = (pm->mask + 1) * 2;
    uint64_t *nk = (uint64_t *)calloc(ncap, sizeof(uint64_t));
    uint32_t *ni = (uint32_t *)calloc(ncap, sizeof(uint32_t));
    if (!nk || !ni) { free(nk); free(ni); return -1; }
    for (uint64_t h = 0; h <= pm->mask; h++) {
        if (!pm->keys[h]) continue;
        uint64_t g = mix64(pm->keys[h]) & (ncap - 1);
        while (nk[g]) g = (g + 1) & (ncap - 1);
        nk[g] = pm->keys[h];
        ni[g] = pm->idx[h];
    }
    free(pm->keys); free(pm->idx);
    pm->keys = nk; pm->idx = ni; pm->mask = ncap - 1;
    return 0;
}

static Pair *pm_get(PairMap *pm, uint32_t a, uint32_t b, int create)
{
    uint64_t key = (((uint64_t)a << 32) | b) + 1;
    uint64_t h = mix64(key) & pm->mask;
    while (pm->keys[h]) {
        if (pm->keys[h] == key) return &pm->pairs[pm->idx[h]];
        h = (h + 1) & pm->mask;
    }
    if (!create) return NULL;
    if (pm->npairs == pm->cappairs) {
        uint64_t nc = pm->cappairs ? 2 * pm->cappairs : 1024;
        Pair *np = (Pair *)realloc(pm->pairs, nc * sizeof(Pair));
        if (!np) return NULL;
        pm->pairs = np; pm->cappairs = nc;
    }
    Pair *p = &pm->pairs[pm->npairs];
    memset(p, 0, sizeof(*p));
    p->a = a; p->b = b; p->tstamp = UINT32_MAX;
    pm->keys[h] = key;
    pm->idx[h] = (uint32_t)pm->npairs++;
    if (++pm->used * 2 > pm->mask + 1 && pm_grow(pm)) return NULL;
    return &pm->pairs[pm->npairs - 1];
}

static int pair_add_word(Pair *p, uint32_t w)
{
    if (p->nw && p->w[p->nw - 1] == w) return 0;
    if (p->nw == p->capw) {
        uint32_t nc = p->capw ? 2 * p->capw : 4;
        uint32_t *nw = (uint32_t *)realloc(p->w, nc * sizeof(uint32_t));
        if (!nw) return -1;
        p->w = nw; p->capw = nc;
    }
    p->w[p->nw++] = w;
    return 0;
}

/* Record a pair whose count changed during this merge step (once per step). */
static int note_touched(PairMap *pm, Pair *q, uint32_t step, uint64_t **t, uint64_t *n, uint64_t *cap)
{
    if (q->tstamp == step) return 0;
    q->tstamp = step;
    if (*n == *cap) {
        uint64_t nc = *cap ? 2 * *cap : 1024;
        uint64_t *nt = (uint64_t *)realloc(*t, nc * sizeof(uint64_t));
        if (!nt) return -1;
        *t = nt; *cap = nc;
    }
    (*t)[(*n)++] = (uint64_t)(q - pm->pairs);
    return 0;
}

/* trainer heap: max by count, then min (a, b) */
typedef struct { int64_t count; uint32_t a, b; } TEnt;
typedef struct { TEnt *v; uint64_t n, cap; } THeap;

static int tent_before(const TEnt *x, const TEnt *y)
{
    if (x->count != y->count) return x->count > y->count;
    if (x->a != y->a) return x->a < y->a;
    return x->b < y->b;
}

static int theap_push(THeap *h, TEnt e)
{
    if (h->n == h->cap) {
        uint64_t nc = h->cap ? 2 * h->cap : 1024;
        TEnt *nv = (TEnt *)realloc(h->v, nc * sizeof(TEnt));
        if (!nv) return -1;
        h->v = nv; h->cap = nc;
    }
    uint64_t i = h->n++;
    while (i > 0) {
        uint64_t par = (i - 1) / 2;
        if (!tent_before(&e, &h->v[par])) break;
        h->v[i] = h->v[par];
        i = par;
    }
    h->v[i] = e;
    return 0;
}

static TEnt theap_pop(THeap *h)
{
    TEnt top = h->v[0], v = h->v[--h->n];
    uint64_t i = 0;
    for (;;) {
        uint64_t l = 2 * i + 1, r = l + 1, m = i;
        const TEnt *best = &v;
        if (l < h->n && tent_before(&h->v[l], best)) { m = l; best = &h->v[l]; }
        if (r < h->n && tent_before(&h->v[r], best)) { m = r; best = &h->v[r]; }
        if (m == i) break;
        h->v[i] = h->v[m];
        i = m;
    }
    if (h->n) h->v[i] = v;
    return top;
}

/* Unique byte strings with counts (hash set keyed by content). */
typedef struct { uint64_t off; uint32_t len; int64_t count; } WordRec;

/* Train n_merges merges on `corpus` pre-tokenized with `family`.  Writes merges (left, right) pairs
 * to out_merges (2 * n_merges uint32).  Returns the number of merges produced (< n_merges when the
 * corpus runs out of pairs seen at least twice), or < 0 on error (-1 UTF-8, -3 family, -5 OOM). */
int64_t orc_train(int family, const uint8_t *corpus, uint64_t n, uint32_t n_merges,
                  uint32_t max_token_bytes, uint32_t *out_merges)
{
    uint64_t offs[2] = { 0, n };
    uint64_t cap = n + 1;
    uint64_t *ps = (uint64_t *)malloc((cap + 1) * sizeof(uint64_t));
    if (!ps) return -5;
    int64_t np = orc_pretokenize(family, corpus, n, offs, 1, ps, cap);
    if (np < 0) { free(ps); return np; }
    ps[np] = n;

    /* unique pieces */
    uint64_t wcap = 1024;
    while (wcap < 2 * (uint64_t)np + 16) wcap <<= 1;
    WordRec *wr = (WordRec *)calloc(wcap, sizeof(WordRec));
    uint32_t *wslot = (uint32_t *)malloc(wcap * sizeof(uint32_t));
    uint64_t nwords = 0;
    uint32_t *order = (uint32_t *)malloc(wcap * sizeof(uint32_t));
    if (!wr || !wslot || !order) { free(ps); free(wr); free(wslot); free(order); return -5; }
    for (uint64_t h = 0; h < wcap; h++) wslot[h] = UINT32_MAX;
    for (int64_t p = 0; p < np; p++) {
        uint64_t off = ps[p];
        uint32_t len = (uint32_t)(ps[p + 1] - off);
        uint64_t hv = 1469598103934665603ULL;
        for (uint32_t i = 0; i < len; i++) { hv ^= corpus[off + i]; hv *= 1099511628211ULL; }
        uint64_t h = mix64(hv) & (wcap - 1);
        for (;;) {
            uint32_t s = wslot[h];
            if (s == UINT32_MAX) {
                wslot[h] = (uint32_t)nwords;
                wr[nwords].off = off; wr[nwords].len = len; wr[nwords].count = 1;
                order[nwords] = (uint32_t)nwords;
                nwords++;
                break;
            }
            if (wr[s].len == len && memcmp(corpus + wr[s].off, corpus + off, len) == 0) {
                wr[s].count++;
                break;
            }
            h = (h + 1) & (wcap - 1);
        }
    }
    free(wslot);
    free(ps);

    /* symbol arrays */
    uint64_t total = 0;
    for (uint64_t w = 0; w < nwords; w++) total += wr[w].len;
    uint32_t *sym = (uint32_t *)malloc((total + 1) * sizeof(uint32_t));
    uint64_t *woff = (uint64_t *)malloc((nwords + 1) * sizeof(uint64_t));
    uint32_t *wlen = (uint32_t *)malloc((nwords + 1) * sizeof(uint32_t));
    int64_t *wcnt = (int64_t *)malloc((nwords + 1) * sizeof(int64_t));
    uint32_t *stamp = (uint32_t *)malloc((nwords + 1) * sizeof(uint32_t));
    uint32_t *tlen = (uint32_t *)malloc((256 + (uint64_t)n_merges) * sizeof(uint32_t));
    uint32_t *tmp = (uint32_t *)malloc((total + 1) * sizeof(uint32_t));
    if (!sym || !woff || !wlen || !wcnt || !stamp || !tlen || !tmp) return -5;
    uint64_t o = 0;
    for (uint64_t w = 0; w < nwords; w++) {
        woff[w] = o; wlen[w] = wr[w].len; wcnt[w] = wr[w].count; stamp[w] = UINT32_MAX;
        for (uint32_t i = 0; i < wr[w].len; i++) sym[o + i] = corpus[wr[w].off + i];
        o += wr[w].len;
    }
    free(wr); free(order);
    for (uint32_t t = 0; t < 256; t++) tlen[t] = 1;

    PairMap pm;
    memset(&pm, 0, sizeof(pm));
    pm.mask = (1u << 20) - 1;
    pm.keys = (uint64_t *)calloc(pm.mask + 1, sizeof(uint64_t));
    pm.idx = (uint32_t *)calloc(pm.mask + 1, sizeof(uint32_t));
    THeap th = { 0, 0, 0 };
    int64_t rc = 0;
    for (uint64_t w = 0; w < nwords && rc == 0; w++) {
        const uint32_t *s = sym + woff[w];
        for (uint32_t i = 0; i + 1 < wlen[w]; i++) {
            Pair *p = pm_get(&pm, s[i], s[i + 1], 1);
            if (!p || pair_add_word(p, (uint32_t)w)) { rc = -5; break; }
            p->count += wcnt[w];
        }
    }
    for (uint64_t i = 0; i < pm.npairs && rc == 0; i++) {
        TEnt e = { pm.pairs[i].count, pm.pairs[i].a, pm.pairs[i].b };
        if (e.count >= 2 && theap_push(&th, e)) rc = -5;
    }

    /* touched-pair list for lazy heap refresh */
    uint64_t *touched = NULL, ntouched = 0, captouched = 0;
    uint32_t made = 0;
    while (rc == 0 && made < n_merges) {
        if (th.n == 0) break;                                  /* corpus exhausted */
        TEnt top = theap_pop(&th);
        Pair *p = pm_get(&pm, top.a, top.b, 0);
        if (!p || p->forbidden) continue;
        if (p->count != top.count) {                           /* stale: refresh */
            if (p->count >= 2) {
                TEnt e = { p->count, p->a, p->b };
                if (theap_push(&th, e)) rc = -5;
            }
            continue;
        }
        if (top.count < 2) break;
        uint32_t a = top.a, b = top.b;
        if (tlen[a] + tlen[b] > max_token_bytes) { p->forbidden = 1; continue; }
        uint32_t z = 256 + made;
        out_merges[2 * made] = a;
        out_merges[2 * made + 1] = b;
        tlen[z] = tlen[a] + tlen[b];
        ntouched = 0;
        /* the word list may grow while we iterate (pair_add_word on other pairs only) */
        uint32_t nw = p->nw;
        uint32_t *wl = p->w;
        p->w = NULL; p->nw = 0; p->capw = 0;
        for (uint32_t k = 0; k < nw && rc == 0; k++) {
            uint32_t w = wl[k];
            if (stamp[w] == made) continue;
            stamp[w] = made;
            uint32_t *s = sym + woff[w];
            uint32_t L = wlen[w], L2 = 0;
            int changed = 0;
            for (uint32_t i = 0; i < L;) {
                if (i + 1 < L && s[i] == a && s[i + 1] == b) { tmp[L2++] = z; i += 2; changed = 1; }
                else tmp[L2++] = s[i++];
            }
            if (!changed) continue;
            int64_t c = wcnt[w];
            for (uint32_t i = 0; i + 1 < L && rc == 0; i++) {
                Pair *q = pm_get(&pm, s[i], s[i + 1], 0);
                q->count -= c;
                if (note_touched(&pm, q, made, &touched, &ntouched, &captouched)) rc = -5;
            }
            for (uint32_t i = 0; i + 1 < L2 && rc == 0; i++) {
                Pair *q = pm_get(&pm, tmp[i], tmp[i + 1], 1);
                if (!q) { rc = -5; break; }
                q->count += c;
                if ((tmp[i] == z || tmp[i + 1] == z) && pair_add_word(q, w)) { rc = -5; break; }
                if (note_touched(&pm, q, made, &touched, &ntouched, &captouched)) rc = -5;
            }
            memcpy(s, tmp, L2 * sizeof(uint32_t));
            wlen[w] = L2;
        }
        free(wl);
        for (uint64_t k = 0; k < ntouched && rc == 0; k++) {
            Pair *q = &pm.pairs[touched[k]];
            if (!q->forbidden && q->count >= 2) {
                TEnt e = { q->count, q->a, q->b };
                if (theap_push(&th, e)) rc = -5;
            }
        }
        made++;
    }
    for (uint64_t i = 0; i < pm.npairs; i++) free(pm.pairs[i].w);
    free(pm.pairs); free(pm.keys); free(pm.idx); free(th.v); free(touched);
    free(sym); free(woff); free(wlen); free(wcnt); free(stamp); free(tlen); free(tmp);
    return rc ? rc : (int64_t)made;
}

/* ------------------------------------------------------------------------------------------ */
/* full path: F = E* o G over a batch                                                           */

/* Tokenize a batch.  out_ids receives all IDs in document order; out_offsets[d] is the index of
 * document d's first ID (out_offsets[n_docs] = total).  Returns the number of IDs or < 0 as in
 * orc_pretokenize / orc_bpe_encode. */
int64_t orc_encode_batch(int family, void *bpe, const uint8_t *text, uint64_t n,
                         const uint64_t *offsets, uint32_t n_docs, uint32_t *out_ids, uint64_t cap,
                         uint64_t *out_offsets)
{
    uint64_t *ps = (uint64_t *)malloc((n + 2) * sizeof(uint64_t));
    uint32_t *ntok = (uint32_t *)malloc((n + 2) * sizeof(uint32_t));
    if (!ps || !ntok) { free(ps); free(ntok); return -5; }
    int64_t np = orc_pretokenize(family, text, n, offsets, n_docs, ps, n + 1);
    if (np < 0) { free(ps); free(ntok); return np; }
    ps[np] = n;
    int64_t nt = orc_bpe_encode(bpe, text, ps, (uint64_t)np, out_ids, cap, ntok);
    if (nt >= 0) {
        /* document d starts at its first piece: the first piece whose start is >= offsets[d] */
        uint64_t p = 0, t = 0;
        for (uint32_t d = 0; d <= n_docs; d++) {
            while (p < (uint64_t)np && ps[p] < offsets[d]) t += ntok[p++];
            out_offsets[d] = t;
        }
    }
    free(ps); free(ntok);
    return nt;
}
