// vocab.h -- the library's vocabulary handle (opaque in the C ABI; host code of the library only).
#pragma once
#include "internal.h"

struct toktier_vocab {
    int device;
    int family;
    uint32_t n_merges;
    void *dmem;     // pair tables, merges, automaton tables
    void *dwords;   // whole-piece tables (may be NULL)
    void *dstr;     // token strings and their hash (may be NULL)
    void *dlen;     // byte length of every token
    void *dadded;   // added-token tables (NULL without added tokens)
    tt::DevVocab dv;
    tt::DevAdded da;   // da.n == 0: no added tokens
    // host copy of the automaton's transition maps (byte s of map c: next state | piece start << 4)
    uint8_t hmap[tt::NCTX_MAX][16];
};
