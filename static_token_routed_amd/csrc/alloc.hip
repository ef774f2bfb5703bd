// LZW-style embedding allocation (host code): which token IDs get how many of the
// v table rows.  "L^3: Large Lookup Layers" allocates the embeddings with a variant
// of LZW compression (kimjy99.github.io page, section "1. Embedding Allocation";
// papernotes.org page, section 关键设计 item 2; sciencestack.ai page, Fig. 5
// caption), given there in prose only.  Readings taken:
//  * Codewords.  The corpus is parsed LZW-style: the current phrase w grows by the
//    next token c while w + c is a known codeword (single tokens are always known);
//    when w + c is new it becomes a codeword with frequency 1, the codeword formed
//    by dropping its first token gets +1 (created with frequency 1 if it is not a
//    codeword yet), and the phrase restarts at c.
//  * Allocation.  Every token first gets one embedding; the codewords are then
//    visited by decreasing frequency (ties: shorter first, then by their token
//    sequence) and each gives one embedding to the token it ends with, unless that
//    token already has k; passes repeat until the total reaches v.
// The codewords live in a trie (node = codeword prefix, child keyed by (node,
// token) in a hash map); equal-length token sequences compare like the trie's
// pre-order with children in token order, so the tie rule needs no sequence
// comparisons.
#include <algorithm>
#include <unordered_map>
#include <vector>

#include "l3_internal.h"

namespace {

struct Trie {
    // nodes 0 .. vocab-1: the single tokens
    std::vector<int32_t> parent, token, depth;
    std::vector<int64_t> freq;
    std::vector<uint8_t> present;  // a codeword (in the frequency table)
    std::unordered_map<uint64_t, int32_t> child;
    int64_t vocab;

    explicit Trie(int64_t v) : vocab(v) {
        parent.assign(v, -1);
        depth.assign(v, 1);
        freq.assign(v, 0);
        present.assign(v, 0);
        token.resize(v);
        for (int64_t t = 0; t < v; ++t) token[t] = (int32_t)t;
    }
    uint64_t key(int32_t node, int32_t tok) const { return (uint64_t)node * (uint64_t)vocab + (uint64_t)tok; }
    int32_t find(int32_t node, int32_t tok) const {
        const auto it = child.find(key(node, tok));
        return it == child.end() ? -1 : it->second;
    }
    int32_t make(int32_t node, int32_t tok) {
        const int32_t f = find(node, tok);
        if (f >= 0) return f;
        const int32_t id = (int32_t)parent.size();
        parent.push_back(node);
        token.push_back(tok);
        depth.push_back(depth[node] + 1);
        freq.push_back(0);
        present.push_back(0);
        child.emplace(key(node, tok), id);
        return id;
    }
};

}  // namespace

extern "C" int l3_allocate_lzw(const int32_t *corpus, int64_t n, int64_t vocab, int64_t v, int32_t k,
                               int64_t *offsets) {
    if (!offsets || vocab <= 0 || k <= 0 || n < 0 || (n > 0 && !corpus)) return L3_ERR_INVALID_ARG;
    if (vocab >= (1ll << 31) || v < vocab || v > vocab * (int64_t)k) return L3_ERR_INVALID_ARG;
    for (int64_t i = 0; i < n; ++i)
        if (corpus[i] < 0 || corpus[i] >= vocab) return L3_ERR_TOKEN_RANGE;
    Trie tr(vocab);
    // codewords and their frequencies; w is a trie node (-1: empty phrase) and
    // toks the phrase's tokens (to form the suffix of a new codeword)
    std::vector<int32_t> toks;
    int32_t w = -1;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t c = corpus[i];
        if (w < 0) {
            w = c;
            toks.assign(1, c);
            continue;
        }
        const int32_t wc = tr.find(w, c);
        if (wc >= 0 && tr.present[wc]) {
            w = wc;
            toks.push_back(c);
            continue;
        }
        const int32_t nw = tr.make(w, c);
        tr.present[nw] = 1;
        tr.freq[nw] = 1;
        // the new codeword without its first token: tokens toks[1..] followed by c
        int32_t s = toks.size() > 1 ? toks[1] : c;
        for (size_t j = 2; j < toks.size(); ++j) s = tr.make(s, toks[j]);
        if (toks.size() > 1) s = tr.make(s, c);
        tr.present[s] = 1;
        tr.freq[s] += 1;
        w = c;
        toks.assign(1, c);
    }
    // pre-order of the trie (children in token order): the tie rank of equal-length codewords
    const int32_t nn = (int32_t)tr.parent.size();
    std::vector<std::vector<int32_t>> kids(nn);
    for (int32_t i = (int32_t)vocab; i < nn; ++i) kids[tr.parent[i]].push_back(i);
    std::vector<int64_t> pre(nn, 0);
    {
        int64_t counter = 0;
        std::vector<int32_t> stack;
        for (int64_t t = vocab - 1; t >= 0; --t) stack.push_back((int32_t)t);
        while (!stack.empty()) {
            const int32_t x = stack.back();
            stack.pop_back();
            pre[x] = counter++;
            auto &ch = kids[x];
            std::sort(ch.begin(), ch.end(), [&](int32_t a, int32_t b) { return tr.token[a] < tr.token[b]; });
            for (auto it = ch.rbegin(); it != ch.rend(); ++it) stack.push_back(*it);
        }
    }
    std::vector<int32_t> order;
    for (int32_t i = 0; i < nn; ++i)
        if (tr.present[i]) order.push_back(i);
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        if (tr.freq[a] != tr.freq[b]) return tr.freq[a] > tr.freq[b];
        if (tr.depth[a] != tr.depth[b]) return tr.depth[a] < tr.depth[b];
        return pre[a] < pre[b];
    });
    // every token one embedding, then one per codeword to its last token, in passes
    std::vector<int64_t> d(vocab, 1);
    int64_t total = vocab;
    while (total < v) {
        bool moved = false;
        for (int32_t cw : order) {
            if (total == v) break;
            const int32_t t = tr.token[cw];
            if (d[t] < k) {
                ++d[t];
                ++total;
                moved = true;
            }
        }
        if (!moved) return L3_ERR_CAPACITY;
    }
    offsets[0] = 0;
    for (int64_t t = 0; t < vocab; ++t) offsets[t + 1] = offsets[t] + d[t];
    return L3_OK;
}
