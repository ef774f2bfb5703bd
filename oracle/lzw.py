"""LZW-style embedding allocation (TEST INFRASTRUCTURE ONLY: the plain, slow
definition the library's l3_allocate_lzw is checked against).

"L^3: Large Lookup Layers" allocates the v embeddings over the vocabulary with a
variant of LZW compression (kimjy99.github.io page, section "1. Embedding
Allocation"; papernotes.org page, section 关键设计 item 2; sciencestack.ai page,
Fig. 5 caption).  The pages give it in prose only; the readings taken here:

1. Codewords.  The corpus is parsed LZW-style: the current phrase w grows by the
   next token c while w + c is a known codeword (single tokens are always known);
   when w + c is new it becomes a codeword with frequency 1, the codeword formed
   by dropping its first token gets +1 (it is created, with frequency 1, if it is
   not a codeword yet), and the phrase restarts at c.
2. Allocation.  Every token first gets one embedding.  The codewords are then
   visited by decreasing frequency (ties: shorter first, then by the token tuple)
   and each gives one embedding to the token it ends with, unless that token
   already has k; passes over the list repeat until the total reaches v.
   v must lie in [vocab, vocab * k].
"""
from __future__ import annotations


def codewords(corpus) -> dict:
    """tuple of tokens -> frequency, per reading 1."""
    freq: dict = {}
    w: tuple = ()
    for c in corpus:
        c = int(c)
        wc = w + (c,)
        if len(wc) == 1 or wc in freq:
            w = wc
            continue
        freq[wc] = 1
        suffix = wc[1:]
        freq[suffix] = freq.get(suffix, 0) + 1
        w = (c,)
    return freq


def allocate(corpus, vocab: int, v: int, k: int) -> list:
    """d_t per token (sum v, each in [1, k]), per reading 2."""
    if not (vocab <= v <= vocab * k):
        raise ValueError("v must lie in [vocab, vocab * k]")
    freq = codewords(corpus)
    order = sorted(freq, key=lambda cw: (-freq[cw], len(cw), cw))
    d = [1] * vocab
    total = vocab
    while total < v:
        moved = False
        for cw in order:
            if total == v:
                break
            t = cw[-1]
            if d[t] < k:
                d[t] += 1
                total += 1
                moved = True
        if not moved:
            # no codeword ends with a token below k: the remaining budget cannot
            # be placed by the codewords alone
            raise ValueError("codewords cannot place the budget")
    return d
