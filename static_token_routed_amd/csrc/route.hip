// Batch sort by token ID and the per-ID blocks ("L^3: Large Lookup Layers":
// sciencestack.ai page, Fig. 3 caption -- the layer mixes channels only, so the
// batch may be sorted by token ID, giving one contiguous block per ID, and the
// sort undone afterwards; kimjy99.github.io page, section "2. Efficient
// Training and Inference" -- sorted, the "allowed tokens" mask is block
// diagonal).
//
// Stable LSD radix sort of the keys (token ID, or `vocab` for an ID outside
// [0, vocab)) in 9-bit digits.  Per pass:
//   k_sort_rank    each workgroup ranks kSortTile (512) keys: every wave takes
//                  kSortTile / 4 consecutive keys, 64 at a time in batch order; lanes with the
//                  same digit find each other with 9 ballots, the lowest lane
//                  reserves their places with one LDS atomic, so ranks are
//                  stable; writes the tile's digit histogram (digit-major).
//   k_sort_scatter each workgroup forms its tile's digit offsets from the whole
//                  digit-major histogram (an exclusive prefix), then writes each
//                  key to offset + rank.  Past kScatterDirectTiles tiles, where
//                  every workgroup summing the whole histogram would cost
//                  O(tiles^2), a wavefront per digit (k_hist_scan) first replaces
//                  each digit's row by its prefix over the tiles.
// Blocks: head flags of the sorted keys, counted per tile, then written at the
// tile's offset (the sum of the earlier tiles' counts).
// Nothing is read back to the host: counts stay on the device.
#include "l3_internal.h"

namespace l3 {
namespace {

__device__ inline int key_of(int32_t id, int32_t vocab) {
    return (id >= 0 && id < vocab) ? id : vocab;
}

__global__ __launch_bounds__(256) void k_zero_i32(int32_t *p, int64_t count) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) p[i] = 0;
}

// Ranks the keys of one kSortTile-key tile for the digit at `shift`.
__global__ __launch_bounds__(256) void k_sort_rank(const int32_t *__restrict__ keys, int n,
                                                   int shift, int from_ids, int vocab,
                                                   int32_t *__restrict__ rank,
                                                   int32_t *__restrict__ hist, int ntiles,
                                                   int32_t *__restrict__ hdr) {
    __shared__ uint32_t cnt[4][kRadix];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int tile = blockIdx.x;
    for (int i = threadIdx.x; i < 4 * kRadix; i += 256) (&cnt[0][0])[i] = 0;
    // the first pass clears the header words the later launches count into (the
    // out-of-range flag is written outright by k_seg_write)
    if (from_ids && tile == 0 && threadIdx.x < HDR_WORDS && threadIdx.x != HDR_ERR) hdr[threadIdx.x] = 0;
    __syncthreads();

    const int base = tile * kSortTile + w * (kSortTile / 4);
    uint32_t dig[kSortPer], rk[kSortPer];
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) {
        const int idx = base + r * 64 + lane;
        const bool valid = idx < n;
        int key = 0;
        if (valid) {
            key = keys[idx];
            if (from_ids) key = key_of(key, vocab);
        }
        const uint32_t d = ((uint32_t)key >> shift) & (kRadix - 1);
        uint64_t mask = __ballot(valid);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            const uint32_t bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            mask &= bit ? bb : ~bb;
        }
        const int leader = valid ? (__ffsll((unsigned long long)mask) - 1) : lane;
        const uint32_t below = (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
        uint32_t old = 0;
        if (valid && lane == leader) old = atomicAdd(&cnt[w][d], (uint32_t)__popcll(mask));
        old = __shfl(old, leader);
        dig[r] = d;
        rk[r] = old + below;
    }
    __syncthreads();
    for (int d = threadIdx.x; d < kRadix; d += 256) {
        uint32_t run = 0;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const uint32_t c = cnt[ww][d];
            cnt[ww][d] = run;
            run += c;
        }
        hist[(int64_t)d * ntiles + tile] = (int32_t)run;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) {
        const int idx = base + r * 64 + lane;
        if (idx < n) rank[idx] = (int32_t)(cnt[w][dig[r]] + rk[r]);
    }
}

// Block-wide exclusive scan of one int32 per thread (256 threads); returns the
// thread's exclusive prefix and writes the total to *total (all threads).
__device__ inline int32_t block_scan_256(int32_t v, int32_t *wsum, int32_t *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(x, o);
        if (lane >= o) x += u;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t pre = 0;
    for (int ww = 0; ww < w; ++ww) pre += wsum[ww];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    return pre + x - v;
}

// Past kScatterDirectTiles tiles: a wavefront per digit replaces the digit's row of
// the histogram by its exclusive prefix over the tiles and writes the digit's total
// after the last row (the histogram region holds kRadix x (ntiles + 1) words).
__global__ __launch_bounds__(256) void k_hist_scan(int32_t *__restrict__ hist, int ntiles) {
    const int lane = threadIdx.x & 63;
    const int d = blockIdx.x * 4 + (threadIdx.x >> 6);
    int32_t *row = hist + (int64_t)d * ntiles;
    int32_t carry = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 64) {
        const int t = t0 + lane;
        const int32_t v = t < ntiles ? row[t] : 0;
        int32_t x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t u = __shfl_up(x, o);
            if (lane >= o) x += u;
        }
        if (t < ntiles) row[t] = carry + x - v;
        carry += __shfl(x, 63);
    }
    if (lane == 0) hist[(int64_t)kRadix * ntiles + d] = carry;
}

// One workgroup per kSortTile-key tile.  The destination of digit d's keys in tile t
// is the exclusive prefix of the digit-major histogram at (d, t): the keys of all
// smaller digits, plus those of digit d in earlier tiles.  Each workgroup forms the
// 512 offsets of its own tile from the histogram (no separate scan pass), then
// scatters its keys to offset + rank.
__global__ __launch_bounds__(256) void k_sort_scatter(const int32_t *__restrict__ keys_in,
                                                      const int32_t *__restrict__ vals_in, int n,
                                                      int shift, int from_ids, int vocab,
                                                      const int32_t *__restrict__ hist, int ntiles,
                                                      int offsets_ready,
                                                      const int32_t *__restrict__ rank,
                                                      int32_t *__restrict__ keys_out,
                                                      int32_t *__restrict__ vals_out) {
    __shared__ int32_t off[kRadix];
    __shared__ int32_t wsum[4];
    const int t = blockIdx.x;
    // thread j owns digits 2j, 2j + 1
    int32_t tot[2], pre[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int32_t *h = hist + (int64_t)(2 * threadIdx.x + e) * ntiles;
        if (offsets_ready) {
            // k_hist_scan has left each row's prefix over the tiles and the totals
            tot[e] = hist[(int64_t)kRadix * ntiles + 2 * threadIdx.x + e];
            pre[e] = h[t];
            continue;
        }
        int32_t a = 0, b = 0;
#pragma unroll 8
        for (int u = 0; u < ntiles; ++u) {
            const int32_t c = h[u];
            a += c;
            b += u < t ? c : 0;
        }
        tot[e] = a;
        pre[e] = b;
    }
    int32_t all;
    const int32_t base = block_scan_256(tot[0] + tot[1], wsum, &all);
    off[2 * threadIdx.x] = base + pre[0];
    off[2 * threadIdx.x + 1] = base + tot[0] + pre[1];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortTile / 256; ++r) {
        const int idx = t * kSortTile + r * 256 + threadIdx.x;
        if (idx >= n) break;
        int key = keys_in[idx];
        if (from_ids) key = key_of(key, vocab);
        const uint32_t d = ((uint32_t)key >> shift) & (kRadix - 1);
        const int pos = off[d] + rank[idx];
        if ((unsigned)pos >= (unsigned)n) continue;  // cannot happen for a consistent ranking
        keys_out[pos] = key;
        vals_out[pos] = from_ids ? idx : vals_in[idx];
    }
}

// Per kSortTile-key tile: number of block heads and the position of its first head (n
// if it has none; tile_cnt[ntiles + tile]); also the inverse permutation.
__global__ __launch_bounds__(256) void k_seg_heads(const int32_t *__restrict__ sk,
                                                   const int32_t *__restrict__ perm, int n, int ntiles,
                                                   int32_t *__restrict__ tile_cnt,
                                                   int32_t *__restrict__ inv_perm) {
    __shared__ int32_t wsum[4], wfirst[4];
    const int base = blockIdx.x * kSortTile;
    int c = 0, first = n;
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) {
        const int s = base + r * 256 + threadIdx.x;
        if (s < n) {
            const bool h = s == 0 || sk[s] != sk[s - 1];
            c += h;
            if (h) first = min(first, s);
            const int i = perm[s];
            if ((unsigned)i < (unsigned)n) inv_perm[i] = s;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        c += __shfl_xor(c, o);
        first = min(first, __shfl_xor(first, o));
    }
    if ((threadIdx.x & 63) == 0) {
        wsum[threadIdx.x >> 6] = c;
        wfirst[threadIdx.x >> 6] = first;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        tile_cnt[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        tile_cnt[ntiles + blockIdx.x] = min(min(wfirst[0], wfirst[1]), min(wfirst[2], wfirst[3]));
    }
}

// Work items of one block (segment) j with S tokens from sorted position sb and ID t
// (t == vocab: IDs outside [0, vocab)).  The MFMA paths take blocks with many tokens
// or many rows (long row chains stall the wavefront-per-item path); long blocks of
// short enough rows are taken in dense items, the rest in streaming items.
struct BlockItems {
    int nl = 0, nh = 0, nd = 0, r0 = 0, d = 0;
};

// (r0, d: the block's first table row and row count, 0 for IDs out of range)
__device__ inline BlockItems block_items(int S, int t, int r0, int d, int vocab, int heavy_min,
                                         int dense_min, int light_tok) {
    BlockItems b;
    b.d = d;
    b.r0 = r0;
    if (heavy_min != INT32_MAX && t < vocab && (S >= heavy_min || b.d >= kHeavyMinRows)) {
        if (S >= dense_min && b.d >= kDenseMinD && b.d <= kDenseMaxD)
            b.nd = (S + kDenseTile - 1) / kDenseTile;
        else
            b.nh = (S + kHeavyTile - 1) / kHeavyTile;
    } else {
        b.nl = (S + light_tok - 1) / light_tok;
    }
    return b;
}

// Writes block j's items at list positions bl, bh, bd.  Light items carry what the
// kernel needs, so it starts loading rows at once.
__device__ inline void write_items(const BlockItems &b, int j, int sb, int S, bool in_range,
                                   int light_tok, int bl, int bh, int bd, int4 *light, int2 *heavy,
                                   int2 *dense) {
    for (int q = 0; q < b.nl; ++q)
        light[bl + q] = make_int4(sb + q * light_tok, min(light_tok, S - q * light_tok), b.r0,
                                  in_range ? b.d : -1);
    for (int q = 0; q < b.nh; ++q) heavy[bh + q] = make_int2(j, q * kHeavyTile);
    for (int q = 0; q < b.nd; ++q) dense[bd + q] = make_int2(j, q * kDenseTile);
}

// Work items of one block per lane (act: the lane holds block j of S tokens from sorted
// position sb, ID t), appended to the light or heavy lists with one wave-aggregated
// reservation per list: reserve(k, c) adds c to list counter k (the header words of
// list_hdr(k)) and returns the old value.  Item order does not affect
// results, only scheduling.  Light items of long blocks go to their own lists (when
// there are any): the longest to the front of light_long, the next longest to its
// back; streaming items of long blocks to the front of the heavy list, of mid-length
// ones to its back, of the others to the back of the dense list.
__device__ constexpr int list_hdr(int k) {
    return k == 0 ? HDR_NLIGHT : k == 1 ? HDR_NLIGHT_LONG : k == 2 ? HDR_NLIGHT_MID
         : k == 3 ? HDR_NLIGHT_SHORT : k == 4 ? HDR_NHEAVY : k == 5 ? HDR_NHEAVY_SHORT
         : k == 6 ? HDR_NHEAVY_TAIL : HDR_NDENSE;
}
template <class Reserve>
__device__ inline void block_worklist(bool act, int j, int sb, int S, int t, int r0, int d, int vocab,
                                      int heavy_min, int dense_min, int light_tok, int4 *light,
                                      int2 *heavy, int2 *dense, int4 *light_long, int nmax,
                                      Reserve reserve) {
    const int lane = threadIdx.x & 63;
    BlockItems bi;
    if (act) bi = block_items(S, t, r0, d, vocab, heavy_min, dense_min, light_tok);
    const bool lng = light_long != nullptr && bi.d >= kLightLongRows;
    const bool mid = light_long != nullptr && !lng && bi.d >= kLightMidRows;
    const bool lsh = light_long != nullptr && bi.d < kLightShortRows;  // to the light list's back
    const int nl = (lng || mid || lsh) ? 0 : bi.nl, nq = lng ? bi.nl : 0, nm = mid ? bi.nl : 0,
              nk = lsh ? bi.nl : 0;
    const bool hlong = bi.d >= kHeavyLongRows, hmid = !hlong && bi.d >= kHeavyMidRows;
    const int nh = hlong ? bi.nh : 0, ns = hmid ? bi.nh : 0, nt = (hlong || hmid) ? 0 : bi.nh,
              nd = bi.nd;
    // wave-inclusive scans of nl, nq, nm, nk, nh, ns, nt and nd
    int sl = nl, sq = nq, sm = nm, sk = nk, sh = nh, ss = ns, st = nt, sd = nd;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int a = __shfl_up(sl, o), e = __shfl_up(sq, o), f = __shfl_up(sm, o), k = __shfl_up(sk, o),
                  b = __shfl_up(sh, o), g = __shfl_up(ss, o), u = __shfl_up(st, o), c = __shfl_up(sd, o);
        if (lane >= o) { sl += a; sq += e; sm += f; sk += k; sh += b; ss += g; st += u; sd += c; }
    }
    int bl = 0, bq = 0, bm = 0, bk = 0, bh = 0, bs = 0, bt = 0, bd = 0;
    if (lane == 63) {
        if (sl) bl = reserve(0, sl);
        if (sq) bq = reserve(1, sq);
        if (sm) bm = reserve(2, sm);
        if (sk) bk = reserve(3, sk);
        if (sh) bh = reserve(4, sh);
        if (ss) bs = reserve(5, ss);
        if (st) bt = reserve(6, st);
        if (sd) bd = reserve(7, sd);
    }
    bl = __shfl(bl, 63) + sl - nl;
    bq = __shfl(bq, 63) + sq - nq;
    bm = __shfl(bm, 63) + sm - nm;
    bk = __shfl(bk, 63) + sk - nk;
    bh = __shfl(bh, 63) + sh - nh;
    bs = __shfl(bs, 63) + ss - ns;
    bt = __shfl(bt, 63) + st - nt;
    bd = __shfl(bd, 63) + sd - nd;
    if (!hlong) {
        // from the back of the heavy list (mid-length blocks) or of the dense list (the
        // others): entries nmax - 1 - b, nmax - 2 - b, ...
        int2 *const back = hmid ? heavy : dense;
        const int b0 = hmid ? bs : bt;
        for (int q = 0; q < bi.nh; ++q) back[nmax - 1 - (b0 + q)] = make_int2(j, q * kHeavyTile);
        bi.nh = 0;
    }
    if (mid || lsh) {
        // from the back of light_long (mid) or of light (short): entries n - 1 - b, ...
        int4 *const back = mid ? light_long : light;
        const int b0 = mid ? bm : bk;
        for (int q = 0; q < bi.nl; ++q)
            back[nmax - 1 - (b0 + q)] =
                make_int4(sb + q * light_tok, min(light_tok, S - q * light_tok), bi.r0,
                          t < vocab ? bi.d : -1);
        bi.nl = 0;
    }
    write_items(bi, j, sb, S, t < vocab, light_tok, lng ? bq : bl, bh, bd, lng ? light_long : light,
                heavy, dense);
}

// One thread per block (segment): its size, and its work items (block_worklist).
__global__ __launch_bounds__(256) void k_worklist(const int32_t *__restrict__ uniq,
                                                  const int32_t *__restrict__ seg_start,
                                                  int32_t *__restrict__ counts,
                                                  const int64_t *__restrict__ off, int vocab,
                                                  int heavy_min, int dense_min, int light_tok,
                                                  int4 *__restrict__ light,
                                                  int2 *__restrict__ heavy,
                                                  int2 *__restrict__ dense,
                                                  int32_t *__restrict__ hdr,
                                                  int4 *__restrict__ light_long, int nmax) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int m = hdr[HDR_NSEG];
    int S = 0, sb = 0, t = vocab, r0 = 0, d = 0;
    if (j < m) {
        sb = seg_start[j];
        S = seg_start[j + 1] - sb;
        counts[j] = S;
        t = uniq[j];
        if (t < vocab) {
            r0 = (int)off[t];
            d = (int)(off[t + 1] - off[t]);
        }
    }
    block_worklist(j < m, j, sb, S, t, r0, d, vocab, heavy_min, dense_min, light_tok, light, heavy,
                   dense, light_long, nmax,
                   [&](int k, int c) { return atomicAdd(&hdr[list_hdr(k)], c); });
}

// Writes uniq[], seg_start[] and counts[] of the blocks whose heads lie in one tile
// (kSortPer consecutive keys per thread), and with light non-null their work items
// (block_worklist).  The tile's first block index is the sum of the earlier tiles' head
// counts; a block ends at the next head: in the tile (a suffix minimum over the threads'
// first heads), else the first head of a later tile (tile_cnt[ntiles + u]), else n.  The
// number of blocks m goes to *nseg and seg_start[m] = n.
__global__ __launch_bounds__(256) void k_seg_write(const int32_t *__restrict__ sk, int n,
                                                   const int32_t *__restrict__ tile_cnt, int ntiles,
                                                   int32_t *__restrict__ hdr, int vocab,
                                                   int32_t *__restrict__ uniq,
                                                   int32_t *__restrict__ seg_start,
                                                   int32_t *__restrict__ counts,
                                                   const int64_t *__restrict__ off, int heavy_min,
                                                   int dense_min, int light_tok,
                                                   int4 *__restrict__ light, int2 *__restrict__ heavy,
                                                   int2 *__restrict__ dense,
                                                   int4 *__restrict__ light_long) {
    __shared__ int32_t wsum[4], wmin[4];
    __shared__ int32_t tile_sums[3];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // the thread's sorted keys, its heads and their blocks' CSR offsets come first, so
    // these dependent reads overlap the tile sums below
    const int base = blockIdx.x * kSortTile + threadIdx.x * kSortPer;
    int flags = 0, c = 0, mine = n;  // mine: this thread's first head
    int key[kSortPer], r0[kSortPer], drows[kSortPer];
    {
        const int prev = base > 0 && base - 1 < n ? sk[base - 1] : -1;
#pragma unroll
        for (int i = 0; i < kSortPer; ++i) key[i] = base + i < n ? sk[base + i] : vocab;
#pragma unroll
        for (int i = kSortPer - 1; i >= 0; --i) {
            const int s = base + i;
            const int f = (s < n) && (s == 0 || key[i] != (i ? key[i - 1] : prev));
            flags |= f << i;
            c += f;
            if (f) mine = s;
        }
#pragma unroll
        for (int i = 0; i < kSortPer; ++i) {
            const bool h = ((flags >> i) & 1) && key[i] < vocab;
            const int64_t a = h ? off[key[i]] : 0, b = h ? off[key[i] + 1] : 0;
            r0[i] = (int)a;
            drows[i] = (int)(b - a);
        }
    }
    // heads before this tile, all heads, and the first head after it
    int32_t before = 0, total = 0, after = n;
    for (int u = threadIdx.x; u < ntiles; u += 256) {
        const int32_t cu = tile_cnt[u];
        total += cu;
        before += u < (int)blockIdx.x ? cu : 0;
        if (u > (int)blockIdx.x) after = min(after, tile_cnt[ntiles + u]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        before += __shfl_xor(before, o);
        total += __shfl_xor(total, o);
        after = min(after, __shfl_xor(after, o));
    }
    if (lane == 0) {
        wsum[w] = before;
        wmin[w] = after;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        tile_sums[0] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        tile_sums[2] = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    }
    __syncthreads();
    if (lane == 0) wsum[w] = total;
    __syncthreads();
    if (threadIdx.x == 0) tile_sums[1] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    const int32_t tile_off = tile_sums[0], m = tile_sums[1], next_tile_head = tile_sums[2];
    // the first head after this thread's positions: a suffix minimum over the later
    // lanes, then the later wavefronts of the tile, then the later tiles
    int suf = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_down(suf, o);
        if (lane + o < 64) suf = min(suf, u);
    }
    int later = __shfl_down(suf, 1);
    if (lane == 63) later = n;
    if (lane == 0) wmin[w] = suf;
    int32_t all;
    int j = tile_off + block_scan_256(c, wsum, &all);  // (its barriers publish wmin)
    for (int ww = w + 1; ww < 4; ++ww) later = min(later, wmin[ww]);
    later = min(later, next_tile_head);
#pragma unroll
    for (int i = 0; i < kSortPer; ++i) {
        const bool h = (flags >> i) & 1;
        int S = 0;
        if (h) {
            const int s = base + i;
            int e = later;
#pragma unroll
            for (int q = kSortPer - 1; q > i; --q)
                if ((flags >> q) & 1) e = base + q;
            S = e - s;
            uniq[j] = key[i];
            seg_start[j] = s;
            counts[j] = S;
        }
        if (light)
            block_worklist(h, j, base + i, S, key[i], r0[i], drows[i], vocab, heavy_min, dense_min,
                           light_tok, light, heavy, dense, light_long, n,
                           [&](int k, int v) { return atomicAdd(&hdr[list_hdr(k)], v); });
        j += h;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[HDR_NSEG] = m;
        seg_start[min(m, n)] = n;
        // IDs outside [0, vocab) have the key vocab, the largest, so they sort last
        hdr[HDR_ERR] = n > 0 && sk[n - 1] == vocab;
    }
}

// Block-wide exclusive scan over kSmallThreads threads (one int32 each); the total
// goes to *total.  wsum holds kSmallThreads / 64 words.
__device__ inline int32_t block_scan_small(int32_t v, int32_t *wsum, int32_t *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(x, o);
        if (lane >= o) x += u;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t pre = 0, all = 0;
    for (int ww = 0; ww < kSmallThreads / 64; ++ww) {
        pre += ww < w ? wsum[ww] : 0;
        all += wsum[ww];
    }
    *total = all;
    __syncthreads();
    return pre + x - v;
}

// The whole route of a batch of at most kRouteSmallMax tokens in one workgroup (one
// token per thread), for small batches where the multi-kernel route is all launch
// latency.  Same outputs as the multi-kernel route and k_worklist: the header words
// are zeroed here, each key's stable rank is the number of keys that are smaller or
// equal and earlier (every thread compares its key with all keys in LDS), the
// sorted keys give the block heads, and one block scan per list places each
// block's items (in block order).
//
// With SPLIT the work lists are the split-row items instead: block j's rows in
// ceil(d_t / rows) chunks and its tokens in groups of `tokens`, one item per (chunk,
// group), written in block order; blkinfo[j] = {first partial slot, chunks, tokens,
// first sorted position} (slots: chunk-major, one per (chunk, token)); blk_of[p] =
// the block of sorted position p.  IDs outside [0, vocab) get no chunks.
template <bool SPLIT>
__global__ __launch_bounds__(kSmallThreads) void k_route_small(
    const int32_t *__restrict__ ids, int n, int vocab, const int64_t *__restrict__ off, int heavy_min,
    int dense_min, int light_tok, int32_t *__restrict__ hdr, int32_t *__restrict__ sorted,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm, int32_t *__restrict__ uniq,
    int32_t *__restrict__ counts, int32_t *__restrict__ seg_start, int4 *__restrict__ light,
    int2 *__restrict__ heavy, int2 *__restrict__ dense, int4 *__restrict__ sitems,
    int4 *__restrict__ blkinfo, int32_t *__restrict__ blk_of) {
    __shared__ int32_t keys[kRouteSmallMax], skeys[kRouteSmallMax];
    __shared__ int32_t sstart[kRouteSmallMax + 1];
    __shared__ int32_t wsum[kSmallThreads / 64];
    const int i = threadIdx.x;
    if (i < HDR_WORDS) hdr[i] = 0;
    int key = INT32_MAX, bad = 0;
    if (i < n) {
        const int id = ids[i];
        key = (id >= 0 && id < vocab) ? id : vocab;
        bad = key != id;
        keys[i] = key;
    }
    int32_t nbad;
    block_scan_small(bad, wsum, &nbad);  // (its barrier also publishes keys[])
    if (i < n) {
        int r = 0;
        for (int q = 0; q < n; ++q) {
            const int kq = keys[q];
            r += (kq < key) | ((kq == key) & (q < i));
        }
        skeys[r] = key;
        sorted[r] = key;
        perm[r] = i;
        inv_perm[i] = r;
    }
    __syncthreads();
    // blocks: heads of the sorted keys
    const int head = (i < n) && (i == 0 || skeys[i] != skeys[i - 1]);
    int32_t m;
    const int j = block_scan_small(head, wsum, &m);
    if (head) {
        uniq[j] = skeys[i];
        seg_start[j] = i;
        sstart[j] = i;
    }
    if (SPLIT && i < n) blk_of[i] = j + head - 1;
    if (i == 0) {
        sstart[m] = n;
        seg_start[m] = n;
        hdr[HDR_NSEG] = m;
        if (nbad) hdr[HDR_ERR] = 1;
    }
    __syncthreads();
    // work lists: thread i describes block i
    int S = 0, sb = 0, t = vocab;
    if (i < m) {
        sb = sstart[i];
        S = sstart[i + 1] - sb;
        counts[i] = S;
        t = skeys[sb];
    }
    if constexpr (SPLIT) {
        // here heavy_min = rows per chunk, light_tok = tokens per group
        const int rows = heavy_min, tokens = light_tok;
        const int d = (i < m && t < vocab) ? (int)(off[t + 1] - off[t]) : 0;
        const int nc = (d + rows - 1) / rows, ng = (S + tokens - 1) / tokens;
        int32_t ti, ts;
        const int bi0 = block_scan_small(nc * ng, wsum, &ti);
        const int bs0 = block_scan_small(nc * S, wsum, &ts);
        if (i < m) {
            blkinfo[i] = make_int4(bs0, nc, S, sb);
            for (int c = 0; c < nc; ++c)
                for (int g = 0; g < ng; ++g) sitems[bi0 + c * ng + g] = make_int4(i, c, g, 0);
        }
        if (i == 0) hdr[HDR_NSPLIT] = ti;
        return;
    }
    BlockItems bi;
    if (i < m) {
        const bool in = t < vocab;
        bi = block_items(S, t, in ? (int)off[t] : 0, in ? (int)(off[t + 1] - off[t]) : 0, vocab, heavy_min,
                         dense_min, light_tok);
    }
    int32_t tl, th, td;
    const int bl = block_scan_small(bi.nl, wsum, &tl);
    const int bh = block_scan_small(bi.nh, wsum, &th);
    const int bd = block_scan_small(bi.nd, wsum, &td);
    write_items(bi, i, sb, S, t < vocab, light_tok, bl, bh, bd, light, heavy, dense);
    if (i == 0) {
        hdr[HDR_NLIGHT] = tl;
        hdr[HDR_NHEAVY] = th;
        hdr[HDR_NDENSE] = td;
    }
}

inline int blocks_for(int64_t n, int per) { return (int)((n + per - 1) / per); }

}  // namespace

hipError_t launch_zero_i32(int32_t *p, int64_t count, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_i32, dim3(blocks_for(count, 256)), dim3(256), 0, s, p, count);
    return hipGetLastError();
}

hipError_t launch_route(const int32_t *ids, int64_t n64, int64_t vocab, RouteBufs &b, int64_t ntiles,
                        const int64_t *off, int heavy_min_tokens, int dense_min_tokens, int light_tokens,
                        int4 *light, int2 *heavy, int2 *dense, int4 *light_long, hipStream_t s) {
    const int n = (int)n64;
    int bits = 1;
    while ((1ll << bits) <= vocab) ++bits;  // keys lie in [0, vocab]
    const int passes = (bits + kRadixBits - 1) / kRadixBits;
    const int32_t *kin = ids;
    const int32_t *vin = nullptr;
    int32_t *kout = b.keys_a, *vout = b.vals_a;
    for (int p = 0; p < passes; ++p) {
        const int shift = p * kRadixBits;
        const int from_ids = p == 0;
        hipLaunchKernelGGL(k_sort_rank, dim3((unsigned)ntiles), dim3(256), 0, s, kin, n, shift,
                           from_ids, (int)vocab, b.rank, b.hist, (int)ntiles, b.hdr);
        const int ready = ntiles > kScatterDirectTiles;
        if (ready) hipLaunchKernelGGL(k_hist_scan, dim3(kRadix / 4), dim3(256), 0, s, b.hist, (int)ntiles);
        hipLaunchKernelGGL(k_sort_scatter, dim3((unsigned)ntiles), dim3(256), 0, s, kin,
                           vin ? vin : kin, n, shift, from_ids, (int)vocab, b.hist, (int)ntiles, ready,
                           b.rank, kout, vout);
        kin = kout;
        vin = vout;
        kout = (kout == b.keys_a) ? b.keys_b : b.keys_a;
        vout = (vout == b.vals_a) ? b.vals_b : b.vals_a;
    }
    b.sorted_ids = const_cast<int32_t *>(kin);
    b.perm = const_cast<int32_t *>(vin);
    hipLaunchKernelGGL(k_seg_heads, dim3((unsigned)ntiles), dim3(256), 0, s, b.sorted_ids, b.perm,
                       n, (int)ntiles, b.tile_cnt, b.inv_perm);
    hipLaunchKernelGGL(k_seg_write, dim3((unsigned)ntiles), dim3(256), 0, s, b.sorted_ids, n,
                       b.tile_cnt, (int)ntiles, b.hdr, (int)vocab, b.uniq, b.seg_start, b.counts, off,
                       heavy_min_tokens, dense_min_tokens, light_tokens, light, heavy, dense, light_long);
    return hipGetLastError();
}

hipError_t launch_route_small(const int32_t *ids, int64_t n, int64_t vocab, const int64_t *off,
                              int heavy_min_tokens, int dense_min_tokens, int light_tokens, RouteBufs &b,
                              int4 *light, int2 *heavy, int2 *dense, hipStream_t s) {
    if (n <= 0 || n > kRouteSmallMax) return hipErrorInvalidValue;
    b.sorted_ids = b.keys_a;
    b.perm = b.vals_a;
    hipLaunchKernelGGL(k_route_small<false>, dim3(1), dim3(kSmallThreads), 0, s, ids, (int)n, (int)vocab,
                       off, heavy_min_tokens, dense_min_tokens, light_tokens, b.hdr, b.keys_a, b.vals_a,
                       b.inv_perm, b.uniq, b.counts, b.seg_start, light, heavy, dense, (int4 *)nullptr,
                       (int4 *)nullptr, (int32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_route_small_split(const int32_t *ids, int64_t n, int64_t vocab, const int64_t *off,
                                    int rows, int tokens, RouteBufs &b, const SplitLists &sl,
                                    hipStream_t s) {
    if (n <= 0 || n > kRouteSmallMax || rows < 1 || tokens < 1) return hipErrorInvalidValue;
    b.sorted_ids = b.keys_a;
    b.perm = b.vals_a;
    hipLaunchKernelGGL(k_route_small<true>, dim3(1), dim3(kSmallThreads), 0, s, ids, (int)n, (int)vocab,
                       off, rows, 0, tokens, b.hdr, b.keys_a, b.vals_a, b.inv_perm, b.uniq, b.counts,
                       b.seg_start, (int4 *)nullptr, (int2 *)nullptr, (int2 *)nullptr, sl.items,
                       sl.blkinfo, sl.blk_of);
    return hipGetLastError();
}

hipError_t launch_worklist(const RouteBufs &b, int64_t n, const int64_t *off, int64_t vocab,
                           int heavy_min_tokens, int dense_min_tokens, int light_tokens,
                           int4 *light, int2 *heavy, int2 *dense, hipStream_t s, int4 *light_long) {
    hipLaunchKernelGGL(k_worklist, dim3(blocks_for(n, 256)), dim3(256), 0, s, b.uniq, b.seg_start,
                       b.counts, off, (int)vocab, heavy_min_tokens, dense_min_tokens, light_tokens,
                       light, heavy, dense, b.hdr, light_long, (int)n);
    return hipGetLastError();
}

}  // namespace l3
