// Gather-attention of the L^3 layer: for every token, softmax(K_t x) over the
// d_t rows its ID selects, then the weighted sum of the same rows of W_V
// ("L^3: Large Lookup Layers": papernotes.org page, section 关键设计 item 1 --
// the token ID picks the embeddings, the hidden state weighs them;
// kimjy99.github.io page, section "Method", the layer equation).
//
// Work comes in items of one distinct ID and a few of its tokens (the batch is
// sorted, so the tokens of an ID are contiguous).  One wavefront per item:
// lane l holds elements [c*512 + 8l, c*512 + 8l + 8) of each d_in vector and
// d_emb/64 consecutive elements of each d_emb vector.  K and V rows are read
// once per item with 16-byte coalesced loads; scores use v_dot2_f32_bf16 (bf16
// pairs, fp32 accumulate) reduced across the wavefront; the softmax over the
// d_t rows is an online (running max / running sum) fp32 softmax, so any d_t
// streams through registers.  The result row goes to the token's original
// batch position, which undoes the sort in the store.
#include <algorithm>
#include <type_traits>

#include "cdna4.h"
#include "l3_internal.h"

namespace l3 {
namespace {

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// v shuffled within each 16-lane row by a DPP control (every source lane is in the row)
template <int CTRL>
__device__ inline float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// Sum over the wavefront (every lane active), the same value in every lane: within each
// 16-lane row by DPP (lane pairs, pairs of pairs, then the half-row and row mirrors;
// each step adds two equal-order partials, so a row's lanes agree bit for bit), then the
// four row sums read from lanes 0, 16, 32, 48 and added in that fixed order.  (Six
// ds_bpermute shuffles per sum kept the wavefront kernel's rows waiting on LDS.)
__device__ inline float wave_sum(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    v += dpp_f32<0x4E>(v);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    v += dpp_f32<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within 8
    v += dpp_f32<0x140>(v);  // row_mirror: lane i <-> 15 - i within 16
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// VE consecutive bf16 of a d_emb row as fp32 (VE = d_emb / 64).
template <int VE>
__device__ inline void load_v(const uint16_t *p, float (&v)[VE]) {
    if constexpr (VE > 8) {
        // VE / 8 consecutive 16-byte pieces (d_emb 1024, 2048)
#pragma unroll
        for (int k = 0; k < VE / 8; ++k) {
            const uint4 u = reinterpret_cast<const uint4 *>(p)[k];
            v[8 * k + 0] = bf_lo(u.x); v[8 * k + 1] = bf_hi(u.x); v[8 * k + 2] = bf_lo(u.y);
            v[8 * k + 3] = bf_hi(u.y); v[8 * k + 4] = bf_lo(u.z); v[8 * k + 5] = bf_hi(u.z);
            v[8 * k + 6] = bf_lo(u.w); v[8 * k + 7] = bf_hi(u.w);
        }
    } else if constexpr (VE == 8) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
        v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
    } else if constexpr (VE == 4) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
    } else if constexpr (VE == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
        v[0] = bf_lo(u); v[1] = bf_hi(u);
    } else {
        v[0] = __uint_as_float((uint32_t)(*p) << 16);
    }
}

template <int VE>
__device__ inline void store_o(uint16_t *p, const float (&v)[VE]) {
    if constexpr (VE > 8) {
#pragma unroll
        for (int k = 0; k < VE / 8; ++k) {
            uint4 u;
            u.x = pack2(v[8 * k + 0], v[8 * k + 1]); u.y = pack2(v[8 * k + 2], v[8 * k + 3]);
            u.z = pack2(v[8 * k + 4], v[8 * k + 5]); u.w = pack2(v[8 * k + 6], v[8 * k + 7]);
            reinterpret_cast<uint4 *>(p)[k] = u;
        }
    } else if constexpr (VE == 8) {
        uint4 u;
        u.x = pack2(v[0], v[1]); u.y = pack2(v[2], v[3]);
        u.z = pack2(v[4], v[5]); u.w = pack2(v[6], v[7]);
        *reinterpret_cast<uint4 *>(p) = u;
    } else if constexpr (VE == 4) {
        uint2 u;
        u.x = pack2(v[0], v[1]); u.y = pack2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(p) = u;
    } else if constexpr (VE == 2) {
        *reinterpret_cast<uint32_t *>(p) = pack2(v[0], v[1]);
    } else {
        *p = (uint16_t)f2bf(v[0]);
    }
}

// A V row slice (VE bf16) kept as loaded and widened to fp32 where it is used.
template <int VE> struct VRawS { uint4 u; };
template <> struct VRawS<4> { uint2 u; };
template <> struct VRawS<2> { uint32_t u; };
template <> struct VRawS<1> { uint16_t u; };

template <int VE>
__device__ inline VRawS<VE> load_vraws(const uint16_t *p) {
    VRawS<VE> r;
    r.u = *reinterpret_cast<const decltype(r.u) *>(p);
    return r;
}

template <int VE>
__device__ inline void vraws_f32(const VRawS<VE> &r, float (&v)[VE]) {
    if constexpr (VE == 8) {
        v[0] = bf_lo(r.u.x); v[1] = bf_hi(r.u.x); v[2] = bf_lo(r.u.y); v[3] = bf_hi(r.u.y);
        v[4] = bf_lo(r.u.z); v[5] = bf_hi(r.u.z); v[6] = bf_lo(r.u.w); v[7] = bf_hi(r.u.w);
    } else if constexpr (VE == 4) {
        v[0] = bf_lo(r.u.x); v[1] = bf_hi(r.u.x); v[2] = bf_lo(r.u.y); v[3] = bf_hi(r.u.y);
    } else if constexpr (VE == 2) {
        v[0] = bf_lo(r.u); v[1] = bf_hi(r.u);
    } else {
        v[0] = __uint_as_float((uint32_t)r.u << 16);
    }
}

struct LightArgs {
    const uint16_t *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    const int4 *items;  // {first sorted position, tokens, first row, d_t (-1: ID out of range)}
    int64_t d_in, d_emb;
    int32_t vocab;
    uint16_t *o;
    const int4 *items_long;  // the same for blocks of >= kLightMidRows rows (taken first)
    int cap;                 // entries of items_long (the batch's tokens)
};

// tokens per light item: as many x rows and output rows as the registers hold (an output
// row takes VE fp32 per lane, 16 or 32 for the tied d_emb 1024 / 2048 tables)
template <int NCI, int VE = 8>
constexpr int light_tokens_for() {
    return VE >= 32 ? 2 : VE >= 16 ? 4 : (NCI <= 2 ? 8 : (NCI == 4 ? 6 : 3));
}

// Light items: one wavefront per item.  The item's K / V rows stream through a
// ring of LR rows of this wavefront's LDS, filled by asynchronous global->LDS
// copies LR - 1 rows ahead, so a wavefront keeps several rows in flight without
// holding them in registers (the kernel is bound by the bytes each CU has in
// flight: a light item's rows are few and their latency is what it waits on).
// A ring slot is NCI 1 KB pieces of the K row (lane l copies bytes [16l, 16l + 16)
// of piece c, which are exactly the columns c*512 + 8l .. + 8 it multiplies) and
// one 1 KB piece of the V row (lanes past the row copy its first bytes again).
// With tied tables (W_V the same buffer as W_K, d_emb = d_in: the pages' tied variant)
// the V row is the K row, whose NCI pieces already hold its d_emb values in order, so no
// V piece is copied and each row enters the CU once (d_emb 1024 and 2048, beyond the
// matrix-core kernel's widths, are tied-only and take this kernel for every block).
constexpr int kLightWaveLds = 20480;  // LDS bytes per wavefront (two workgroups per CU)
template <int NCI>
constexpr int light_ring_rows() {
    return kLightWaveLds / ((NCI + 1) * 1024) < 8 ? kLightWaveLds / ((NCI + 1) * 1024) : 8;
}

// s_waitcnt vmcnt(N * later) for a runtime later in [0, MAXL]
template <int N, int MAXL>
__device__ inline void wait_rows(int later) {
    if constexpr (MAXL > 0) {
        if (later >= MAXL) { wait_vmcnt<N * MAXL>(); return; }
        wait_rows<N, MAXL - 1>(later);
    } else {
        wait_vmcnt<0>();
    }
}

// One light item with exactly NT tokens.  SPLIT = 1: one wavefront takes all its
// rows.  SPLIT = 4: the four wavefronts of the workgroup take rows w, w + 4, ...
// each with its own online softmax, then wavefronts 1..3 leave their partials
// (unnormalised row, running max and sum per token) in their own ring and
// wavefront 0 merges them: M = max_w m_w, o = sum_w e^(m_w - M) acc_w / sum_w
// e^(m_w - M) l_w.  Long items thus run four times as many rows in parallel.
template <int NCI, int VE, int NT, int SPLIT, bool TIED>
__device__ __forceinline__ void light_item(const LightArgs &a, int p0, int64_t r0, int d, int w,
                                           int lane, unsigned char *lds_all) {
    // tied tables: d_emb = d_in, and the row's NCI pieces lie in order in the slot, so
    // the lane's VE values of the V row are read from the K pieces
    static_assert(!TIED || NCI == 1 || VE == 8 * NCI, "tied: d_emb = d_in");
    constexpr int NP = NCI + (TIED ? 0 : 1);  // 1 KB copies per row
    constexpr int LR = light_ring_rows<NCI>();
    constexpr int SLOT = NP * 1024;
    unsigned char *const ring = lds_all + w * kLightWaveLds;
    const uint32_t ring0 = lds_addr(ring);
    const int64_t d_in = a.d_in, d_emb = a.d_emb;
    const int wr = SPLIT == 1 ? 0 : w;                      // this wavefront's first row
    const int nr = wr < d ? (d - wr + SPLIT - 1) / SPLIT : 0;  // and its number of rows
    const int kcol = lane * 8;
    const int vcol = lane * 8 < d_emb ? lane * 8 : 0;
    // local row j of this wavefront is row wr + SPLIT j of the item
    auto issue = [&](int j) {
        const uint32_t slot = ring0 + (uint32_t)((j % LR) * SLOT);
        const int64_t row = r0 + wr + (int64_t)SPLIT * j;
        const uint16_t *krow = a.WK + row * d_in;
        static_for<NCI>([&](auto c) {
            const int64_t col = c * 512 + kcol;
            async_ld16_o_nt<c * 1024>(krow + (col < d_in ? col : 0), slot);
        });
        if constexpr (!TIED) async_ld16_o_nt<NCI * 1024>(a.WV + row * d_emb + vcol, slot);
    };
    // The first rows' copies go out before the tokens' x rows are looked up, so their
    // latency overlaps that of the two dependent reads (positions, then x).
    for (int j = 0; j < LR && j < nr; ++j) issue(j);
    int tok[NT];  // the item's tokens: sorted positions p0 .. p0 + NT - 1
#pragma unroll
    for (int q = 0; q < NT; ++q) tok[q] = a.perm[p0 + q];
    uint4 xv[NT][NCI];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int c = 0; c < NCI; ++c) {
            const int64_t col = c * 512 + lane * 8;
            xv[q][c] = col < d_in
                           ? *reinterpret_cast<const uint4 *>(a.x + (int64_t)tok[q] * d_in + col)
                           : make_uint4(0, 0, 0, 0);
        }
    // Take delivery of x here: the wait also covers the copies issued before it
    // (completions come in issue order; the compiler does not count the copies), which
    // the first row needs anyway, and leaves no x read pending under the waits below.
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
        for (int c = 0; c < NCI; ++c)
            __asm__ volatile("" ::"v"(xv[q][c].x), "v"(xv[q][c].y), "v"(xv[q][c].z), "v"(xv[q][c].w));
    float m[NT], l[NT], acc[NT][VE];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        m[q] = -INFINITY;
        l[q] = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[q][e] = 0.f;
    }
    for (int j = 0; j < nr; ++j) {
        // rows issued after row j: min(nr, j + LR) - j - 1
        wait_rows<NP, LR - 1>(min(nr, j + LR) - j - 1);
        __asm__ volatile("" ::: "memory");
        const unsigned char *sl = ring + (j % LR) * SLOT;
        uint4 kv[NCI];
#pragma unroll
        for (int c = 0; c < NCI; ++c) kv[c] = *reinterpret_cast<const uint4 *>(sl + c * 1024 + lane * 16);
        float vv[VE];
        load_v<VE>(reinterpret_cast<const uint16_t *>(sl + (TIED ? 0 : NCI * 1024)) + lane * VE, vv);
        if (j + LR < nr) {
            // the slot is refilled only after this wavefront's reads of it are done
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __asm__ volatile("" ::: "memory");
            issue(j + LR);
        }
        float s[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            float p = 0.f;
#pragma unroll
            for (int c = 0; c < NCI; ++c) {
                p = dot2(kv[c].x, xv[q][c].x, p);
                p = dot2(kv[c].y, xv[q][c].y, p);
                p = dot2(kv[c].z, xv[q][c].z, p);
                p = dot2(kv[c].w, xv[q][c].w, p);
            }
            s[q] = p;
        }
#pragma unroll
        for (int q = 0; q < NT; ++q) s[q] = wave_sum(s[q]);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const float mn = fmaxf(m[q], s[q]);
            const float al = __expf(m[q] - mn);
            const float p = __expf(s[q] - mn);
            l[q] = fmaf(l[q], al, p);
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[q][e] = fmaf(p, vv[e], acc[q][e] * al);
            m[q] = mn;
        }
    }
    if constexpr (SPLIT == 1) {
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const float inv = 1.f / l[q];
            float r[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) r[e] = acc[q][e] * inv;
            store_o<VE>(a.o + (int64_t)tok[q] * d_emb + lane * VE, r);
        }
        // the ring is reused by the next item's copies only after these reads: every
        // read above was waited for (lgkmcnt) before its value was used
    } else {
        // partials in the wavefront's own ring (every copy into it has been consumed):
        // token q's row at float 64 VE q, then (m, l) pairs after the last row
        constexpr int ML = NT * 64 * VE;
        static_assert((ML + 2 * NT) * 4 <= kLightWaveLds, "merge area");
        if (w > 0) {
            float *pa = reinterpret_cast<float *>(ring);
#pragma unroll
            for (int q = 0; q < NT; ++q) {
#pragma unroll
                for (int e = 0; e < VE; ++e) pa[q * 64 * VE + lane * VE + e] = acc[q][e];
                if (lane == 0) {
                    pa[ML + 2 * q] = m[q];
                    pa[ML + 2 * q + 1] = l[q];
                }
            }
        }
        __syncthreads();
        if (w == 0) {
            // wavefront 0 always holds row 0, so M is finite; a wavefront without rows
            // left m = -inf, l = 0, acc = 0, which weigh nothing
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                float M = m[q];
#pragma unroll
                for (int v = 1; v < 4; ++v)
                    M = fmaxf(M, reinterpret_cast<const float *>(lds_all + v * kLightWaveLds)[ML + 2 * q]);
                const float a0 = __expf(m[q] - M);
                float L = l[q] * a0, r[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) r[e] = acc[q][e] * a0;
#pragma unroll
                for (int v = 1; v < 4; ++v) {
                    const float *pv = reinterpret_cast<const float *>(lds_all + v * kLightWaveLds);
                    const float wv = __expf(pv[ML + 2 * q] - M);
                    L = fmaf(pv[ML + 2 * q + 1], wv, L);
#pragma unroll
                    for (int e = 0; e < VE; ++e) r[e] = fmaf(wv, pv[q * 64 * VE + lane * VE + e], r[e]);
                }
                const float inv = 1.f / L;
#pragma unroll
                for (int e = 0; e < VE; ++e) r[e] *= inv;
                store_o<VE>(a.o + (int64_t)tok[q] * d_emb + lane * VE, r);
            }
        }
        __syncthreads();  // the rings are refilled only after wavefront 0 has read them
    }
}

template <int NCI, int VE, int SPLIT, bool TIED>
__device__ __forceinline__ void light_item_nt(const LightArgs &a, int p0, int64_t r0, int d, int nt,
                                              int w, int lane, unsigned char *lds) {
    constexpr int TL = light_tokens_for<NCI, VE>();
    switch (nt) {
        case 1: light_item<NCI, VE, 1, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 2: if constexpr (TL >= 2) light_item<NCI, VE, 2, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 3: if constexpr (TL >= 3) light_item<NCI, VE, 3, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 4: if constexpr (TL >= 4) light_item<NCI, VE, 4, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 5: if constexpr (TL >= 5) light_item<NCI, VE, 5, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 6: if constexpr (TL >= 6) light_item<NCI, VE, 6, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 7: if constexpr (TL >= 7) light_item<NCI, VE, 7, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        case 8: if constexpr (TL >= 8) light_item<NCI, VE, 8, SPLIT, TIED>(a, p0, r0, d, w, lane, lds); break;
        default: break;
    }
}

// Light items, persistent workgroups (the ones that fit on the chip at once) in two
// phases.  The work list gives the items of blocks with >= kLightLongRows rows, then
// those with >= kLightMidRows (both in items_long), then the rest (items).  Phase 1:
// a workgroup per long item, its four wavefronts splitting the rows.  Phase 2: a
// wavefront per item, each walking its own items without waiting for the others.
// Both hand items out in snake order (index g in even rounds, count - 1 - g in odd
// ones), so the longest start first and each share mixes long and short ones.
// (Handing items out through per-XCD atomic counters measured 2.6 times slower: the
// counters serialise thousands of short items.)
template <int NCI, int VE, bool TIED = false>
__global__ __launch_bounds__(256, 2) void k_attn_light_bf16(LightArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * kLightWaveLds];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nlong = a.items_long ? a.hdr[HDR_NLIGHT_LONG] : 0;
    const int nmid = a.items_long ? a.hdr[HDR_NLIGHT_MID] : 0;
    const int ncoop = nlong + nmid, nfront = ncoop + a.hdr[HDR_NLIGHT];
    const int nitems = nfront + (a.items_long ? a.hdr[HDR_NLIGHT_SHORT] : 0);
    auto item_at = [&](int it) {
        return it < nlong    ? a.items_long[it]
               : it < ncoop  ? a.items_long[a.cap - 1 - (it - nlong)]
               : it < nfront ? a.items[it - ncoop]
                             : a.items[a.cap - 1 - (it - nfront)];
    };
    // Each round reads the next round's entry before running its own item, so the
    // entry's latency hides behind the item.
    const int nb = gridDim.x;
    auto coop_at = [&](int k) { return k * nb + ((k & 1) ? nb - 1 - blockIdx.x : blockIdx.x); };
    int it = coop_at(0);
    int4 item = it < ncoop ? item_at(it) : make_int4(0, 0, 0, 0);
    for (int k = 1; it < ncoop; ++k) {
        const int itn = coop_at(k);
        const int4 next = itn < ncoop ? item_at(itn) : item;
        // a valid ID with >= kLightMidRows rows
        const int p0 = __builtin_amdgcn_readfirstlane(item.x);
        const int nt = __builtin_amdgcn_readfirstlane(item.y);
        light_item_nt<NCI, VE, 4, TIED>(a, p0, __builtin_amdgcn_readfirstlane(item.z),
                                        __builtin_amdgcn_readfirstlane(item.w), nt, w, lane, lds);
        it = itn;
        item = next;
    }
    const int nw = gridDim.x * 4, g = blockIdx.x * 4 + w;
    auto wave_at = [&](int k) { return ncoop + k * nw + ((k & 1) ? nw - 1 - g : g); };
    it = wave_at(0);
    item = it < nitems ? item_at(it) : make_int4(0, 0, 0, 0);
    for (int k = 1; it < nitems; ++k) {
        const int itn = wave_at(k);
        const int4 next = itn < nitems ? item_at(itn) : item;
        const int p0 = __builtin_amdgcn_readfirstlane(item.x);
        const int nt = __builtin_amdgcn_readfirstlane(item.y);
        const int64_t r0 = __builtin_amdgcn_readfirstlane(item.z);
        const int d = __builtin_amdgcn_readfirstlane(item.w);
        if (d < 0) {  // ID out of range: the flag is set, the rows are zeroed
            for (int q = 0; q < nt; ++q) {
                float z[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) z[e] = 0.f;
                store_o<VE>(a.o + (int64_t)a.perm[p0 + q] * a.d_emb + lane * VE, z);
            }
        } else {
            light_item_nt<NCI, VE, 1, TIED>(a, p0, r0, d, nt, w, lane, lds);
        }
        it = itn;
        item = next;
    }
}

// fp32 path: one wavefront per token, any dims.  Scores go to a per-token scratch
// row, then become probabilities, then weigh the V rows (lanes over d_emb).
struct F32Args {
    const float *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    const int4 *items;  // as LightArgs::items, one token each
    int64_t d_in, d_emb;
    int32_t vocab, max_d;
    float *o, *scores;
};

__global__ __launch_bounds__(256) void k_attn_f32(F32Args a) {
    const int lane = threadIdx.x & 63;
    const int nw = gridDim.x * 4;
    const int nitems = a.hdr[HDR_NLIGHT];
    for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < nitems; it += nw) {
        const int4 item = a.items[it];
        const int tok = a.perm[item.x];
        float *o = a.o + (int64_t)tok * a.d_emb;
        if (item.w < 0) {
            for (int64_t e = lane; e < a.d_emb; e += 64) o[e] = 0.f;
            continue;
        }
        const int64_t r0 = item.z;
        const int64_t d = item.w;
        const float *x = a.x + (int64_t)tok * a.d_in;
        float *sc = a.scores + (int64_t)tok * a.max_d;
        float mx = -INFINITY;
        for (int64_t r = 0; r < d; ++r) {
            const float *kr = a.WK + (r0 + r) * a.d_in;
            float p = 0.f;
            for (int64_t c = lane; c < a.d_in; c += 64) p = fmaf(kr[c], x[c], p);
            p = wave_sum(p);
            mx = fmaxf(mx, p);
            if (lane == 0) sc[r] = p;
        }
        __threadfence_block();
        float z = 0.f;
        for (int64_t r = lane; r < d; r += 64) {
            const float e = expf(sc[r] - mx);
            sc[r] = e;
            z += e;
        }
        z = wave_sum(z);
        __threadfence_block();
        const float inv = 1.f / z;
        for (int64_t e = lane; e < a.d_emb; e += 64) {
            float acc = 0.f;
            for (int64_t r = 0; r < d; ++r) acc = fmaf(sc[r], a.WV[(r0 + r) * a.d_emb + e], acc);
            o[e] = acc * inv;
        }
        __threadfence_block();
    }
}

// ---------------------------------------------------------------- MFMA path
//
// Blocks with many tokens, or with many rows (d_t), run on the matrix cores.
// One workgroup takes one ID and up to 32 of its tokens.  Its 4 wavefronts form
// 2 token groups (16 tokens each) x 2 column halves: wavefront (tg, ch) keeps
// x[token][ch half of d_in] of its 16 tokens in registers as MFMA operands and
// produces the ch half of their d_emb outputs.  K_t and V_t stream once, in
// 128-row groups, through a ring of 16 KB LDS stages filled by asynchronous
// global->LDS copies (1 KB contiguous row pieces):
//   scores  partial S^T (16 rows x 16 tokens) over the wavefront's d_in half,
//           v_mfma_f32_16x16x32_bf16, from K stages of 16 rows x 512 columns;
//           the two halves of a token group swap partials through LDS once per
//           group, so both hold the full scores.
//   softmax running max and sum per token, updated once per group (its scores
//           are all in registers); rows past d_t are masked.
//   values  O^T (d_emb half x 16 tokens) += V_t^T P^T, the same MFMA, from V
//           stages of 16 KB (rows x up to 256 columns, row-major) read
//           transposed with ds_read_b64_tr_b16.
// The K and V stages of all groups form one sequence that the copies run ahead
// of by kSlots - 1 stages, so the softmax and the switch between K and V do not
// drain the ring.  The MFMA reduction index k maps to rows as
// k = 8*(lane/16) + j  <->  row 4*(lane/16) + j for j < 4, 16 + 4*(lane/16) +
// (j - 4) for j >= 4: exactly the rows whose scores that lane holds in two
// consecutive 16-row accumulators, so P never moves between lanes.
typedef short i16x4_t __attribute__((ext_vector_type(4)));

struct HeavyArgs {
    const uint16_t *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    int32_t *queue;  // 8 per-XCD work counters, then the dense items' counter (zeroed with the header)
    const int2 *items;   // streaming items (ID block, first token), 32 tokens
    const int2 *dense;   // dense items, 64 tokens, d_t <= 512; taken before the others
    int64_t d_in;
    uint16_t *o;
    int64_t nmax;        // entries of the items and dense arrays (their backs hold streaming
                         // items of the mid-length and of the short blocks)
    int tied;            // W_V is W_K (d_emb = d_in): a K row is read again as a V row
};

constexpr int kSlot = 16384;       // bytes per ring stage
constexpr int kSlots = 8;          // ring depth
constexpr int kXchg = 4 * 64 * 32 * 4;  // score partials of the 4 wavefronts (32 KB)
constexpr int kGroup = 128;        // rows per softmax group
constexpr int kKCols = 512;        // d_in columns per K stage
constexpr int QCHUNK = 4;          // items per round-robin chunk of the XCD queues
static_assert(kHeavyTile == 32, "two 16-token groups per item");

// s_waitcnt vmcnt(N * later) for a runtime later in [0, MAXL]
template <int N, int MAXL>
__device__ inline void wait_stages(int later) {
    if constexpr (MAXL > 0) {
        if (later >= MAXL) { wait_vmcnt<N * MAXL>(); return; }
        wait_stages<N, MAXL - 1>(later);
    } else {
        wait_vmcnt<0>();
    }
}

// s_waitcnt vmcnt(n) for a wave-uniform runtime n in [0, 24] (a larger n waits for
// vmcnt(24), which is always safe: it only waits for more)
__device__ inline void wait_vmcnt_rt(int n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 13: wait_vmcnt<13>(); break;
        case 14: wait_vmcnt<14>(); break;
        case 15: wait_vmcnt<15>(); break;
        case 16: wait_vmcnt<16>(); break;
        case 17: wait_vmcnt<17>(); break;
        case 18: wait_vmcnt<18>(); break;
        case 19: wait_vmcnt<19>(); break;
        case 20: wait_vmcnt<20>(); break;
        case 21: wait_vmcnt<21>(); break;
        case 22: wait_vmcnt<22>(); break;
        case 23: wait_vmcnt<23>(); break;
        case 24: wait_vmcnt<24>(); break;
        case 25: wait_vmcnt<25>(); break;
        case 26: wait_vmcnt<26>(); break;
        case 27: wait_vmcnt<27>(); break;
        case 28: wait_vmcnt<28>(); break;
        case 29: wait_vmcnt<29>(); break;
        case 30: wait_vmcnt<30>(); break;
        case 31: wait_vmcnt<31>(); break;
        default: wait_vmcnt<32>(); break;
    }
}

// Dense work item: one ID with up to 64 tokens (kDenseTile) and d_t <= 512 rows, so
// that the rows of the IDs that fill most of a batch are read once per 64 tokens
// (instead of once per 32).  All d_t scores of a token stay in MFMA accumulators,
// so the softmax is exact.
// Scores: the K rows go through a ring of 4 slots of 32 KB, the copies running 3
// stages ahead, each stage a barrier: for each 64-column chunk of d_in, the rows
// [0, 256) and, when d_t > 256, [256, 512) (128-byte row pieces).  Wavefront w takes
// rows 64w + [0, 64) of each half for all 64 tokens (32 accumulators of
// v_mfma_f32_16x16x32_bf16), so every K fragment is read from LDS once per item (a
// split by tokens would have each wavefront read all of them: LDS reads, not copies
// or MFMAs, bounded that form).  The tokens' x chunks (8 KB; read once per item,
// from HBM) have 4 slots of their own and are copied 3 chunks ahead; the wavefront
// keeps a chunk's x fragments in registers for both halves.
// Softmax: per-token maxima and sums of the four row quarters meet in LDS, and the
// probabilities (bf16, in the MFMA register layout) go through LDS to the wavefront
// that owns the token (tokens 16w + [0, 16)) for the values.
// Values: V rows in blocks of 32 (d_emb 512) or 64 through the same 4-slot ring, read
// transposed; the ring runs on from the scores, so the first two values stages are
// copied during the last scores stages and the exchange uses the two slots the last
// scores stages free.  K row groups wholly past d_t are not copied (their stale scores
// are masked); the waits count the copies each stage actually issued.
template <int XQ, int DE>
__device__ __forceinline__ void dense_item(const HeavyArgs &a, unsigned char *lds, uint32_t lds0,
                                           int sb, int tq, int ntok, int64_t r0, int d, int w) {
    constexpr int64_t d_in = 64 * XQ;
    constexpr int NKC = XQ;                  // 64-column chunks of d_in
    constexpr int SLOT = 256 * 128;          // K stage: 256 rows x 128 bytes (32 KB)
    constexpr int NSLOT = 4;                 // ring slots: copies run NSLOT - 1 stages ahead
    constexpr int XS = 64 * 128;             // x chunk: 64 tokens x 128 bytes
    constexpr int NXS = 4;                   // x slots: chunks run NXS - 1 column chunks ahead
    constexpr int XBASE = NSLOT * SLOT;
    constexpr int VROWS = DE == 512 ? 32 : 64;  // V rows per values stage
    constexpr int VST = VROWS * DE * 2;      // <= 32 KB
    constexpr int VCP = VST / 1024 / 4;      // V copies per wavefront and stage
    constexpr int VKB = VROWS / 32;          // 32-row blocks per values stage
    constexpr int RPC = 512 / DE;            // V rows per 1 KB copy
    constexpr int CPR = DE / 8;              // 16-byte chunks per V row
    constexpr int OE = DE / 16;              // 16-column output blocks
    static_assert(VCP >= 1 && CPR >= 8 && VST <= SLOT && XBASE + NXS * XS <= kSlots * kSlot + kXchg,
                  "stages");
    static_assert(2 * SLOT == 4 * 16 * 64 * 16, "probability exchange: two ring slots");
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, kg = lane >> 4;
    const int nh = d > 256 ? 2 : 1;          // K row halves holding rows below d_t
    const int NK = NKC * nh;                 // scores stages
    const int nvs = (d + VROWS - 1) / VROWS; // values stages

    // every wavefront has read the item index before the LDS is overwritten
    lds_barrier();

    // Copies of a scores stage of half r: K rows 256r + 64w + [8i, 8i + 8) for i < 8
    // (rows past d_t repeat row d_t - 1; groups wholly past it are skipped); of an x
    // chunk: the x rows of tokens [8q, 8q + 8) for q = 2w + i.  Lane l fills chunk
    // l % 8 of row 8q + l / 8 with global chunk (l % 8) ^ (l / 8).
    const int gch = (lane & 7) ^ (lane >> 3);
    uint32_t koff[16];  // [8r + i]
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int row = 256 * (j >> 3) + 64 * w + 8 * (j & 7) + (lane >> 3);
        koff[j] = (uint32_t)(min(row, d - 1) * d_in * 2 + gch * 16);
    }
    const uint16_t *xsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tk = 8 * (2 * w + i) + (lane >> 3);
        xsrc[i] = a.x + (int64_t)a.perm[sb + tq + min(tk, ntok - 1)] * d_in + gch * 8;
    }
    const uint16_t *kbase = a.WK + r0 * d_in;
    // Every item of an ID walks the column chunks in the same order: items of the ID
    // running at once then ask for the same lines at about the same time, and L2 serves
    // them with one fetch (starting each item at another chunk cost 13 % more HBM reads
    // for no gain in time).
    auto colof = [&](int c) { return (int64_t)c * 64; };
    // K copies this wavefront issues for scores stage t (0 past the last)
    auto k_copies = [&](int t) -> int {
        if (t >= NK) return 0;
        const int r = nh == 2 ? (t & 1) : 0;
        return max(0, min(8, (d - 256 * r - 64 * w + 7) / 8));
    };
    // copies of ring stage s: scores stages, then the values stages copied early
    constexpr int VEARLY = NSLOT - 2;
    auto stage_copies = [&](int s) -> int {
        return s < NK ? k_copies(s) : (s - NK < VEARLY && s - NK < nvs ? VCP : 0);
    };
    // x chunk copies issued when scores stage s starts: chunk c(s) + NXS - 1, at the
    // first stage of chunk c(s) (its slot's previous chunk, c(s) - 1, is done by then)
    auto x_copies = [&](int s) -> int {
        if (s < 0 || s >= NK || (nh == 2 && (s & 1))) return 0;
        return (nh == 2 ? s >> 1 : s) + NXS - 1 < NKC ? 2 : 0;
    };
    auto issue_x = [&](int c) {
        const uint32_t xb = lds0 + (uint32_t)(XBASE + (c % NXS) * XS) + 2 * w * 1024;
        static_for<2>([&](auto i) { async_ld16_o_nt<i * 1024>(xsrc[i] + colof(c), xb); });
    };
    auto issue_k = [&](int t) {
        if (t >= NK) return;
        const uint32_t kb = lds0 + (uint32_t)((t % NSLOT) * SLOT) + 8 * w * 1024;
        const int c = nh == 2 ? (t >> 1) : t, r = nh == 2 ? (t & 1) : 0;
        const int64_t col = colof(c);
        if (r == 0) {
            static_for<8>([&](auto i) {
                if (64 * w + 8 * i < d) async_ld16_sbo<i * 1024>(kbase + col, koff[i], kb);
            });
        } else {
            static_for<8>([&](auto i) {
                if (256 + 64 * w + 8 * i < d) async_ld16_sbo<i * 1024>(kbase + col, koff[8 + i], kb);
            });
        }
    };
    // values stage g: rows [VROWS g, +VROWS) (past d_t repeat row d_t - 1) into ring
    // slot (NK + g) mod NSLOT; copy q = VCP w + i holds rows [RPC q, +RPC); chunk c of
    // row r holds global chunk c ^ 2 (r & 3)
    auto issue_v = [&](int g) {
        if (g >= nvs) return;
        const uint32_t vb = lds0 + (uint32_t)(((NK + g) % NSLOT) * SLOT) + VCP * w * 1024;
        static_for<VCP>([&](auto i) {
            const int q = VCP * w + i;
            const int row = RPC * q + lane / CPR;
            const int64_t grow = r0 + min(VROWS * g + row, d - 1);
            const int cc = (lane % CPR) ^ (2 * (row & 3));
            async_ld16_o<i * 1024>(a.WV + grow * DE + 8 * cc, vb);
        });
    };
    auto issue_s = [&](int s) {
        if (s < NK) issue_k(s);
        else if (s - NK < VEARLY) issue_v(s - NK);
    };
    // Issue order: x chunks 0 .. NXS - 2, stages 0 .. NSLOT - 2, then when stage s
    // starts the copies of ring stage s + NSLOT - 1 and (at a chunk's first stage) an x
    // chunk (none once the ring stage is a values one).  Stage t needs its rows (issued
    // when stage t - 3 started) and, at a chunk's first stage, its x chunk: with two
    // stages per chunk issued earlier still, with one right after those rows.  Copies
    // complete in order, so what may still be in flight is everything issued after the
    // later of the two.
    auto enter_k = [&](int t) {
        wait_vmcnt_rt((nh == 2 ? x_copies(t - 3) : 0) + stage_copies(t + 1) + x_copies(t - 2) +
                      stage_copies(t + 2) + x_copies(t - 1));
        lds_barrier();
        issue_s(t + NSLOT - 1);
        if (x_copies(t)) issue_x((nh == 2 ? t >> 1 : t) + NXS - 1);
    };

    // fragment addresses: row (or token) 16b + (l & 15), chunk (4ks + l/16) ^ (l & 7)
    uint32_t fofs[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) fofs[ks] = (uint32_t)l16 * 128 + 16 * ((4 * ks + kg) ^ (lane & 7));

    // S[4r + j][tb]: lane (l16, kg) holds rows 256r + 64w + 16j + 4kg + i of token 16tb + l16
    f32x4_t S[8][4];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) S[rb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < NXS - 1 && c < NKC; ++c) issue_x(c);
#pragma unroll
    for (int t = 0; t < NSLOT - 1; ++t) issue_s(t);
    // One scores stage: the wavefront's 4 row blocks of half H against the 4 token
    // blocks.  The scheduler is told to keep the fragment reads ahead of the MFMAs (by
    // itself it waits for each read right before its MFMA).
    bf16x8_t xr[4][2];
    auto kstage = [&](const unsigned char *st, auto half) {
        constexpr int H = decltype(half)::value;
        bf16x8_t Af[8];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Af[4 * ks + j] = *reinterpret_cast<const bf16x8_t *>(st + (64 * w + 16 * j) * 128 + fofs[ks]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    S[4 * H + j][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[4 * ks + j], xr[tb][ks],
                                                                              S[4 * H + j][tb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // 4 LDS reads
        static_for<4>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // 4 MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        });
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);    // the last 16 MFMAs
    };
    auto xload = [&](int c) {
        const unsigned char *xs = lds + XBASE + (c % NXS) * XS;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                xr[tb][ks] = *reinterpret_cast<const bf16x8_t *>(xs + (16 * tb) * 128 + fofs[ks]);
    };
    if (nh == 2) {
        // both halves of a column chunk in one iteration, so each accumulator has one home
        for (int c = 0; c < NKC; ++c) {
            enter_k(2 * c);
            xload(c);
            kstage(lds + ((2 * c) % NSLOT) * SLOT, std::integral_constant<int, 0>{});
            enter_k(2 * c + 1);
            kstage(lds + ((2 * c + 1) % NSLOT) * SLOT, std::integral_constant<int, 1>{});
        }
    } else {
        for (int c = 0; c < NKC; ++c) {
            enter_k(c);
            xload(c);
            kstage(lds + (c % NSLOT) * SLOT, std::integral_constant<int, 0>{});
        }
    }

    // Exact softmax per token over its d_t rows.  Every scores copy has landed (only
    // the early values stages may be in flight), and after this barrier no wavefront
    // reads a K slot or an x slot again: the slots of the last two scores stages and
    // the x slots hold the exchange until the values loop starts.
    lds_barrier();
    auto rowof = [&](int rb, int i) { return 256 * (rb >> 2) + 64 * w + 16 * (rb & 3) + 4 * kg + i; };
    float *const xm = reinterpret_cast<float *>(lds + XBASE);         // [wavefront][tb][16] maxima
    float *const xs = reinterpret_cast<float *>(lds + XBASE + 1024);  // [wavefront][tb][16] sums
    // probabilities of token block tb: [32-row block][lane], 16 KB
    auto pbt = [&](int tb) {
        return reinterpret_cast<uint4 *>(lds + ((NK + VEARLY + (tb >> 1)) % NSLOT) * SLOT + (tb & 1) * 16384);
    };
    float M[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        float mx = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (rowof(rb, i) < d) mx = fmaxf(mx, S[rb][tb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (kg == 0) xm[(4 * w + tb) * 16 + l16] = mx;
    }
    lds_barrier();
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
        M[tb] = fmaxf(fmaxf(xm[tb * 16 + l16], xm[(4 + tb) * 16 + l16]),
                      fmaxf(xm[(8 + tb) * 16 + l16], xm[(12 + tb) * 16 + l16]));
    // probabilities (bf16, packed as the values' MFMAs take them) of this wavefront's
    // 32-row blocks p = 8r + 2w + q, and their partial sums per token
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        float ls = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int rb = 4 * h + 2 * q;
                float pr[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = rowof(rb, i) < d ? __expf(S[rb][tb][i] - M[tb]) : 0.f;
                    pr[4 + i] = rowof(rb + 1, i) < d ? __expf(S[rb + 1][tb][i] - M[tb]) : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) ls += pr[i];
                pbt(tb)[(8 * h + 2 * w + q) * 64 + lane] =
                    make_uint4(pack2(pr[0], pr[1]), pack2(pr[2], pr[3]), pack2(pr[4], pr[5]), pack2(pr[6], pr[7]));
            }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        if (kg == 0) xs[(4 * w + tb) * 16 + l16] = ls;
    }
    lds_barrier();
    // this wavefront's tokens 16w + l16: all their 32-row blocks, and the total sum
    uint4 Pk[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) Pk[p] = pbt(w)[p * 64 + lane];
    const float inv = 1.f / ((xs[w * 16 + l16] + xs[(4 + w) * 16 + l16]) +
                             (xs[(8 + w) * 16 + l16] + xs[(12 + w) * 16 + l16]));
    lds_barrier();  // the values' copies overwrite the exchange
    // values stages 0 .. VEARLY - 1 are issued; the ring is filled up to NSLOT - 2 ahead
#pragma unroll
    for (int g = VEARLY; g < NSLOT - 1; ++g) issue_v(g);

    // values: O^T (DE x 16 tokens) += V^T P^T per 32-row block kb of each stage
    const int r3 = (l16 >> 2) & 3;
    uint32_t vbase[OE < 4 ? OE : 4];
#pragma unroll
    for (int n = 0; n < (OE < 4 ? OE : 4); ++n)
        vbase[n] = (4 * kg + (l16 >> 2)) * (2 * DE) + 16 * ((l16 & 3) >> 1) + 8 * (l16 & 1) + 32 * (n ^ r3);
    f32x4_t O[OE];
#pragma unroll
    for (int e = 0; e < OE; ++e) O[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < nvs; ++g) {
        wait_vmcnt_rt(VCP * (min(nvs - 1 - g, NSLOT - 2)));
        lds_barrier();
        issue_v(g + NSLOT - 1);
        const unsigned char *vt = lds + ((NK + g) % NSLOT) * SLOT;
#pragma unroll
        for (int kb = 0; kb < VKB; ++kb) {
            // P of rows [32 (VKB g + kb), +32): block VKB g + kb
            uint4 pk = Pk[kb];
#pragma unroll
            for (int gg = 1; gg < 16 / VKB; ++gg)
                if (g == gg) pk = Pk[VKB * gg + kb];
            const bf16x8_t P = __builtin_bit_cast(bf16x8_t, pk);
            // the transposed reads run LV MFMAs ahead (2 reads per MFMA)
            constexpr int LV = OE < 4 ? OE : 4;
            i16x4_t va[OE], vb[OE];
#pragma unroll
            for (int e = 0; e < OE; ++e) {
                const uint32_t pa = vbase[e & 3] + 128 * (e >> 2) + 64 * DE * kb;
                va[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(vt + pa));
                vb[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(vt + pa + 32 * DE));
            }
#pragma unroll
            for (int e = 0; e < OE; ++e) {
                const uint2 ua = __builtin_bit_cast(uint2, va[e]), ub = __builtin_bit_cast(uint2, vb[e]);
                const bf16x8_t Av = __builtin_bit_cast(bf16x8_t, make_uint4(ua.x, ua.y, ub.x, ub.y));
                O[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, P, O[e], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * LV, 0);
            static_for<OE - LV>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            });
            __builtin_amdgcn_sched_group_barrier(0x008, LV, 0);
        }
    }
    const int qi = 16 * w + l16;
    if (qi < ntok) {
        uint16_t *orow = a.o + (int64_t)a.perm[sb + tq + qi] * DE + 4 * kg;
#pragma unroll
        for (int e = 0; e < OE; ++e) {
            const uint2 u = make_uint2(pack2(O[e][0] * inv, O[e][1] * inv), pack2(O[e][2] * inv, O[e][3] * inv));
            *reinterpret_cast<uint2 *>(orow + e * 16) = u;
        }
    }
}

// XQ: x fragments (32 columns each) per lane, d_in = 64 XQ.  Each K stage's 512
// columns (16 fragments; fewer when d_in < 512) are split in two halves of HW
// fragments: half ch holds fragments [ch HW, ch HW + HW) of every stage, so all 4
// wavefronts work on every stage.  DE: d_emb.
template <int XQ, int DE>
__global__ __launch_bounds__(256, 1) void k_attn_mfma(HeavyArgs a) {
    constexpr int DEV = DE < 256 ? DE : 256;  // d_emb columns per V stage
    constexpr int NVH = DE / DEV;             // V stages per row block (column parts)
    constexpr int RV = kSlot / 2 / DEV;       // V rows per stage (32, 64 or 128)
    constexpr int VPG = kGroup / RV;          // V row blocks per full group
    constexpr int OB = DE / 32;               // 16-column output blocks per wavefront
    constexpr int CPR = DEV / 8;              // 16-byte chunks per V stage row
    constexpr int RPC = 64 / CPR;             // V rows per 1 KB copy
    constexpr int64_t d_in = 64 * XQ;
    constexpr int nq = (int)((d_in + kKCols - 1) / kKCols);  // K stages per 16-row block
    constexpr int HW = XQ < 8 ? XQ : 8;       // fragments per wavefront and K stage
    static_assert(CPR >= 8 && RV % 32 == 0 && (NVH == 1 || OB == 2 * (DEV / 32)), "V stage shape");
    static_assert(HW % 2 == 0 && XQ % HW == 0, "K stage split");
    // d_in 4096 (QU): a token's x row is too long for two 16-token groups side by side,
    // so the four wavefronts share one group and each takes a quarter of every K stage
    // (its x fragments: 128 VGPRs, as at d_in 2048) and of the d_emb columns; the
    // item's two groups go one after the other.  Otherwise wavefront w takes group
    // w & 1 and half w >> 1.
    constexpr bool QU = XQ > 32;
    constexpr int HWW = QU ? 4 : HW;      // fragment steps per wavefront and K stage
    constexpr int OBW = QU ? OB / 2 : OB; // 16-column output blocks per wavefront
    constexpr int NXR = QU ? XQ / 2 : XQ; // x fragments per lane
    static_assert(!QU || (XQ == 64 && OBW >= 1), "quarter layout");

    // one 160 KB allocation: the streaming ring, then the score exchange area; the
    // dense path uses it as two 72 KB stages
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[kSlots * kSlot + kXchg];
    unsigned char *const ring = lds_all;
    float *const xchg = reinterpret_cast<float *>(lds_all + kSlots * kSlot);
    int *const s_item = reinterpret_cast<int *>(xchg);  // free between items
    const uint32_t ring0 = lds_addr(ring);
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform (scalar) from here on
    const int tg = QU ? 0 : (w & 1), ch = QU ? w : (w >> 1);
    const int l16 = lane & 15, kg = lane >> 4;
    const int ndense = a.hdr[HDR_NDENSE];
    // streaming items, longest blocks first: those of long blocks from the list's front,
    // then those of mid-length blocks from its back (entry nmax - 1 first), then the
    // others from the back of the dense array
    const int nlong = a.hdr[HDR_NHEAVY];
    const int nmid = nlong + a.hdr[HDR_NHEAVY_SHORT];
    const int nitems = nmid + a.hdr[HDR_NHEAVY_TAIL];
    // The list is cut into chunks of QCHUNK consecutive items dealt round-robin to
    // the 8 XCDs (workgroup id mod 8); the workgroups of one XCD take that XCD's
    // items from its own counter, in order, and once it is empty take the other
    // XCDs' remaining items, so no XCD idles while another still has a queue.
    const int xcd = blockIdx.x & 7;

    // LDS read addresses as per-lane bases plus compile-time offsets.
    // K stage: row r at 1024 r, logical 16-byte chunk c at physical chunk c ^ (r & 7).
    // Fragment step kk reads row l16, chunk 4kk + kg: (4kk + kg) ^ (l16 & 7) =
    // 4 (kk ^ b) + cq with b = bit 2 of l16, cq = (kg ^ l16) & 3; kk ^ b is kk + b for
    // even kk and (kk - 1) + (1 - b) for odd kk.  Half ch starts at step ch HW.
    const int kb2 = (l16 >> 2) & 1, kcq = (kg ^ l16) & 3;
    const uint32_t k_even = l16 * 1024 + 16 * kcq + 64 * kb2 + 64 * HWW * ch;
    const uint32_t k_odd = l16 * 1024 + 16 * kcq + 64 * (1 - kb2) + 64 * HWW * ch;
    // V stage: row r at 2 DEV r, chunk c at physical chunk c ^ 2 (r & 3).  A transposed
    // read for output block E (16 columns) takes row 4kg + l16/4 (+ 32kb, + 16) and
    // column quad l16 % 4: chunk 2E + h, h = (l16 & 3) / 2, byte (l16 & 1) * 8; with
    // r3 = (l16 / 4) & 3 the physical chunk is 2 (E ^ r3) + h.  Blocks E = eb0 + 4m + n
    // (eb0 a multiple of 4, or OB <= 2) sit at vbase[n] + 128 m.
    const int eb0 = NVH == 1 ? ch * OBW : (QU ? (w & 1) * OBW : 0);
    const int r3 = (l16 >> 2) & 3;
    uint32_t vbase[OBW < 4 ? OBW : 4];
#pragma unroll
    for (int n = 0; n < (OBW < 4 ? OBW : 4); ++n)
        vbase[n] = (4 * kg + (l16 >> 2)) * (2 * DEV) + 16 * ((l16 & 3) >> 1) + 8 * (l16 & 1) +
                   32 * ((eb0 + n) ^ r3);

    // dense items first (one shared counter), then the streaming items; the two loops
    // keep the two paths' registers apart
    for (;;) {
        if (t == 0) {
            const int n = atomicAdd(&a.queue[8], 1);
            *s_item = n < ndense ? n : -1;
        }
        lds_barrier();
        const int it = *s_item;
        if (it < 0) break;
        const int2 di = a.dense[it];
        const int dsb = a.seg_start[di.x];
        const int dn = min(kDenseTile, a.seg_start[di.x + 1] - dsb - di.y);
        const int did = a.uniq[di.x];
        const int64_t dr0 = a.off[did];
        dense_item<XQ, DE>(a, ring, ring0, dsb, di.y, dn, dr0, (int)(a.off[did + 1] - dr0), w);
        lds_barrier();  // the next item's copies reuse the LDS and its index slot
    }
    lds_barrier();  // every wavefront has read the last dense index before it is rewritten
    int steal = 0;  // queues found empty so far (thread 0 only): own XCD's first, then the others'
    for (;;) {
        if (t == 0) {
            int it = -1;
            for (; steal < 8; ++steal) {
                const int q = (xcd + steal) & 7;
                const int n = atomicAdd(&a.queue[q], 1);
                const int c = ((n / QCHUNK) * 8 + q) * QCHUNK + n % QCHUNK;
                if (c < nitems) {
                    it = c;
                    break;
                }
            }
            *s_item = it;
        }
        lds_barrier();
        const int it = *s_item;
        if (it < 0) break;
        const int2 item = it < nlong  ? a.items[it]
                          : it < nmid ? a.items[a.nmax - 1 - (it - nlong)]
                                      : a.dense[a.nmax - 1 - (it - nmid)];
        const int j = item.x, tq = item.y;
        const int sb = a.seg_start[j];
        const int ntok = min(kHeavyTile, a.seg_start[j + 1] - sb - tq);
        const int id = a.uniq[j];
        const int64_t r0 = a.off[id];
        const int d = (int)(a.off[id + 1] - r0);
        for (int sub = 0; sub < (QU ? 2 : 1); ++sub) {
        if (QU && 16 * sub >= ntok) break;
        const int grp = QU ? sub : tg;  // this wavefront's 16-token group of the item
        const bool active = 16 * grp < ntok;
        const int qi = 16 * grp + l16;
        const int tok = a.perm[sb + tq + min(qi, ntok - 1)];

        // x fragments: xr[f] = x[tok][32 kc + 8kg, +8) with kc = 16 (f / HWW) + ch HWW + f % HWW
        bf16x8_t xr[NXR];
        if (active) {
            const uint16_t *xp = a.x + (int64_t)tok * d_in + 32 * HWW * ch + 8 * kg;
#pragma unroll
            for (int f = 0; f < NXR; ++f)
                xr[f] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t *>(xp + 32 * (16 * (f / HWW) + f % HWW)));
            // Take delivery of x here, before any copy of this item is in flight: the
            // compiler's own wait for these loads would otherwise be repeated in every
            // group and drain the copy ring (it does not count the asynchronous copies).
#pragma unroll
            for (int f = 0; f < NXR; ++f) __asm__ volatile("" ::"v"(xr[f]));
        }

        // stage sequence: per group, nrb * nq K stages (16-row block major), then
        // ceil(rows / RV) * NVH V stages (row block major).  The copy side walks it
        // with a cursor (rows before the group, phase, block, part).
        const int ng = (d + kGroup - 1) / kGroup;
        const int rows_last = d - kGroup * (ng - 1);
        const int NS = (ng - 1) * (8 * nq + VPG * NVH) + ((rows_last + 15) / 16) * nq +
                       ((rows_last + RV - 1) / RV) * NVH;
        int c_gr = 0, c_v = 0, c_b = 0, c_p = 0;
        auto issue = [&](int st) {
            const uint32_t base = ring0 + (uint32_t)((st % kSlots) * kSlot);
            const int rows_g = min(kGroup, d - c_gr);
            if (!c_v) {
                // K rows [gr + 16b, +16), columns [512p, +512): copy c = row of the block;
                // lane l fills chunk l of the 1 KB row with global chunk l ^ (row & 7)
                static_for<4>([&](auto c) {
                    const int row = 4 * w + c;
                    const int64_t grow = r0 + min(c_gr + 16 * c_b + row, d - 1);
                    int64_t col = (int64_t)kKCols * c_p + 8 * (lane ^ (row & 7));
                    if (col >= d_in) col = 0;  // past d_in: filler, never read
                    // (read once, unless the same row comes back as a V row)
                    if (a.tied) async_ld16_o<c * 1024>(a.WK + grow * d_in + col, base + 4 * w * 1024);
                    else async_ld16_o_nt<c * 1024>(a.WK + grow * d_in + col, base + 4 * w * 1024);
                });
                if (++c_p == nq) {
                    c_p = 0;
                    if (16 * ++c_b >= rows_g) { c_b = 0; c_v = 1; }
                }
            } else {
                // V rows [gr + RV b, +RV), columns [DEV p, +DEV): copy cp holds rows
                // [RPC cp, +RPC); chunk c of row r holds global chunk c ^ 2(r & 3)
                static_for<4>([&](auto c) {
                    const int cp = 4 * w + c;
                    const int row = cp * RPC + lane / CPR;
                    const int64_t grow = r0 + min(c_gr + RV * c_b + row, d - 1);
                    const int cc = (lane % CPR) ^ (2 * (row & 3));
                    async_ld16_o_nt<c * 1024>(a.WV + grow * DE + DEV * c_p + 8 * cc, base + 4 * w * 1024);
                });
                if (++c_p == NVH) {
                    c_p = 0;
                    if (RV * ++c_b >= rows_g) { c_b = 0; c_v = 0; c_gr += kGroup; }
                }
            }
        };
        int st = 0;
        for (int i = 0; i < kSlots - 1 && i < NS; ++i) issue(i);
        // wait for stage st, then refill the slot every wave has finished with
        auto next_stage = [&]() -> uint32_t {
            wait_stages<4, kSlots - 2>(min(kSlots - 2, NS - 1 - st));
            lds_barrier();
            if (st + kSlots - 1 < NS) issue(st + kSlots - 1);
            const uint32_t p = (uint32_t)((st % kSlots) * kSlot);
            ++st;
            return p;
        };
        auto lds16 = [&](uint32_t byte) {
            return *reinterpret_cast<const bf16x8_t *>(ring + byte);
        };

        float m_run = -INFINITY, l_run = 0.f;
        f32x4_t O[OBW];
#pragma unroll
        for (int e = 0; e < OBW; ++e) O[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        f32x4_t *const xw = reinterpret_cast<f32x4_t *>(xchg) + w * 8 * 64 + lane;
        const f32x4_t *const xo = reinterpret_cast<const f32x4_t *>(xchg) + (w ^ 2) * 8 * 64 + lane;
        for (int g = 0; g < ng; ++g) {
            const int rows_g = g == ng - 1 ? rows_last : kGroup;
            const int nrb = (rows_g + 15) / 16;
            // scores of one 16-row block per iteration (two accumulator chains, even and
            // odd fragment steps); the partial goes to this wavefront's exchange slot
            for (int rb = 0; rb < nrb; ++rb) {
                f32x4_t S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < nq; ++q) {
                    const uint32_t kt = next_stage();
                    if (active) {
                        bf16x8_t A[HWW];
#pragma unroll
                        for (int i = 0; i < HWW; ++i)
                            A[i] = lds16(kt + ((i & 1) ? k_odd + 64 * (i - 1) : k_even + 64 * i));
#pragma unroll
                        for (int i = 0; i < HWW; i += 2) {
                            S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], xr[q * HWW + i], S0, 0, 0, 0);
                            S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i + 1], xr[q * HWW + i + 1], S1, 0, 0, 0);
                        }
                        // keep LK fragment reads ahead of the MFMAs (by itself the
                        // scheduler waits for each read right before its MFMA)
                        constexpr int LK = HWW < 4 ? HWW : 4;
                        __builtin_amdgcn_sched_group_barrier(0x100, LK, 0);
                        static_for<HWW - LK>([&](auto) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        });
                        __builtin_amdgcn_sched_group_barrier(0x008, LK, 0);
                    }
                }
                xw[rb * 64] = S0 + S1;
            }

            // full scores: own partial plus the other column half's (row blocks past
            // the group's rows are masked below, whatever their slots hold)
            lds_barrier();
            f32x4_t Sc[8];
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                if constexpr (QU) {
                    // the four quarters' partials, added in the same order by every wavefront
                    const f32x4_t *const x0 = reinterpret_cast<const f32x4_t *>(xchg) + lane + rb * 64;
                    Sc[rb] = ((x0[0] + x0[8 * 64]) + x0[16 * 64]) + x0[24 * 64];
                } else {
                    Sc[rb] = xw[rb * 64] + xo[rb * 64];
                }
            }

            // online softmax: lane holds rows 128g + 16rb + 4kg + i of token l16
            float gm = -INFINITY;
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = (16 * rb + 4 * kg + i < rows_g) ? Sc[rb][i] : -INFINITY;
                    Sc[rb][i] = v;
                    gm = fmaxf(gm, v);
                }
            gm = fmaxf(gm, __shfl_xor(gm, 16));
            gm = fmaxf(gm, __shfl_xor(gm, 32));
            const float mn = fmaxf(m_run, gm);
            const float al = __expf(m_run - mn);
            m_run = mn;
#pragma unroll
            for (int e = 0; e < OBW; ++e) O[e] *= al;
            float ls = 0.f;
            uint4 Pk[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float pr[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = __expf(Sc[2 * p][i] - mn);
                    pr[4 + i] = __expf(Sc[2 * p + 1][i] - mn);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) ls += pr[i];
                Pk[p] = make_uint4(pack2(pr[0], pr[1]), pack2(pr[2], pr[3]), pack2(pr[4], pr[5]),
                                   pack2(pr[6], pr[7]));
            }
            ls += __shfl_xor(ls, 16);
            ls += __shfl_xor(ls, 32);
            l_run = fmaf(l_run, al, ls);

            // values: V stage (vr, vh) holds rows [RV vr, +RV) of the group, row-major.
            // With two V stages per row block (d_emb 512) half ch takes stage vh = ch
            // whole; otherwise it takes blocks [ch OB, +OB) of each.
            const int nvr = (rows_g + RV - 1) / RV;
            for (int vr = 0; vr < nvr; ++vr) {
#pragma unroll
                for (int vh = 0; vh < NVH; ++vh) {
                    const uint32_t vt = next_stage();
                    if (active && (NVH == 1 || vh == (QU ? (w >> 1) : ch))) {
#pragma unroll
                        for (int kb = 0; kb < RV / 32; ++kb) {
                            // P of rows [32 (vr RV/32 + kb), +32) of the group
                            uint4 pk = Pk[kb];
                            if constexpr (RV / 32 < 4) {
#pragma unroll
                                for (int p = 1; p < 4 * 32 / RV; ++p)
                                    if (vr == p) pk = Pk[p * (RV / 32) + kb];
                            }
                            const bf16x8_t P = __builtin_bit_cast(bf16x8_t, pk);
                            // rows 32kb + 4kg + l16/4 (first read) and 16 rows further
                            // (second); the reads run LV MFMAs ahead
                            constexpr int LV = OBW < 3 ? OBW : 3;
                            i16x4_t va[OBW], vb[OBW];
#pragma unroll
                            for (int e = 0; e < OBW; ++e) {
                                const uint32_t pa = vt + vbase[e & 3] + 128 * (e >> 2) + 64 * DEV * kb;
                                va[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                    (__attribute__((address_space(3))) i16x4_t *)(ring + pa));
                                vb[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                    (__attribute__((address_space(3))) i16x4_t *)(ring + pa + 32 * DEV));
                            }
#pragma unroll
                            for (int e = 0; e < OBW; ++e) {
                                const uint2 ua = __builtin_bit_cast(uint2, va[e]), ub = __builtin_bit_cast(uint2, vb[e]);
                                const bf16x8_t Av = __builtin_bit_cast(bf16x8_t, make_uint4(ua.x, ua.y, ub.x, ub.y));
                                O[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, P, O[e], 0, 0, 0);
                            }
                            __builtin_amdgcn_sched_group_barrier(0x100, 2 * LV, 0);
                            static_for<OBW - LV>([&](auto) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                            });
                            __builtin_amdgcn_sched_group_barrier(0x008, LV, 0);
                        }
                    }
                }
            }
        }

        if (active && qi < ntok) {
            const float inv = 1.f / l_run;
            uint16_t *orow = a.o + (int64_t)tok * DE + 16 * OBW * ch + 4 * kg;
#pragma unroll
            for (int e = 0; e < OBW; ++e) {
                const uint2 u = make_uint2(pack2(O[e][0] * inv, O[e][1] * inv),
                                           pack2(O[e][2] * inv, O[e][3] * inv));
                *reinterpret_cast<uint2 *>(orow + e * 16) = u;
            }
        }
        lds_barrier();  // the next group's or item's copies reuse the ring and s_item
        }
    }
}

constexpr int kHeavyBlocks = 256;   // one per CU, a multiple of 8 (XCD order)

template <int XQ>
hipError_t launch_heavy_xq(const HeavyArgs &ha, int64_t d_emb, hipStream_t s) {
    switch (d_emb) {
        case 64: hipLaunchKernelGGL((k_attn_mfma<XQ, 64>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        case 128: hipLaunchKernelGGL((k_attn_mfma<XQ, 128>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        case 256: hipLaunchKernelGGL((k_attn_mfma<XQ, 256>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        case 512: hipLaunchKernelGGL((k_attn_mfma<XQ, 512>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// d_in widths of the matrix-core kernel's two-group streaming items (each token's x
// row held in registers); the dense items (x streamed through LDS) and the quarter
// layout of the streaming items also take d_in 4096
bool heavy_d_in(int64_t d_in) {
    return d_in == 128 || d_in == 256 || d_in == 512 || d_in == 1024 || d_in == 2048;
}

hipError_t launch_heavy(const HeavyArgs &ha, int64_t d_emb, hipStream_t s) {
    switch (ha.d_in) {
        case 128: return launch_heavy_xq<2>(ha, d_emb, s);
        case 256: return launch_heavy_xq<4>(ha, d_emb, s);
        case 512: return launch_heavy_xq<8>(ha, d_emb, s);
        case 1024: return launch_heavy_xq<16>(ha, d_emb, s);
        case 2048: return launch_heavy_xq<32>(ha, d_emb, s);
        case 4096: return launch_heavy_xq<64>(ha, d_emb, s);
        default: return hipErrorInvalidValue;
    }
}

constexpr int kAttnBlocks = 4096;  // fp32 path: enough wavefronts for one token each at 32768 tokens
// Light kernel: persistent, the workgroups that fit on the chip at once (two per CU:
// 80 KB of LDS rings each)
constexpr int kLightBlocks = 512;

template <int NCI>
hipError_t launch_light_nci(const LightArgs &la, int64_t d_emb, hipStream_t s) {
    // tied tables of d_emb = d_in = 1024, 2048 (only tied: the wavefront kernel is the one
    // gather path for them)
    if constexpr (NCI == 2 || NCI == 4) {
        if (la.WK == la.WV && la.d_in == d_emb && d_emb == 512 * NCI) {
            hipLaunchKernelGGL((k_attn_light_bf16<NCI, 8 * NCI, true>), dim3(kLightBlocks), dim3(256), 0, s,
                               la);
            return hipGetLastError();
        }
    }
    if constexpr (NCI == 1) {
        // tied tables: one copy per row serves both roles
        if (la.WK == la.WV && la.d_in == d_emb) {
            switch (d_emb / 64) {
                case 1: hipLaunchKernelGGL((k_attn_light_bf16<1, 1, true>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
                case 2: hipLaunchKernelGGL((k_attn_light_bf16<1, 2, true>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
                case 4: hipLaunchKernelGGL((k_attn_light_bf16<1, 4, true>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
                case 8: hipLaunchKernelGGL((k_attn_light_bf16<1, 8, true>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    }
    switch (d_emb / 64) {
        case 1: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 1>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
        case 2: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 2>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
        case 4: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 4>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
        case 8: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 8>), dim3(kLightBlocks), dim3(256), 0, s, la); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------- small batches
// Split-row gather-attention.  With few tokens per block, the per-block paths
// above are one long row chain per wavefront or workgroup and the batch's time is
// that chain's latency.  Here every block's rows are cut into chunks of RC rows
// (RC d_in = 8192 columns, so a chunk's K and V rows fit in registers at once)
// and its tokens into groups of TG; one wavefront per (chunk, group) item loads
// the whole chunk and the group's x rows in one go, forms the scores (v_dot2,
// wavefront sums), and stores for each token the chunk's softmax partial: the
// max m_c, the sum l_c of exp(s - m_c) and the fp32 row sum_r exp(s_r - m_c) V_r.
// A second kernel, one wavefront per token, merges its block's chunks in chunk
// order with a running max (o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c,
// M = max_c m_c).  The result is the same softmax, summed in another order.
// d_in / 512 rounded up to the slice counts the kernels are built for (1, 2, 4, 8)
inline int64_t next_pow2_nci(int64_t d_in) {
    const int64_t nci = (d_in + 511) / 512;
    return nci <= 1 ? 1 : (nci <= 2 ? 2 : (nci <= 4 ? 4 : 8));
}
template <int NCI> constexpr int split_rc() { return 16 / NCI; }
template <int NCI> constexpr int split_tg() { return NCI <= 2 ? 4 : (NCI == 4 ? 2 : 1); }

template <int NCI, int VE>
__global__ __launch_bounds__(256) void k_attn_split(SplitArgs a) {
    constexpr int RC = split_rc<NCI>(), TG = split_tg<NCI>();
    const int lane = threadIdx.x & 63;
    const int nitems = a.hdr[HDR_NSPLIT];
    const int64_t d_in = a.d_in, d_emb = a.d_emb;
    const uint16_t *X = static_cast<const uint16_t *>(a.x);
    const uint16_t *WK = static_cast<const uint16_t *>(a.WK);
    const uint16_t *WV = static_cast<const uint16_t *>(a.WV);
    for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < nitems; it += gridDim.x * 4) {
        const int4 item = a.items[it];
        const int j = __builtin_amdgcn_readfirstlane(item.x);
        const int c = __builtin_amdgcn_readfirstlane(item.y);
        const int g = __builtin_amdgcn_readfirstlane(item.z);
        const int4 bi = a.blkinfo[j];
        const int slot0 = __builtin_amdgcn_readfirstlane(bi.x);
        const int S = __builtin_amdgcn_readfirstlane(bi.z);
        const int sb = __builtin_amdgcn_readfirstlane(bi.w);
        const int id = __builtin_amdgcn_readfirstlane(a.uniq[j]);
        const int64_t r0 = a.off[id];
        const int d = (int)(a.off[id + 1] - r0);
        const int rb = c * RC, nr = min(RC, d - rb);
        const int k0 = g * TG, nt = min(TG, S - k0);
        // every load first (tokens and rows past the item's repeat its last one)
        uint4 xv[TG][NCI], kr[RC][NCI];
        VRawS<VE> vr[RC];
#pragma unroll
        for (int q = 0; q < TG; ++q) {
            const int tok = a.perm[sb + k0 + min(q, nt - 1)];
#pragma unroll
            for (int cc = 0; cc < NCI; ++cc) {
                const int64_t col = cc * 512 + lane * 8;
                xv[q][cc] = col < d_in ? *reinterpret_cast<const uint4 *>(X + (int64_t)tok * d_in + col)
                                       : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < RC; ++r) {
            const int64_t row = r0 + rb + min(r, nr - 1);
#pragma unroll
            for (int cc = 0; cc < NCI; ++cc) {
                const int64_t col = cc * 512 + lane * 8;
                kr[r][cc] = col < d_in ? *reinterpret_cast<const uint4 *>(WK + row * d_in + col)
                                       : make_uint4(0, 0, 0, 0);
            }
            vr[r] = load_vraws<VE>(WV + row * d_emb + lane * VE);
        }
        float sc[TG][RC];
#pragma unroll
        for (int q = 0; q < TG; ++q)
#pragma unroll
            for (int r = 0; r < RC; ++r) {
                float p = 0.f;
#pragma unroll
                for (int cc = 0; cc < NCI; ++cc) {
                    p = dot2(kr[r][cc].x, xv[q][cc].x, p);
                    p = dot2(kr[r][cc].y, xv[q][cc].y, p);
                    p = dot2(kr[r][cc].z, xv[q][cc].z, p);
                    p = dot2(kr[r][cc].w, xv[q][cc].w, p);
                }
                sc[q][r] = wave_sum(p);
            }
#pragma unroll
        for (int q = 0; q < TG; ++q) {
            if (q >= nt) break;
            float m = -INFINITY;
#pragma unroll
            for (int r = 0; r < RC; ++r)
                if (r < nr) m = fmaxf(m, sc[q][r]);
            float l = 0.f, acc[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
            for (int r = 0; r < RC; ++r) {
                if (r >= nr) break;
                const float p = __expf(sc[q][r] - m);
                l += p;
                float v[VE];
                vraws_f32<VE>(vr[r], v);
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[e] = fmaf(p, v[e], acc[e]);
            }
            const int64_t slot = slot0 + (int64_t)c * S + k0 + q;
            float *dst = a.po + slot * d_emb + lane * VE;
#pragma unroll
            for (int e = 0; e < VE; ++e) dst[e] = acc[e];
            if (lane == 0) a.pml[slot] = make_float2(m, l);
        }
    }
}

constexpr int kMergeU = 4;  // chunks whose partials are loaded together in the merge

template <int VE>
__global__ __launch_bounds__(256) void k_attn_merge(SplitArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t d_emb = a.d_emb;
    uint16_t *O = static_cast<uint16_t *>(a.o);
    for (int p = blockIdx.x * 4 + (threadIdx.x >> 6); p < a.n; p += gridDim.x * 4) {
        const int j = __builtin_amdgcn_readfirstlane(a.blk_of[p]);
        const int4 bi = a.blkinfo[j];
        const int slot0 = __builtin_amdgcn_readfirstlane(bi.x);
        const int nc = __builtin_amdgcn_readfirstlane(bi.y);
        const int S = __builtin_amdgcn_readfirstlane(bi.z);
        const int k = p - __builtin_amdgcn_readfirstlane(bi.w);
        float res[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) res[e] = 0.f;
        if (nc > 0) {  // else an ID outside [0, vocab): its row is zero (the flag is set)
            // one pass with a running max, kMergeU chunks' loads in flight at a time
            // (chunks past nc re-read the last one and are skipped)
            float M = -INFINITY, L = 0.f;
            for (int c0 = 0; c0 < nc; c0 += kMergeU) {
                float2 ml[kMergeU];
                float src[kMergeU][VE];
#pragma unroll
                for (int u = 0; u < kMergeU; ++u) {
                    const int64_t slot = slot0 + (int64_t)min(c0 + u, nc - 1) * S + k;
                    ml[u] = a.pml[slot];
#pragma unroll
                    for (int e = 0; e < VE; ++e) src[u][e] = a.po[slot * d_emb + lane * VE + e];
                }
#pragma unroll
                for (int u = 0; u < kMergeU; ++u) {
                    if (c0 + u >= nc) break;
                    const float mn = fmaxf(M, ml[u].x);
                    const float al = __expf(M - mn), w = __expf(ml[u].x - mn);
                    L = fmaf(L, al, ml[u].y * w);
#pragma unroll
                    for (int e = 0; e < VE; ++e) res[e] = fmaf(w, src[u][e], res[e] * al);
                    M = mn;
                }
            }
            const float inv = 1.f / L;
#pragma unroll
            for (int e = 0; e < VE; ++e) res[e] *= inv;
        }
        store_o<VE>(O + (int64_t)a.perm[p] * d_emb + lane * VE, res);
    }
}

template <int NCI>
hipError_t launch_split_nci(const SplitArgs &sa, int64_t d_emb, int nblocks, hipStream_t s) {
    switch (d_emb / 64) {
        case 1: hipLaunchKernelGGL((k_attn_split<NCI, 1>), dim3(nblocks), dim3(256), 0, s, sa); break;
        case 2: hipLaunchKernelGGL((k_attn_split<NCI, 2>), dim3(nblocks), dim3(256), 0, s, sa); break;
        case 4: hipLaunchKernelGGL((k_attn_split<NCI, 4>), dim3(nblocks), dim3(256), 0, s, sa); break;
        case 8: hipLaunchKernelGGL((k_attn_split<NCI, 8>), dim3(nblocks), dim3(256), 0, s, sa); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int attn_light_tokens(int64_t d_in, int64_t d_emb, int dtype) {
    if (dtype != L3_BF16) return 1;
    if (d_emb == 2048) return light_tokens_for<4, 32>();  // tied d_in = d_emb tables
    if (d_emb == 1024) return light_tokens_for<2, 16>();
    if (d_in <= 1024) return light_tokens_for<2>();
    if (d_in <= 2048) return light_tokens_for<4>();
    return light_tokens_for<8>();
}

int attn_dense_min_tokens(int64_t d_in, int64_t d_emb, int dtype) {
    return dtype == L3_BF16 && d_emb <= 512 && (heavy_d_in(d_in) || d_in == 4096) ? kDenseMinTokens
                                                                                  : INT32_MAX;
}

int attn_heavy_min_tokens(int64_t d_in, int64_t d_emb, int dtype, int32_t) {
    // Streaming items also at d_in 4096 (the quarter layout).  There an item's two
    // 16-token groups run one after the other, so blocks of few rows stay with the
    // wavefront kernel unless they have many tokens.  The matrix-core kernel holds
    // d_emb up to 512 (wider tied tables take the wavefront kernel only).
    if (dtype != L3_BF16 || d_emb > 512) return INT32_MAX;
    if (heavy_d_in(d_in)) return kHeavyMinTokens;
    return d_in == 4096 ? kHeavyMinTokensWide : INT32_MAX;
}

hipError_t launch_attn_heavy(const AttnArgs &a, hipStream_t s) {
    HeavyArgs ha{(const uint16_t *)a.x, (const uint16_t *)a.WK, (const uint16_t *)a.WV, a.off,
                 a.uniq, a.seg_start, a.perm, a.hdr, a.queue, a.heavy, a.dense, a.d_in,
                 (uint16_t *)a.o, a.n, a.WK == a.WV && a.d_in == a.d_emb};
    return launch_heavy(ha, a.d_emb, s);
}

int split_rows(int64_t d_in) { return 16 / (int)std::min<int64_t>(8, next_pow2_nci(d_in)); }
int split_tokens(int64_t d_in) {
    const int64_t nci = next_pow2_nci(d_in);
    return nci <= 2 ? 4 : (nci == 4 ? 2 : 1);
}

int64_t split_slots(const Dims &d, int64_t n, int32_t max_d) {
    if (d.dtype != L3_BF16 || n < 1 || n > kSplitMaxN || d.d_in > 4096) return 0;
    if (d.d_emb != 64 && d.d_emb != 128 && d.d_emb != 256 && d.d_emb != 512) return 0;
    const int rc = split_rows(d.d_in);
    const int64_t slots = n * ((std::max<int64_t>(max_d, 1) + rc - 1) / rc);
    return slots <= kSplitMaxSlots ? slots : 0;
}

hipError_t launch_attn_split(const SplitArgs &sa, hipStream_t s) {
    // items: at most one per (chunk, token); a grid of up to 1024 workgroups strides over them
    const int64_t nci = next_pow2_nci(sa.d_in);
    const int nblocks = 1024;
    hipError_t e;
    if (nci <= 1) e = launch_split_nci<1>(sa, sa.d_emb, nblocks, s);
    else if (nci <= 2) e = launch_split_nci<2>(sa, sa.d_emb, nblocks, s);
    else if (nci <= 4) e = launch_split_nci<4>(sa, sa.d_emb, nblocks, s);
    else e = launch_split_nci<8>(sa, sa.d_emb, nblocks, s);
    if (e != hipSuccess) return e;
    const int mb = (int)std::min<int64_t>((sa.n + 3) / 4, 1024);
    switch (sa.d_emb / 64) {
        case 1: hipLaunchKernelGGL((k_attn_merge<1>), dim3(mb), dim3(256), 0, s, sa); break;
        case 2: hipLaunchKernelGGL((k_attn_merge<2>), dim3(mb), dim3(256), 0, s, sa); break;
        case 4: hipLaunchKernelGGL((k_attn_merge<4>), dim3(mb), dim3(256), 0, s, sa); break;
        case 8: hipLaunchKernelGGL((k_attn_merge<8>), dim3(mb), dim3(256), 0, s, sa); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_light(const AttnArgs &a, int dtype, hipStream_t s) {
    if (dtype == L3_F32) {
        F32Args fa{(const float *)a.x, (const float *)a.WK, (const float *)a.WV, a.off, a.uniq,
                   a.seg_start, a.perm, a.hdr, a.light, a.d_in, a.d_emb, (int32_t)a.vocab,
                   a.max_d, (float *)a.o, a.scores};
        hipLaunchKernelGGL(k_attn_f32, dim3(kAttnBlocks), dim3(256), 0, s, fa);
        return hipGetLastError();
    }
    LightArgs la{(const uint16_t *)a.x, (const uint16_t *)a.WK, (const uint16_t *)a.WV, a.off,
                 a.uniq, a.seg_start, a.perm, a.hdr, a.light, a.d_in, a.d_emb, (int32_t)a.vocab,
                 (uint16_t *)a.o, a.light_long, (int)a.n};
    const int64_t nci = (a.d_in + 511) / 512;
    if (nci <= 1) return launch_light_nci<1>(la, a.d_emb, s);
    if (nci <= 2) return launch_light_nci<2>(la, a.d_emb, s);
    if (nci <= 4) return launch_light_nci<4>(la, a.d_emb, s);
    if (nci <= 8) return launch_light_nci<8>(la, a.d_emb, s);
    return hipErrorInvalidValue;
}

}  // namespace l3
