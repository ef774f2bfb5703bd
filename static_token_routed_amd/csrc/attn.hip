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
#include "cdna4.h"
#include "l3_internal.h"

namespace l3 {
namespace {

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// VE consecutive bf16 of a d_emb row as fp32 (VE = d_emb / 64).
template <int VE>
__device__ inline void load_v(const uint16_t *p, float (&v)[VE]) {
    if constexpr (VE == 8) {
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
    if constexpr (VE == 8) {
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

struct LightArgs {
    const uint16_t *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    const int2 *items;
    int64_t d_in, d_emb;
    int32_t vocab;
    uint16_t *o;
};

// One item with exactly NT tokens.
template <int NCI, int VE, int NT>
__device__ __forceinline__ void light_item(const LightArgs &a, const int (&tok)[8], int64_t r0,
                                           int64_t d, int lane) {
    const int64_t d_in = a.d_in;
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
    float m[NT], l[NT], acc[NT][VE];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        m[q] = -INFINITY;
        l[q] = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[q][e] = 0.f;
    }
    const uint16_t *kp = a.WK + r0 * d_in + lane * 8;
    const uint16_t *vp = a.WV + r0 * a.d_emb + lane * VE;
    uint4 kv[NCI];
    float vv[VE];
#pragma unroll
    for (int c = 0; c < NCI; ++c)
        kv[c] = (c * 512 + lane * 8 < d_in) ? *reinterpret_cast<const uint4 *>(kp + c * 512)
                                            : make_uint4(0, 0, 0, 0);
    load_v<VE>(vp, vv);
    for (int64_t r = 0; r < d; ++r) {
        // prefetch the next row while this one is reduced
        uint4 kn[NCI];
        float vn[VE];
        if (r + 1 < d) {
            const uint16_t *kq = kp + (r + 1) * d_in;
#pragma unroll
            for (int c = 0; c < NCI; ++c)
                kn[c] = (c * 512 + lane * 8 < d_in) ? *reinterpret_cast<const uint4 *>(kq + c * 512)
                                                    : make_uint4(0, 0, 0, 0);
            load_v<VE>(vp + (r + 1) * a.d_emb, vn);
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
        if (r + 1 < d) {
#pragma unroll
            for (int c = 0; c < NCI; ++c) kv[c] = kn[c];
#pragma unroll
            for (int e = 0; e < VE; ++e) vv[e] = vn[e];
        }
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const float inv = 1.f / l[q];
        float r[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) r[e] = acc[q][e] * inv;
        store_o<VE>(a.o + (int64_t)tok[q] * a.d_emb + lane * VE, r);
    }
}

template <int NCI>
constexpr int light_tokens_for() { return NCI <= 2 ? 8 : (NCI == 4 ? 6 : 3); }

template <int NCI, int VE>
__global__ __launch_bounds__(256) void k_attn_light_bf16(LightArgs a) {
    constexpr int TL = light_tokens_for<NCI>();
    const int lane = threadIdx.x & 63;
    const int nw = gridDim.x * 4;
    const int nitems = a.hdr[HDR_NLIGHT];
    for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < nitems; it += nw) {
        const int2 item = a.items[it];
        const int j = __builtin_amdgcn_readfirstlane(item.x);
        const int c0 = __builtin_amdgcn_readfirstlane(item.y);
        const int sb = a.seg_start[j];
        const int S = a.seg_start[j + 1] - sb;
        const int nt = min(TL, S - c0);
        const int t = a.uniq[j];
        int tok[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) tok[q] = q < nt ? a.perm[sb + c0 + q] : 0;
        if (t >= a.vocab) {  // ID out of range: the flag is set, the row is zeroed
            for (int q = 0; q < nt; ++q) {
                float z[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) z[e] = 0.f;
                store_o<VE>(a.o + (int64_t)tok[q] * a.d_emb + lane * VE, z);
            }
            continue;
        }
        const int64_t r0 = a.off[t];
        const int64_t d = a.off[t + 1] - r0;
        switch (nt) {
            case 1: light_item<NCI, VE, 1>(a, tok, r0, d, lane); break;
            case 2: if constexpr (TL >= 2) light_item<NCI, VE, 2>(a, tok, r0, d, lane); break;
            case 3: if constexpr (TL >= 3) light_item<NCI, VE, 3>(a, tok, r0, d, lane); break;
            case 4: if constexpr (TL >= 4) light_item<NCI, VE, 4>(a, tok, r0, d, lane); break;
            case 5: if constexpr (TL >= 5) light_item<NCI, VE, 5>(a, tok, r0, d, lane); break;
            case 6: if constexpr (TL >= 6) light_item<NCI, VE, 6>(a, tok, r0, d, lane); break;
            case 7: if constexpr (TL >= 7) light_item<NCI, VE, 7>(a, tok, r0, d, lane); break;
            case 8: if constexpr (TL >= 8) light_item<NCI, VE, 8>(a, tok, r0, d, lane); break;
            default: break;
        }
    }
}

// fp32 path: one wavefront per token, any dims.  Scores go to a per-token scratch
// row, then become probabilities, then weigh the V rows (lanes over d_emb).
struct F32Args {
    const float *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    const int2 *items;
    int64_t d_in, d_emb;
    int32_t vocab, max_d;
    float *o, *scores;
};

__global__ __launch_bounds__(256) void k_attn_f32(F32Args a) {
    const int lane = threadIdx.x & 63;
    const int nw = gridDim.x * 4;
    const int nitems = a.hdr[HDR_NLIGHT];
    for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < nitems; it += nw) {
        const int2 item = a.items[it];
        const int j = item.x;
        const int sb = a.seg_start[j];
        const int tok = a.perm[sb + item.y];
        const int t = a.uniq[j];
        float *o = a.o + (int64_t)tok * a.d_emb;
        if (t >= a.vocab) {
            for (int64_t e = lane; e < a.d_emb; e += 64) o[e] = 0.f;
            continue;
        }
        const int64_t r0 = a.off[t];
        const int64_t d = a.off[t + 1] - r0;
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
// One workgroup takes one ID and up to 64 of its tokens; wavefront w owns tokens
// [16w, 16w + 16).
//   scores  S^T (d_t x 16 tokens) = K_t x^T with v_mfma_f32_16x16x32_bf16.  K
//           tiles (128 rows x 64 columns) and the gathered x tiles (64 tokens x
//           64 columns) stream through a 3-stage LDS ring filled by asynchronous
//           global->LDS copies; all d_t <= 512 scores stay in the accumulators,
//           so the softmax is exact (one max, one sum) and no accumulator is
//           rescaled.
//   values  O^T (d_emb x 16 tokens) = V_t^T P^T, the same MFMA, over 32-row
//           stages of V copied row-major into the ring and read transposed with
//           ds_read_b64_tr_b16.
// The MFMA reduction index k maps to rows as k = 8*(lane/16) + j  <->  row
// 4*(lane/16) + j for j < 4, 16 + 4*(lane/16) + (j - 4) for j >= 4: exactly the
// rows whose scores that lane holds in two consecutive 16-row accumulators, so
// P never moves between lanes.  Work items of one ID are consecutive in the
// list; each XCD takes a contiguous eighth of the list, so the tiles of one ID
// mostly share that XCD's L2.
typedef short i16x4_t __attribute__((ext_vector_type(4)));

struct HeavyArgs {
    const uint16_t *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    int32_t *queue;  // 8 per-XCD work counters (zeroed with the header)
    const int2 *items;
    int64_t d_in;
    uint16_t *o;
};

constexpr int QK_RB = 128;                           // K rows per row block
constexpr int QK_KC = 64;                            // d_in columns per scores stage
constexpr int QK_XBYTES = kHeavyTile * QK_KC * 2;    // gathered x tile per stage (8 KB)
constexpr int RING_BYTES = 144 * 1024;
constexpr int PV_ROWS = 64;                          // V rows per values stage
constexpr int QCHUNK = 4;                            // items per round-robin chunk of the XCD queues

// wait until at most N * later copies of this wave are in flight (later <= MAXL)
template <int N, int MAXL>
__device__ inline void wait_upto(int later) {
    if constexpr (MAXL >= 4) { if (later >= 4) { wait_vmcnt<4 * N>(); return; } }
    if constexpr (MAXL >= 3) { if (later == 3) { wait_vmcnt<3 * N>(); return; } }
    if constexpr (MAXL >= 2) { if (later == 2) { wait_vmcnt<2 * N>(); return; } }
    if constexpr (MAXL >= 1) { if (later == 1) { wait_vmcnt<N>(); return; } }
    wait_vmcnt<0>();
}

// One work item with NRB 128-row blocks of K_t (d_t <= 128 * NRB).  Every score and
// value MFMA of the item runs unconditionally: rows past d_t are copies of row
// d_t - 1 whose scores are masked to -inf, so they weigh nothing.
template <int VEB, int NRB>
__device__ __forceinline__ void mfma_item(const HeavyArgs &a, unsigned char *ring, uint32_t ring0,
                                          int sb, int tq, int ntok, int64_t r0, int d) {
    constexpr int DE = VEB * 16;
    constexpr int NPASS = VEB > 16 ? 2 : 1;                  // values passes over halves of d_emb
    constexpr int VEBH = VEB / NPASS;
    constexpr int DEH = VEBH * 16;                           // d_emb columns per pass
    constexpr int CPR = DEH / 8;                             // 16-byte chunks per (half) V row
    constexpr int KBYTES = NRB * QK_RB * QK_KC * 2;          // K tile per scores stage
    constexpr int QSTAGE = KBYTES + QK_XBYTES;
    constexpr int QNS = RING_BYTES / QSTAGE >= 6 ? 6 : RING_BYTES / QSTAGE;  // scores ring depth
    constexpr int QLOADS = QSTAGE / 1024 / 4;                // copies per wave and scores stage
    constexpr int KCOPIES = KBYTES / 1024 / 4;               // ... of which K
    constexpr int V_STAGE = PV_ROWS * DEH * 2;               // bytes per values stage
    constexpr int VNS = RING_BYTES / V_STAGE >= 6 ? 6 : RING_BYTES / V_STAGE;  // values ring depth
    constexpr int V_LOADS = V_STAGE / 1024 / 4;              // copies per wave and values stage
    constexpr int RPC = 1024 / (DEH * 2);                    // V rows per 1 KB copy
    constexpr int NB = 8 * NRB;                              // 16-row score blocks
    constexpr int NPV = (QK_RB / PV_ROWS) * NRB;             // values stages
    static_assert(QNS >= 2 && VNS >= 2 && V_LOADS >= 1, "ring");
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int l16 = lane & 15, kg = lane >> 4, cph = lane & 7;
    const int64_t d_in = a.d_in;
    const int nkc = (int)(d_in / QK_KC);
    const bool active = 16 * w < ntok;

    // x rows (tokens) this lane copies: tile rows 8 * (2w + i) + lane / 8
    int64_t xoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tr = 8 * (2 * w + i) + (lane >> 3);
        xoff[i] = (int64_t)a.perm[sb + tq + min(tr, ntok - 1)] * d_in;
    }
    // stage c: K[all rows][64c, 64c + 64) and x[tokens][same columns]; copy q of
    // the K tile covers tile rows [8q, 8q + 8)
    auto issue_qk = [&](int c) {
        const uint32_t base = ring0 + (uint32_t)((c % QNS) * QSTAGE);
        const int64_t col = (int64_t)c * QK_KC;
#pragma unroll
        for (int i = 0; i < KCOPIES; ++i) {
            const int q = KCOPIES * w + i;
            const int row = 8 * q + (lane >> 3);
            const int64_t grow = r0 + min(row, d - 1);
            async_ld16(a.WK + grow * d_in + col + (cph ^ (row & 7)) * 8, base + q * 1024);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = 2 * w + i;
            const int row = 8 * q + (lane >> 3);
            async_ld16(a.x + xoff[i] + col + (cph ^ (row & 7)) * 8, base + KBYTES + q * 1024);
        }
    };

    f32x4_t Sc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) Sc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < QNS - 1 && i < nkc; ++i) issue_qk(i);
    for (int c = 0; c < nkc; ++c) {
        wait_upto<QLOADS, QNS - 2>(min(QNS - 2, nkc - 1 - c));
        lds_barrier();
        if (c + QNS - 1 < nkc) issue_qk(c + QNS - 1);
        if (active) {
            const uint16_t *kt = reinterpret_cast<const uint16_t *>(ring + (c % QNS) * QSTAGE);
            const uint16_t *xt = kt + KBYTES / 2;
#pragma unroll
            for (int kk = 0; kk < QK_KC / 32; ++kk) {
                const int ch = kk * 4 + kg;
                const int xr = 16 * w + l16;
                const bf16x8_t B = *reinterpret_cast<const bf16x8_t *>(&xt[xr * QK_KC + ((ch ^ (xr & 7)) * 8)]);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int kr = 16 * b + l16;
                    const bf16x8_t A = *reinterpret_cast<const bf16x8_t *>(&kt[kr * QK_KC + ((ch ^ (kr & 7)) * 8)]);
                    Sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, Sc[b], 0, 0, 0);
                    // keep operand reads within a 128-row block (bounds live registers)
                    if ((b & 7) == 7) __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // exact softmax over the d_t rows (lane: token l16, rows 16b + 4kg + i)
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = (16 * b + 4 * kg + i < d) ? Sc[b][i] : -INFINITY;
            Sc[b][i] = v;
            mx = fmaxf(mx, v);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float lsum = 0.f;
    uint4 Pk[NB / 2];
#pragma unroll
    for (int g = 0; g < NB / 2; ++g) {
        float pr[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = __expf(Sc[2 * g][i] - mx);
            pr[4 + i] = __expf(Sc[2 * g + 1][i] - mx);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) lsum += pr[i];
        Pk[g] = make_uint4(pack2(pr[0], pr[1]), pack2(pr[2], pr[3]), pack2(pr[4], pr[5]), pack2(pr[6], pr[7]));
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const float inv = 1.f / lsum;
    const int qi = 16 * w + l16;
    const int tok = qi < ntok ? a.perm[sb + tq + qi] : 0;

    // values stages: rows [64g, 64g + 64) of V_t and columns [hp*DEH, (hp+1)*DEH).
    // A stage is stored as 1 KB blocks of 16 rows x 64 bytes (4 chunks): block
    // (cg, rg) holds chunks [4cg, 4cg + 4) of rows [16rg, 16rg + 16), row-major.  One
    // async copy fills one block (4 lanes per 64-byte row segment).  A transposed
    // read by 16 lanes touches 4 rows x 4 column quads: 32 distinct banks.
    constexpr int NRG = PV_ROWS / 16;  // row groups per stage
    static_assert((CPR / 4) * NRG == V_STAGE / 1024, "values blocks");
    // lane part of the transposed-read address (bytes): row 4kg + l16/4 of a row
    // group, column quad l16 % 4 (two per 16-byte chunk)
    const uint32_t tr_lane = (4 * kg + (l16 >> 2)) * 64 + ((l16 & 3) >> 1) * 16 + (l16 & 1) * 8;
#pragma unroll
    for (int hp = 0; hp < NPASS; ++hp) {
        auto issue_pv = [&](int g) {
            const uint32_t base = ring0 + (uint32_t)((g % VNS) * V_STAGE);
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i) {
                const int q = V_LOADS * w + i;
                const int cg = q / NRG, rg = q % NRG;
                const int row = rg * 16 + (lane >> 2);
                const int64_t grow = r0 + min(PV_ROWS * g + row, d - 1);
                async_ld16(a.WV + grow * DE + hp * DEH + (cg * 4 + (lane & 3)) * 8, base + q * 1024);
            }
        };
        lds_barrier();  // every wave is done with the previous stages in the ring
#pragma unroll
        for (int i = 0; i < VNS - 1 && i < NPV; ++i) issue_pv(i);
        f32x4_t O[VEBH];
#pragma unroll
        for (int e = 0; e < VEBH; ++e) O[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NPV; ++g) {
            wait_upto<V_LOADS, VNS - 2>(min(VNS - 2, NPV - 1 - g));
            lds_barrier();
            if (g + VNS - 1 < NPV) issue_pv(g + VNS - 1);
            if (active) {
#pragma unroll
                for (int ks = 0; ks < PV_ROWS / 32; ++ks) {
                    const unsigned char *vt = ring + (g % VNS) * V_STAGE + tr_lane;
                    const bf16x8_t P = __builtin_bit_cast(bf16x8_t, Pk[g * (PV_ROWS / 32) + ks]);
#pragma unroll
                    for (int eb = 0; eb < VEBH; ++eb) {
                        // rows 32ks + 4kg + e (first read) and 32ks + 16 + 4kg + e (second):
                        // row groups 2ks and 2ks + 1; chunks 2eb, 2eb + 1 (block eb / 2)
                        const int blk_a = (eb >> 1) * NRG + 2 * ks, blk_b = blk_a + 1;
                        const int cofs = (eb & 1) * 32;
                        const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4_t *)(vt + blk_a * 1024 + cofs));
                        const i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4_t *)(vt + blk_b * 1024 + cofs));
                        const uint2 ua = __builtin_bit_cast(uint2, va), ub = __builtin_bit_cast(uint2, vb);
                        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(ua.x, ua.y, ub.x, ub.y));
                        O[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, P, O[eb], 0, 0, 0);
                    }
                }
            }
        }
        if (active && qi < ntok) {
            uint16_t *orow = a.o + (int64_t)tok * DE + hp * DEH + 4 * kg;
#pragma unroll
            for (int eb = 0; eb < VEBH; ++eb) {
                const uint2 u = make_uint2(pack2(O[eb][0] * inv, O[eb][1] * inv),
                                           pack2(O[eb][2] * inv, O[eb][3] * inv));
                *reinterpret_cast<uint2 *>(orow + eb * 16) = u;
            }
        }
    }
    lds_barrier();  // the next item's copies reuse the ring
}

template <int VEB>  // d_emb / 16
__global__ __launch_bounds__(256, 1) void k_attn_mfma(HeavyArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char ring[RING_BYTES];
    __shared__ int s_item;
    const uint32_t ring0 = lds_addr(ring);
    const int nitems = a.hdr[HDR_NHEAVY];
    // The list is cut into chunks of QCHUNK consecutive items dealt round-robin to
    // the 8 XCDs (workgroup id mod 8); the workgroups of one XCD take that XCD's
    // items from its own counter, in order.  Consecutive items (tiles of one ID)
    // share an XCD's L2; every XCD gets a similar mix of large and small IDs.
    const int xcd = blockIdx.x & 7;
    for (;;) {
        if (threadIdx.x == 0) {
            const int n = atomicAdd(&a.queue[xcd], 1);
            const int it = ((n / QCHUNK) * 8 + xcd) * QCHUNK + n % QCHUNK;
            s_item = it < nitems ? it : -1;
        }
        lds_barrier();
        const int it = s_item;
        if (it < 0) break;
        const int2 item = a.items[it];
        const int j = item.x, tq = item.y;
        const int sb = a.seg_start[j];
        const int S = a.seg_start[j + 1] - sb;
        const int ntok = min(kHeavyTile, S - tq);
        const int id = a.uniq[j];
        const int64_t r0 = a.off[id];
        const int d = (int)(a.off[id + 1] - r0);
        switch ((d + QK_RB - 1) / QK_RB) {
            case 1: mfma_item<VEB, 1>(a, ring, ring0, sb, tq, ntok, r0, d); break;
            case 2: mfma_item<VEB, 2>(a, ring, ring0, sb, tq, ntok, r0, d); break;
            case 3: mfma_item<VEB, 3>(a, ring, ring0, sb, tq, ntok, r0, d); break;
            default: mfma_item<VEB, 4>(a, ring, ring0, sb, tq, ntok, r0, d); break;
        }
    }
}

constexpr int kHeavyBlocks = 256;   // one per CU, a multiple of 8 (XCD order)

hipError_t launch_heavy(const HeavyArgs &ha, int64_t d_emb, hipStream_t s) {
    switch (d_emb) {
        case 64: hipLaunchKernelGGL((k_attn_mfma<4>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        case 128: hipLaunchKernelGGL((k_attn_mfma<8>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        case 256: hipLaunchKernelGGL((k_attn_mfma<16>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        case 512: hipLaunchKernelGGL((k_attn_mfma<32>), dim3(kHeavyBlocks), dim3(256), 0, s, ha); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

constexpr int kAttnBlocks = 2048;

template <int NCI>
hipError_t launch_light_nci(const LightArgs &la, int64_t d_emb, hipStream_t s) {
    switch (d_emb / 64) {
        case 1: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 1>), dim3(kAttnBlocks), dim3(256), 0, s, la); break;
        case 2: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 2>), dim3(kAttnBlocks), dim3(256), 0, s, la); break;
        case 4: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 4>), dim3(kAttnBlocks), dim3(256), 0, s, la); break;
        case 8: hipLaunchKernelGGL((k_attn_light_bf16<NCI, 8>), dim3(kAttnBlocks), dim3(256), 0, s, la); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int attn_light_tokens(int64_t d_in, int dtype) {
    if (dtype != L3_BF16) return 1;
    if (d_in <= 1024) return light_tokens_for<2>();
    if (d_in <= 2048) return light_tokens_for<4>();
    return light_tokens_for<8>();
}

int attn_heavy_min_tokens(int64_t, int64_t, int dtype, int32_t) {
    return dtype == L3_BF16 ? kHeavyMinTokens : INT32_MAX;
}

hipError_t launch_attn(const AttnArgs &a, int dtype, int use_heavy, hipStream_t s) {
    if (dtype == L3_F32) {
        F32Args fa{(const float *)a.x, (const float *)a.WK, (const float *)a.WV, a.off, a.uniq,
                   a.seg_start, a.perm, a.hdr, a.light, a.d_in, a.d_emb, (int32_t)a.vocab,
                   a.max_d, (float *)a.o, a.scores};
        hipLaunchKernelGGL(k_attn_f32, dim3(kAttnBlocks), dim3(256), 0, s, fa);
        return hipGetLastError();
    }
    LightArgs la{(const uint16_t *)a.x, (const uint16_t *)a.WK, (const uint16_t *)a.WV, a.off,
                 a.uniq, a.seg_start, a.perm, a.hdr, a.light, a.d_in, a.d_emb, (int32_t)a.vocab,
                 (uint16_t *)a.o};
    if (use_heavy) {
        HeavyArgs ha{(const uint16_t *)a.x, (const uint16_t *)a.WK, (const uint16_t *)a.WV, a.off,
                     a.uniq, a.seg_start, a.perm, a.hdr, a.queue, a.heavy, a.d_in, (uint16_t *)a.o};
        const hipError_t e = launch_heavy(ha, a.d_emb, s);
        if (e != hipSuccess) return e;
    }
    const int64_t nci = (a.d_in + 511) / 512;
    if (nci <= 1) return launch_light_nci<1>(la, a.d_emb, s);
    if (nci <= 2) return launch_light_nci<2>(la, a.d_emb, s);
    if (nci <= 4) return launch_light_nci<4>(la, a.d_emb, s);
    if (nci <= 8) return launch_light_nci<8>(la, a.d_emb, s);
    return hipErrorInvalidValue;
}

}  // namespace l3
