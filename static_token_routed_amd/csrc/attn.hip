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
#include "l3_internal.h"

namespace l3 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t f2bf(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ inline uint32_t pack2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

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

int attn_heavy_min_tokens(int64_t, int64_t, int, int32_t) { return INT32_MAX; }

hipError_t launch_attn(const AttnArgs &a, int dtype, int use_heavy, hipStream_t s) {
    (void)use_heavy;
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
    const int64_t nci = (a.d_in + 511) / 512;
    if (nci <= 1) return launch_light_nci<1>(la, a.d_emb, s);
    if (nci <= 2) return launch_light_nci<2>(la, a.d_emb, s);
    if (nci <= 4) return launch_light_nci<4>(la, a.d_emb, s);
    if (nci <= 8) return launch_light_nci<8>(la, a.d_emb, s);
    return hipErrorInvalidValue;
}

}  // namespace l3
