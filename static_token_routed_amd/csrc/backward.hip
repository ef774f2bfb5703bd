// Backward pass of the L^3 layer ("L^3: Large Lookup Layers": the layer equation
// on the papernotes.org page, section 整体框架, and the kimjy99.github.io page,
// section "Method"; the pages train it end to end after sorting the batch by
// token ID -- sciencestack.ai page, Fig. 3 caption; kimjy99.github.io page,
// section "2. Efficient Training and Inference").  The gradients are the plain
// derivatives of the forward steps, taken in reverse order:
//   out = W_mix [y ; x]:  dW_mix += dout [y ; x]^T,  dy = W1^T dout,  dx = W2^T dout
//   y = yhat * gamma + beta:  dgamma += dy * yhat,  dbeta += dy
//   yhat = (h - mean) rstd:  dh = rstd (g - mean(g) - yhat mean(g yhat)),  g = dy * gamma
//   h = W_up o:  dW_up += dh o^T,  do = W_up^T dh
//   o = V_t^T p, p = softmax(K_t x):  dp_j = <V_t[j], do>,  ds_j = p_j (dp_j - <o, do>),
//                                     dV_t[j] += p_j do,  dK_t[j] += ds_j x,  dx += K_t^T ds
// The dense products run on the library's GEMMs (explicit transposes feed them
// k-contiguous operands); this file holds the transposes, the LayerNorm backward,
// the per-token attention backward and the per-block key / value gradients.
// Parameter gradients are fp32 and accumulated (+=), in a fixed order (no atomics):
// the batch is sorted by ID, so each table row's gradient is one workgroup's sum
// over its block's tokens.
#include <algorithm>

#include "cdna4.h"
#include "l3_internal.h"

namespace l3 {
namespace {

template <typename T> __device__ inline float ld(const T *p);
template <> __device__ inline float ld<float>(const float *p) { return *p; }
template <> __device__ inline float ld<uint16_t>(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
template <typename T> __device__ inline void st(T *p, float v);
template <> __device__ inline void st<float>(float *p, float v) { *p = v; }
template <> __device__ inline void st<uint16_t>(uint16_t *p, float v) { *p = (uint16_t)f2bf(v); }

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// dst[c][r] = src[r][c] for r < rows, 0 for rows <= r < rows_pad (dst row stride
// ld_dst); 64 x 64 tiles through LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T *__restrict__ src, int64_t ld_src,
                                                   int64_t rows, int64_t cols, T *__restrict__ dst,
                                                   int64_t ld_dst, int64_t rows_pad) {
    __shared__ T tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        T v{};
        if (r < rows && c < cols) v = src[r * ld_src + c];
        tile[i][tx] = v;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows_pad) dst[c * ld_dst + r] = tile[tx][i];
    }
}

// The same for bf16 with 16-byte loads and stores (8 elements per thread and step):
// rows of the source tile go to LDS whole, and each thread gathers 8 consecutive
// source rows of one column into a 16-byte piece of a destination row.  Needs
// 16-byte aligned bases and row strides that are multiples of 8 (checked by the
// launcher).
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t *__restrict__ src, int64_t ld_src,
                                                        int64_t rows, int64_t cols,
                                                        uint16_t *__restrict__ dst, int64_t ld_dst,
                                                        int64_t rows_pad) {
    constexpr int TS = 72;  // LDS row stride (elements): 144 bytes keeps 16-byte alignment
    __shared__ __attribute__((aligned(16))) uint16_t tile[64 * TS];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    for (int q = threadIdx.x; q < 512; q += 256) {
        const int i = q >> 3, ch = q & 7;  // tile row i, columns 8 ch .. 8 ch + 7
        const int64_t r = r0 + i, c = c0 + 8 * ch;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < rows) {
            const uint16_t *sp = src + r * ld_src + c;
            if (c + 8 <= cols) {
                v = *reinterpret_cast<const uint4 *>(sp);
            } else {
                uint16_t e[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) e[k] = c + k < cols ? sp[k] : (uint16_t)0;
                v = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                               e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
            }
        }
        *reinterpret_cast<uint4 *>(&tile[i * TS + 8 * ch]) = v;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 512; q += 256) {
        const int j = q >> 3, ch = q & 7;  // destination row c0 + j, source rows 8 ch .. 8 ch + 7
        const int64_t c = c0 + j, r = r0 + 8 * ch;
        if (c >= cols || r >= rows_pad) continue;
        uint16_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = tile[(8 * ch + k) * TS + j];
        uint16_t *dp = dst + c * ld_dst + r;
        if (r + 8 <= rows_pad) {
            *reinterpret_cast<uint4 *>(dp) = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                                                         e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (r + k < rows_pad) dp[k] = e[k];
        }
    }
}

// One wavefront per row: g = dy * gamma, dh = rstd (g - mean(g) - yhat mean(g yhat)),
// and y = yhat * gamma + beta (the W_mix operand of dW_mix).
template <typename T>
__global__ __launch_bounds__(256) void k_ln_bwd(const T *__restrict__ h, const float *__restrict__ stats,
                                                const float *__restrict__ gamma,
                                                const float *__restrict__ beta,
                                                const float *__restrict__ dy, int64_t n, int64_t d_up,
                                                T *__restrict__ dh, T *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const float mean = stats[2 * row], rstd = stats[2 * row + 1];
    const T *hr = h + row * d_up;
    const float *gr = dy + row * d_up;
    float sg = 0.f, sgy = 0.f;
    for (int64_t c = lane; c < d_up; c += 64) {
        const float yh = (ld(hr + c) - mean) * rstd, g = gr[c] * gamma[c];
        sg += g;
        sgy += g * yh;
    }
    sg = wave_sum(sg) / (float)d_up;
    sgy = wave_sum(sgy) / (float)d_up;
    for (int64_t c = lane; c < d_up; c += 64) {
        const float yh = (ld(hr + c) - mean) * rstd, g = gr[c] * gamma[c];
        st(dh + row * d_up + c, rstd * (g - sg - yh * sgy));
        st(y + row * d_up + c, yh * gamma[c] + beta[c]);
    }
}

// Column partial sums of dy * yhat and dy over a chunk of kLnRows rows:
// part[chunk][c] = (sum dy*yhat, sum dy).
constexpr int kLnRows = 64;

// Both of the above in one pass for bf16 plans with d_up = 512 NCH (NCH 1, 2, 4): a workgroup per
// chunk of kLnRows rows, 16 consecutive rows per wavefront, lane l holding columns
// 512 i + 8 l .. + 7 of the row (h and dy read once, kept in registers).  The
// column partials are summed over each wavefront's rows in order, then over the 4
// wavefronts in order (through LDS), and written per chunk as k_ln_param_part does.
template <int NCH>
__global__ __launch_bounds__(256) void k_ln_bwd_bf16(const uint16_t *__restrict__ h,
                                                     const float *__restrict__ stats,
                                                     const float *__restrict__ gamma,
                                                     const float *__restrict__ beta,
                                                     const float *__restrict__ dy, int64_t n,
                                                     uint16_t *__restrict__ dh, uint16_t *__restrict__ y,
                                                     float2 *__restrict__ part) {
    constexpr int d_up = 512 * NCH;
    static_assert(kLnRows == 64, "16 rows per wavefront");
    __shared__ __attribute__((aligned(16))) float2 red[4][d_up];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float pa[NCH][8], pb[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) pa[c][e] = pb[c][e] = 0.f;
    const int64_t r0 = (int64_t)blockIdx.x * kLnRows + 16 * w;
    for (int i = 0; i < 16; ++i) {
        const int64_t row = r0 + i;
        if (row >= n) break;
        const float mean = stats[2 * row], rstd = stats[2 * row + 1];
        float yh[NCH][8], g[NCH][8];
        float sg = 0.f, sgy = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t col = 512 * c + 8 * lane;
            const uint4 hv = *reinterpret_cast<const uint4 *>(h + row * d_up + col);
            const float4 d0 = *reinterpret_cast<const float4 *>(dy + row * d_up + col);
            const float4 d1 = *reinterpret_cast<const float4 *>(dy + row * d_up + col + 4);
            const float4 g0 = *reinterpret_cast<const float4 *>(gamma + col);
            const float4 g1 = *reinterpret_cast<const float4 *>(gamma + col + 4);
            const float hf[8] = {bf_lo(hv.x), bf_hi(hv.x), bf_lo(hv.y), bf_hi(hv.y),
                                 bf_lo(hv.z), bf_hi(hv.z), bf_lo(hv.w), bf_hi(hv.w)};
            const float df[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            const float gf[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                yh[c][e] = (hf[e] - mean) * rstd;
                g[c][e] = df[e] * gf[e];
                sg += g[c][e];
                sgy += g[c][e] * yh[c][e];
                pa[c][e] += df[e] * yh[c][e];
                pb[c][e] += df[e];
            }
        }
        sg = wave_sum(sg) / (float)d_up;
        sgy = wave_sum(sgy) / (float)d_up;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t col = 512 * c + 8 * lane;
            const float4 g0 = *reinterpret_cast<const float4 *>(gamma + col);
            const float4 g1 = *reinterpret_cast<const float4 *>(gamma + col + 4);
            const float4 b0 = *reinterpret_cast<const float4 *>(beta + col);
            const float4 b1 = *reinterpret_cast<const float4 *>(beta + col + 4);
            const float gf[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float bf[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            float o[8], yo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = rstd * (g[c][e] - sg - yh[c][e] * sgy);
                yo[e] = yh[c][e] * gf[e] + bf[e];
            }
            *reinterpret_cast<uint4 *>(dh + row * d_up + col) =
                make_uint4(pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7]));
            *reinterpret_cast<uint4 *>(y + row * d_up + col) =
                make_uint4(pack2(yo[0], yo[1]), pack2(yo[2], yo[3]), pack2(yo[4], yo[5]), pack2(yo[6], yo[7]));
        }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[w][512 * c + 8 * lane + e] = make_float2(pa[c][e], pb[c][e]);
    __syncthreads();
    for (int q = threadIdx.x; q < d_up; q += 256) {
        float2 v = red[0][q];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            v.x += red[ww][q].x;
            v.y += red[ww][q].y;
        }
        part[(int64_t)blockIdx.x * d_up + q] = v;
    }
}
template <typename T>
__global__ __launch_bounds__(256) void k_ln_param_part(const T *__restrict__ h,
                                                       const float *__restrict__ stats,
                                                       const float *__restrict__ dy, int64_t n,
                                                       int64_t d_up, float2 *__restrict__ part) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= d_up) return;
    const int64_t r0 = (int64_t)blockIdx.y * kLnRows, r1 = std::min<int64_t>(r0 + kLnRows, n);
    float a = 0.f, b = 0.f;
    for (int64_t r = r0; r < r1; ++r) {
        const float g = dy[r * d_up + c];
        a += g * (ld(h + r * d_up + c) - stats[2 * r]) * stats[2 * r + 1];
        b += g;
    }
    part[blockIdx.y * d_up + c] = make_float2(a, b);
}

// dgamma[c] += sum over chunks of part.x, dbeta[c] += of part.y, in a fixed order:
// 16 columns per workgroup, 16 threads per column each summing a contiguous range
// of chunks in chunk order, then the 16 range sums added in range order.
__global__ __launch_bounds__(256) void k_ln_param_reduce(const float2 *__restrict__ part, int nchunk,
                                                         int64_t d_up, float *__restrict__ dgamma,
                                                         float *__restrict__ dbeta) {
    __shared__ float2 red[16][16];
    const int cl = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int64_t c = (int64_t)blockIdx.x * 16 + cl;
    const int per = (nchunk + 15) / 16, k0 = g * per, k1 = min(nchunk, k0 + per);
    float a = 0.f, b = 0.f;
    if (c < d_up) {
#pragma unroll 8
        for (int k = k0; k < k1; ++k) {
            const float2 v = part[k * d_up + c];
            a += v.x;
            b += v.y;
        }
    }
    red[g][cl] = make_float2(a, b);
    __syncthreads();
    if (g == 0 && c < d_up) {
        float2 t = red[0][cl];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            t.x += red[i][cl].x;
            t.y += red[i][cl].y;
        }
        dgamma[c] += t.x;
        dbeta[c] += t.y;
    }
}

// 16-byte chunk c (elements CH c .. CH c + CH - 1) of a row, as floats.
template <typename T, int CH>
__device__ inline void load_chunk(const T *row, int64_t c, float (&v)[CH]) {
    if constexpr (sizeof(T) == 2 && CH == 8) {
        const uint4 u = *reinterpret_cast<const uint4 *>(row + c * 8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else if constexpr (sizeof(T) == 4 && CH == 4) {
        const float4 f = *reinterpret_cast<const float4 *>(row + c * 4);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
#pragma unroll
        for (int e = 0; e < CH; ++e) v[e] = ld(row + c * CH + e);
    }
}

// One wavefront per work item: up to TB tokens of one block (sorted positions
// s0 .. s0 + cnt - 1), the block's rows r0 .. r0 + d - 1.  Lane l holds 16-byte
// chunks l, l + 64, ... of each row (NI chunks of d_in, NE of d_emb).  Pass 1 over
// the rows: scores, running max and sum, and o = V_t^T p, giving <o, do> per
// token.  Pass 2: p_j, dp_j = <V_t[j], do>, ds_j, dx += ds_j K_t[j] (the K row is
// still in registers from the score), and P, dS stored per sorted position for
// the key / value gradients.  Every row is read once per pass for all TB tokens.
template <typename T, int CH, int NI, int NE, int TB>
__global__ __launch_bounds__(256) void k_attn_bwd(const T *__restrict__ x, const T *__restrict__ WK,
                                                  const T *__restrict__ WV,
                                                  const int32_t *__restrict__ perm,
                                                  const int4 *__restrict__ items,
                                                  const int32_t *__restrict__ hdr,
                                                  const float *__restrict__ dov, int64_t d_in,
                                                  int64_t d_emb, int max_d, float *__restrict__ dx,
                                                  float *__restrict__ P, float *__restrict__ dS) {
    const int lane = threadIdx.x & 63;
    const int nitems = hdr[HDR_NLIGHT];
    const int nw = gridDim.x * 4;
    const int64_t ci = d_in / CH, ce = d_emb / CH;  // chunks per row
    for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < nitems; it += nw) {
        const int4 item = items[it];
        if (item.w < 0) continue;  // ID out of range: no gradient (flagged by the route)
        const int s0 = item.x, cnt = item.y;
        const int64_t r0 = item.z;
        const int d = item.w;
        int tok[TB];
        float xv[TB][NI][CH], dxv[TB][NI][CH], dv[TB][NE][CH], ov[TB][NE][CH];
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            tok[b] = b < cnt ? perm[s0 + b] : perm[s0];
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const int64_t c = lane + 64 * q;
                if (c < ci) load_chunk<T, CH>(x + (int64_t)tok[b] * d_in, c, xv[b][q]);
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    if (c >= ci) xv[b][q][e] = 0.f;
                    dxv[b][q][e] = 0.f;
                }
            }
#pragma unroll
            for (int q = 0; q < NE; ++q) {
                const int64_t c = lane + 64 * q;
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    dv[b][q][e] = c < ce ? dov[(int64_t)tok[b] * d_emb + c * CH + e] : 0.f;
                    ov[b][q][e] = 0.f;
                }
            }
        }
        // the K row's chunks, and the TB scores against it
        auto krow = [&](int j, float (&kv)[NI][CH], float (&sc)[TB]) {
            const T *kr = WK + (r0 + j) * d_in;
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const int64_t c = lane + 64 * q;
                if (c < ci) load_chunk<T, CH>(kr, c, kv[q]);
                else
#pragma unroll
                    for (int e = 0; e < CH; ++e) kv[q][e] = 0.f;
            }
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                float a = 0.f;
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int e = 0; e < CH; ++e) a = fmaf(kv[q][e], xv[b][q][e], a);
                sc[b] = a;
            }
#pragma unroll
            for (int b = 0; b < TB; ++b) sc[b] = wave_sum(sc[b]);
        };
        auto vrow = [&](int j, float (&vv)[NE][CH]) {
            const T *vr = WV + (r0 + j) * d_emb;
#pragma unroll
            for (int q = 0; q < NE; ++q) {
                const int64_t c = lane + 64 * q;
                if (c < ce) load_chunk<T, CH>(vr, c, vv[q]);
                else
#pragma unroll
                    for (int e = 0; e < CH; ++e) vv[q][e] = 0.f;
            }
        };
        // pass 1: max, sum, o
        float m[TB], l[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) { m[b] = -INFINITY; l[b] = 0.f; }
        for (int j = 0; j < d; ++j) {
            float kv[NI][CH], sc[TB], vv[NE][CH];
            krow(j, kv, sc);
            vrow(j, vv);
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                const float mn = fmaxf(m[b], sc[b]), alpha = __expf(m[b] - mn), e = __expf(sc[b] - mn);
                l[b] = l[b] * alpha + e;
                m[b] = mn;
#pragma unroll
                for (int q = 0; q < NE; ++q)
#pragma unroll
                    for (int c = 0; c < CH; ++c) ov[b][q][c] = fmaf(e, vv[q][c], ov[b][q][c] * alpha);
            }
        }
        float inv[TB], od[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            inv[b] = 1.f / l[b];
            float a = 0.f;
#pragma unroll
            for (int q = 0; q < NE; ++q)
#pragma unroll
                for (int c = 0; c < CH; ++c) a = fmaf(ov[b][q][c] * inv[b], dv[b][q][c], a);
            od[b] = a;
        }
#pragma unroll
        for (int b = 0; b < TB; ++b) od[b] = wave_sum(od[b]);
        // pass 2
        for (int j = 0; j < d; ++j) {
            float kv[NI][CH], sc[TB], vv[NE][CH], dp[TB];
            krow(j, kv, sc);
            vrow(j, vv);
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                float a = 0.f;
#pragma unroll
                for (int q = 0; q < NE; ++q)
#pragma unroll
                    for (int c = 0; c < CH; ++c) a = fmaf(vv[q][c], dv[b][q][c], a);
                dp[b] = a;
            }
#pragma unroll
            for (int b = 0; b < TB; ++b) dp[b] = wave_sum(dp[b]);
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                const float p = __expf(sc[b] - m[b]) * inv[b], ds = p * (dp[b] - od[b]);
#pragma unroll
                for (int q = 0; q < NI; ++q)
#pragma unroll
                    for (int c = 0; c < CH; ++c) dxv[b][q][c] = fmaf(ds, kv[q][c], dxv[b][q][c]);
                if (lane == 0 && b < cnt) {
                    P[(int64_t)(s0 + b) * max_d + j] = p;
                    dS[(int64_t)(s0 + b) * max_d + j] = ds;
                }
            }
        }
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            if (b >= cnt) break;
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                const int64_t c = lane + 64 * q;
                if (c < ci) {
                    float *dst = dx + (int64_t)tok[b] * d_in + c * CH;
#pragma unroll
                    for (int e = 0; e < CH; ++e) dst[e] += dxv[b][q][e];
                }
            }
        }
    }
}

// Work items of the key / value gradients: (block, 16-row tile) pairs, appended
// one thread per block (the order of items does not affect the results: each item
// owns its rows' gradients outright).
constexpr int kKvRows = 16;
constexpr int kKvTok = 32;
__global__ __launch_bounds__(256) void k_kv_items(const int64_t *__restrict__ off,
                                                  const int32_t *__restrict__ uniq,
                                                  int32_t *__restrict__ hdr, int64_t vocab,
                                                  int2 *__restrict__ items, int cap) {
    const int m = hdr[HDR_NSEG];
    for (int b = blockIdx.x * 256 + threadIdx.x; b < m; b += gridDim.x * 256) {
        const int t = uniq[b];
        if (t < 0 || t >= vocab) continue;
        const int d = (int)(off[t + 1] - off[t]);
        const int nt = (d + kKvRows - 1) / kKvRows;
        const int at = atomicAdd(&hdr[HDR_NKV], nt);
        for (int r = 0; r < nt && at + r < cap; ++r) items[at + r] = make_int2(b, r * kKvRows);
    }
}

// One workgroup per item: rows j0 .. j0+15 of block b, every column of K (d_in) and V
// (d_emb).  Thread t owns one 16-byte chunk of columns per pass (CH elements of x for
// K, 4 floats of do for V).  For each chunk of 32 tokens (sorted order) the workgroup
// stages their dS and P values for the 16 rows and their token indices in LDS;
// each thread then adds dS * x (K) or P * do (V) over the chunk into 16 x CH
// accumulators: one vector load feeds 16 CH multiply-adds.
template <typename T, int CH>
__global__ __launch_bounds__(256) void k_kv_grad(const T *__restrict__ x, const int64_t *__restrict__ off,
                                                 const int32_t *__restrict__ uniq,
                                                 const int32_t *__restrict__ seg_start,
                                                 const int32_t *__restrict__ perm,
                                                 const int32_t *__restrict__ hdr,
                                                 const int2 *__restrict__ items, int cap,
                                                 const float *__restrict__ dov, int64_t d_in,
                                                 int64_t d_emb, int max_d,
                                                 const float *__restrict__ P,
                                                 const float *__restrict__ dS,
                                                 float *__restrict__ dWK, float *__restrict__ dWV) {
    __shared__ float sds[kKvTok][kKvRows], sp[kKvTok][kKvRows];
    __shared__ int stok[kKvTok];
    constexpr int CV = CH == 8 ? 4 : CH;  // floats of do per chunk
    const int nitems = min(hdr[HDR_NKV], cap);
    const int64_t ck = d_in / CH, cv = d_emb / CV;  // chunks per row
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        const int2 item = items[it];
        const int t = uniq[item.x];
        const int64_t r0 = off[t];
        const int d = (int)(off[t + 1] - r0), j0 = item.y;
        const int nr = min(kKvRows, d - j0);
        const int s0 = seg_start[item.x], s1 = seg_start[item.x + 1];
        // passes of 256 chunks: first the K chunks, then the V chunks
        for (int64_t cb = 0; cb < ck + cv; cb += 256) {
            const int64_t c = cb + threadIdx.x;
            const bool isk = c < ck, live = c < ck + cv;
            float acc[kKvRows][CH];
#pragma unroll
            for (int r = 0; r < kKvRows; ++r)
#pragma unroll
                for (int e = 0; e < CH; ++e) acc[r][e] = 0.f;
            for (int sc = s0; sc < s1; sc += kKvTok) {
                const int nt = min(kKvTok, s1 - sc);
                __syncthreads();
                for (int e = threadIdx.x; e < kKvTok * kKvRows; e += 256) {
                    const int tt = e / kKvRows, r = e % kKvRows;
                    const bool ok = tt < nt && r < nr;
                    sds[tt][r] = ok ? dS[(int64_t)(sc + tt) * max_d + j0 + r] : 0.f;
                    sp[tt][r] = ok ? P[(int64_t)(sc + tt) * max_d + j0 + r] : 0.f;
                }
                if (threadIdx.x < kKvTok) stok[threadIdx.x] = threadIdx.x < nt ? perm[sc + threadIdx.x] : 0;
                __syncthreads();
                if (!live) continue;
                for (int tt = 0; tt < nt; ++tt) {
                    const int tok = stok[tt];
                    float v[CH];
                    const float *w;
                    if (isk) {
                        load_chunk<T, CH>(x + (int64_t)tok * d_in, c, v);
                        w = sds[tt];
                    } else {
                        const float *src = dov + (int64_t)tok * d_emb + (c - ck) * CV;
#pragma unroll
                        for (int e = 0; e < CH; ++e) v[e] = e < CV ? src[e] : 0.f;
                        w = sp[tt];
                    }
#pragma unroll
                    for (int r = 0; r < kKvRows; ++r)
#pragma unroll
                        for (int e = 0; e < CH; ++e) acc[r][e] = fmaf(w[r], v[e], acc[r][e]);
                }
            }
            if (!live) continue;
            for (int r = 0; r < nr; ++r) {
                float *dst = isk ? dWK + (r0 + j0 + r) * d_in + c * CH
                                 : dWV + (r0 + j0 + r) * d_emb + (c - ck) * CV;
                const int ne = isk ? CH : CV;
#pragma unroll
                for (int e = 0; e < CH; ++e)
                    if (e < ne) dst[e] += acc[r][e];
            }
        }
    }
}

template <typename T, int CH, int NI, int NE, int TB>
hipError_t launch_token_kernels(const BwdArgs &a, int part, hipStream_t s) {
    if (part == 0) {
        hipLaunchKernelGGL((k_attn_bwd<T, CH, NI, NE, TB>), dim3(1024), dim3(256), 0, s, (const T *)a.x,
                           (const T *)a.WK, (const T *)a.WV, a.perm, a.items, a.hdr, a.dov, a.d_in,
                           a.d_emb, a.max_d, a.dx, a.P, a.dS);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_kv_items, dim3(64), dim3(256), 0, s, a.off, a.uniq, const_cast<int32_t *>(a.hdr),
                       a.vocab, a.kv_items, a.kv_cap);
    hipLaunchKernelGGL((k_kv_grad<T, CH>), dim3(2048), dim3(256), 0, s, (const T *)a.x, a.off, a.uniq,
                       a.seg_start, a.perm, a.hdr, a.kv_items, a.kv_cap, a.dov, a.d_in, a.d_emb,
                       a.max_d, a.P, a.dS, a.dWK, a.dWV);
    return hipGetLastError();
}

// chunks per lane for d_in (NI) and d_emb (NE): rows of up to 64 * NI * CH elements
template <typename T, int CH, int NI>
hipError_t launch_token_ne(const BwdArgs &a, int part, hipStream_t s) {
    constexpr int TB = NI * CH <= 32 ? 2 : 1;
    if (a.d_emb <= 64 * CH) return launch_token_kernels<T, CH, NI, 1, TB>(a, part, s);
    if (a.d_emb <= 128 * CH) return launch_token_kernels<T, CH, NI, 2, TB>(a, part, s);
    return launch_token_kernels<T, CH, NI, (1024 + 64 * CH - 1) / (64 * CH), TB>(a, part, s);
}

template <typename T, int CH>
hipError_t launch_token_ch(const BwdArgs &a, int part, hipStream_t s) {
    if (a.d_in <= 64 * CH) return launch_token_ne<T, CH, 1>(a, part, s);
    if (a.d_in <= 128 * CH) return launch_token_ne<T, CH, 2>(a, part, s);
    if (a.d_in <= 256 * CH) return launch_token_ne<T, CH, 4>(a, part, s);
    return launch_token_ne<T, CH, (4096 + 64 * CH - 1) / (64 * CH)>(a, part, s);
}

// ---------------------------------------------------------------- matrix cores (bf16)
// Attention backward on the matrix cores, for bf16 plans with d_in in {512, 1024,
// 2048} and d_emb in {128, 256, 512}.  One workgroup per item of up to 16 tokens of
// one block (sorted positions s0 .. s0 + cnt - 1; token j of the item is MFMA
// column j), so each K and V row is read once per 16 tokens:
//  * the block's rows stream through LDS in 16-row stages (double-buffered
//    asynchronous copies; the lane's slice of the stage's V row is loaded into
//    registers one stage ahead);
//  * one pass with an online softmax: D = <dO, o> is known beforehand (o is the
//    forward output the recompute left in the workspace), so with the running max m
//    and sum l, dx^T accumulates K_t^T (e^(s - m) (dP - D)), rescaled by e^(m_old -
//    m) when m grows and divided by l at the end, which is dx^T += K_t^T dS with
//    dS = P (dP - D), dP = V dO^T; the raw scores and dP go to the P and dS arrays,
//    and the token's (lse, D, d_t) to tstat, from which k_bwd_normalize forms P and
//    dS for the key / value gradients;
//  * wavefront w of NW (4, or 8 at d_in 2048 to keep x and the dx sums in
//    registers) owns 1/NW of d_in (scores' partial sums, dx columns) and of d_emb
//    (dP's partial sums); the wavefronts' partial scores and dP are added through
//    LDS in a fixed order;
//  * scores use v_mfma_f32_16x16x32_bf16 with K rows as the first operand, so a
//    lane holds rows 4 (l / 16) + v of token l % 16 -- which is the layout the
//    second operand of v_mfma_f32_16x16x16_bf16 wants for dS; the first operand
//    (K transposed) comes from ds_read_b64_tr_b16: lane (g, j) passing the address
//    of row 4g + j / 4, columns c0 + 4 (j % 4) .. +3 receives rows 4g .. 4g + 3 of
//    column c0 + j.
// dO enters the dP product rounded to bf16 (the other products already take bf16
// operands); everything accumulates in fp32.
constexpr int kBwdT = 16;  // tokens per matrix-core item
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int XQ, int DE, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_attn_bwd_mfma(BwdArgs a) {
    constexpr int d_in = 64 * XQ;
    constexpr int KROW = d_in * 2 + 48;   // LDS bytes per K row (padding: conflict-free reads)
    constexpr int KST = 16 * KROW;        // one 16-row stage
    constexpr int CPR = d_in / 512;       // 1 KB copies per row
    constexpr int CPW = 16 * CPR / NW;    // copies per wavefront and stage
    constexpr int QI = d_in / NW;         // d_in columns per wavefront
    constexpr int NXK = QI / 32;          // their 32-column steps
    constexpr int QE = DE / NW;           // d_emb columns per wavefront
    constexpr int NEK = QE / 32;
    constexpr int NCB = QI / 16;          // 16-column dx blocks per wavefront
    constexpr int XB = NW * 64 * 16;      // bytes of one exchange area (a f32x4 per lane)
    static_assert(CPR >= 1 && CPW * NW == 16 * CPR && NEK >= 1 && 2 * KST + 2 * XB <= 163840,
                  "bwd stages");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * KST + 2 * XB];
    f32x4_t *const spart = reinterpret_cast<f32x4_t *>(lds + 2 * KST);
    f32x4_t *const dpart = reinterpret_cast<f32x4_t *>(lds + 2 * KST + XB);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l16 = lane & 15, kg = lane >> 4;
    const uint16_t *X = static_cast<const uint16_t *>(a.x);
    const uint16_t *WK = static_cast<const uint16_t *>(a.WK);
    const uint16_t *WV = static_cast<const uint16_t *>(a.WV);
    const uint16_t *O = static_cast<const uint16_t *>(a.o);
    const uint32_t lds0 = lds_addr(lds);
    const int nitems = a.hdr[HDR_NLIGHT];
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        const int4 item = a.items[it];
        const int s0 = __builtin_amdgcn_readfirstlane(item.x);
        const int cnt = __builtin_amdgcn_readfirstlane(item.y);
        const int64_t r0 = __builtin_amdgcn_readfirstlane(item.z);
        const int d = __builtin_amdgcn_readfirstlane(item.w);
        if (d < 0) {  // ID out of range: no gradient (flagged by the route)
            if (w == 0 && lane < cnt) a.tstat[s0 + lane] = make_float4(0.f, 0.f, __int_as_float(0), 0.f);
            continue;
        }
        const int nc = (d + 15) / 16;
        const int tok = a.perm[s0 + min(l16, cnt - 1)];
        // this lane's token: x and dO over the wavefront's quarters, and <dO, o>
        bf16x8_t xf[NXK], df[NEK];
#pragma unroll
        for (int ks = 0; ks < NXK; ++ks)
            xf[ks] = *reinterpret_cast<const bf16x8_t *>(X + (int64_t)tok * d_in + w * QI + 32 * ks + 8 * kg);
#pragma unroll
        for (int ks = 0; ks < NEK; ++ks) {
            const float4 *dp = reinterpret_cast<const float4 *>(a.dov + (int64_t)tok * DE + w * QE + 32 * ks + 8 * kg);
            const float4 u0 = dp[0], u1 = dp[1];
            df[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(pack2(u0.x, u0.y), pack2(u0.z, u0.w),
                                                             pack2(u1.x, u1.y), pack2(u1.z, u1.w)));
        }
        float D = 0.f;
#pragma unroll 2
        for (int j = 0; j < DE / 32; ++j) {
            const int64_t e0 = (int64_t)tok * DE + 32 * j + 8 * kg;
            const float4 *dp = reinterpret_cast<const float4 *>(a.dov + e0);
            const float4 u0 = dp[0], u1 = dp[1];
            const uint4 ov = *reinterpret_cast<const uint4 *>(O + e0);
            D = fmaf(u0.x, bf_lo(ov.x), D); D = fmaf(u0.y, bf_hi(ov.x), D);
            D = fmaf(u0.z, bf_lo(ov.y), D); D = fmaf(u0.w, bf_hi(ov.y), D);
            D = fmaf(u1.x, bf_lo(ov.z), D); D = fmaf(u1.y, bf_hi(ov.z), D);
            D = fmaf(u1.z, bf_lo(ov.w), D); D = fmaf(u1.w, bf_hi(ov.w), D);
        }
        D += __shfl_xor(D, 16);
        D += __shfl_xor(D, 32);

        f32x4_t acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.f;

        // stage c: K rows [16c, +16) (past d_t: row d_t - 1) by asynchronous copies, and
        // this lane's slice of V row 16c + l16 into registers (issued after the copies,
        // consumed in the next stage, so no vector load waits on copies in flight)
        auto issue = [&](int c) {
            const uint32_t base = lds0 + (uint32_t)((c & 1) * KST);
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int q = w * CPW + i, row = q / CPR, piece = q % CPR;
                const int64_t grow = r0 + min(16 * c + row, d - 1);
                async_ld16(WK + grow * d_in + piece * 512 + lane * 8, base + row * KROW + piece * 1024);
            }
        };
        auto load_v = [&](int c, bf16x8_t (&v)[NEK]) {
            const uint16_t *vr = WV + (r0 + min(16 * c + l16, d - 1)) * DE + w * QE + 8 * kg;
#pragma unroll
            for (int ks = 0; ks < NEK; ++ks) v[ks] = *reinterpret_cast<const bf16x8_t *>(vr + 32 * ks);
        };
        bf16x8_t vcur[NEK], vnext[NEK];
        issue(0);
        load_v(0, vcur);
        for (int c = 0; c < nc; ++c) {
            wait_vmcnt<0>();
            lds_barrier();
            if (c + 1 < nc) {
                issue(c + 1);
                load_v(c + 1, vnext);
            }
            const unsigned char *kt = lds + (c & 1) * KST;
            f32x4_t sp = {0.f, 0.f, 0.f, 0.f}, dpp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NXK; ++ks) {
                const bf16x8_t A = *reinterpret_cast<const bf16x8_t *>(kt + l16 * KROW + (w * QI + 32 * ks + 8 * kg) * 2);
                sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, xf[ks], sp, 0, 0, 0);
            }
#pragma unroll
            for (int ks = 0; ks < NEK; ++ks)
                dpp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur[ks], df[ks], dpp, 0, 0, 0);
            spart[w * 64 + lane] = sp;
            dpart[w * 64 + lane] = dpp;
            lds_barrier();
            f32x4_t S = spart[lane], dP = dpart[lane];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) {
                S += spart[64 * ww + lane];
                dP += dpart[64 * ww + lane];
            }
            // online softmax over this lane's rows rb .. rb + 3 of token l16: the running
            // max m and sum l, and dx^T accumulated from e^(s - m) (dP - D), rescaled
            // whenever m grows
            const int rb = 16 * c + 4 * kg;
            float cm = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (rb + v < d) cm = fmaxf(cm, S[v]);
            cm = fmaxf(cm, __shfl_xor(cm, 16));
            cm = fmaxf(cm, __shfl_xor(cm, 32));
            const float mn = fmaxf(m, cm);
            const float sc = __expf(m - mn);
            float e[4], ls = 0.f, dsv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                e[v] = rb + v < d ? __expf(S[v] - mn) : 0.f;
                ls += e[v];
                dsv[v] = e[v] * (dP[v] - D);
            }
            ls += __shfl_xor(ls, 16);
            ls += __shfl_xor(ls, 32);
            l = fmaf(l, sc, ls);
            m = mn;
            // raw scores and dP per sorted position; normalised into P and dS afterwards
            if (w == 0 && l16 < cnt) {
                float *Sp = a.P + (int64_t)(s0 + l16) * a.max_d, *dPp = a.dS + (int64_t)(s0 + l16) * a.max_d;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (rb + v < d) {
                        Sp[rb + v] = S[v];
                        dPp[rb + v] = dP[v];
                    }
            }
            const i16x4_t B = __builtin_bit_cast(i16x4_t, make_uint2(pack2(dsv[0], dsv[1]), pack2(dsv[2], dsv[3])));
            const unsigned char *trb = kt + (4 * kg + (l16 >> 2)) * KROW + (w * QI + 4 * (l16 & 3)) * 2;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const i16x4_t Ak = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(trb + 32 * cb));
                acc[cb] *= sc;
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Ak, B, acc[cb], 0, 0, 0);
            }
            if (c + 1 < nc) {
#pragma unroll
                for (int ks = 0; ks < NEK; ++ks) vcur[ks] = vnext[ks];
            }
        }
        // dx[token][columns] += dx^T / l: lane holds columns 16 cb + 4 kg .. + 3 of token l16
        const float inv_l = 1.f / l;
        if (l16 < cnt) {
            float *dxr = a.dx + (int64_t)tok * d_in + w * QI + 4 * kg;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                float4 *dst = reinterpret_cast<float4 *>(dxr + 16 * cb);
                float4 v = *dst;
                v.x += acc[cb][0] * inv_l; v.y += acc[cb][1] * inv_l;
                v.z += acc[cb][2] * inv_l; v.w += acc[cb][3] * inv_l;
                *dst = v;
            }
            if (w == 0 && kg == 0)
                a.tstat[s0 + l16] = make_float4(m + __logf(l), D, __int_as_float(d), 0.f);
        }
        lds_barrier();  // the next item's first copies reuse the stages and the exchange area
    }
}

// P = e^(s - lse) and dS = P (dP - D) in place of the raw scores and dP the
// matrix-core attention backward stored, for rows j < d_t of every sorted position
// (d_t = 0 for tokens whose ID is out of range).
__global__ __launch_bounds__(256) void k_bwd_normalize(const float4 *__restrict__ tstat, int64_t n, int max_d,
                                                       float *__restrict__ P, float *__restrict__ dS) {
    const int64_t total = n * max_d;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t pos = i / max_d;
        const int j = (int)(i - pos * max_d);
        const float4 st = tstat[pos];
        if (j < __float_as_int(st.z)) {
            const float p = __expf(P[i] - st.x);
            P[i] = p;
            dS[i] = p * (dS[i] - st.y);
        }
    }
}

// Key / value gradients on the matrix cores (bf16, the same dims as the matrix-core
// attention backward):
//   dW_K[rows] += dS^T x,  dW_V[rows] += P^T dO
// taken as dW^T (columns x rows) += x^T (columns x tokens) dS (tokens x rows) with
// v_mfma_f32_16x16x16_bf16.  Work items are (block, 64 rows, column slice): a slice
// is 256 columns of W_K or of W_V (all of d_emb when it is 128), so a staged token
// tile feeds 64 table rows (a block's x rows are read once per 64 rows and slice,
// not per 16 rows) and the item's accumulators (64 rows x 256 columns over 4
// wavefronts) stay in registers; four workgroups share a CU, so one's start-up and
// read-modify-write overlap the others' streaming.  The block's tokens go by in
// tiles of 16 through a ring of three LDS slots, two tiles in flight while one is
// multiplied: per tile and wavefront, two 1 KB asynchronous copies of two token rows
// each (x, or dO rounded to bf16 beforehand) and four 256-byte copies of tokens' dS
// (or P) values for the item's rows, whose token indices come through the scalar
// cache so that no vector load drains the copies in flight.  Token rows are read
// transposed (ds_read_b64_tr_b16: lane (g, j) passing the address of row 4g + j / 4,
// columns c0 + 4 (j % 4) .. +3 receives rows 4g .. 4g + 3 of column c0 + j) as the
// first operand; the dS / P values, rounded to bf16, are the second.  A lane ends
// with 4 consecutive columns of one row per 16 x 16 block, added to the fp32
// gradient by one 16-byte read-modify-write per block.  Every row's gradient is one
// workgroup's ordered sum over the block's tokens (no atomics).
constexpr int kKvGroup = 64;     // table rows per item
constexpr int kKvSlice = 256;    // columns per item
constexpr int kKvRing = 3;       // LDS slots (token tiles)

__host__ __device__ constexpr int kv_slices(int64_t d_in, int64_t d_emb) {
    return (int)(d_in / kKvSlice + (d_emb > kKvSlice ? d_emb / kKvSlice : 1));
}

__global__ __launch_bounds__(256) void k_kv_items_sliced(const int64_t *__restrict__ off,
                                                         const int32_t *__restrict__ uniq,
                                                         int32_t *__restrict__ hdr, int64_t vocab,
                                                         int2 *__restrict__ items, int cap, int nslice) {
    const int m = hdr[HDR_NSEG];
    for (int b = blockIdx.x * 256 + threadIdx.x; b < m; b += gridDim.x * 256) {
        const int t = uniq[b];
        if (t < 0 || t >= vocab) continue;
        const int d = (int)(off[t + 1] - off[t]);
        const int nt = (d + kKvGroup - 1) / kKvGroup * nslice;
        const int at = atomicAdd(&hdr[HDR_NKV], nt);
        // (block, first row * 16 + slice)
        for (int r = 0; r < nt && at + r < cap; ++r)
            items[at + r] = make_int2(b, (r / nslice) * kKvGroup * 16 + r % nslice);
    }
}

// dO rounded to bf16, 8 values per thread (the key / value gradients' token rows)
__global__ __launch_bounds__(256) void k_round_bf16(const float4 *__restrict__ src, int64_t n8,
                                                    uint4 *__restrict__ dst) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
        const float4 u0 = src[2 * i], u1 = src[2 * i + 1];
        dst[i] = make_uint4(pack2(u0.x, u0.y), pack2(u0.z, u0.w), pack2(u1.x, u1.y), pack2(u1.z, u1.w));
    }
}

template <int XQ, int DE>
__global__ __launch_bounds__(256, 4) void k_kv_grad_mfma(BwdArgs a) {
    constexpr int d_in = 64 * XQ;
    constexpr int KS = d_in / kKvSlice;            // W_K slices; then the W_V slices
    constexpr int VW = DE < kKvSlice ? DE : kKvSlice;  // W_V slice width
    constexpr int PAIR = 4 * kKvSlice + 48;        // LDS: two token rows (bf16) + pad
    constexpr int TSTR = 4 * kKvGroup + 16;        // LDS: one token's dS / P values (fp32) + pad
    constexpr int SLOT = 8 * PAIR + 16 * TSTR;
    static_assert(KS >= 1 && DE % 128 == 0 && 4 * kKvRing * SLOT <= 163840, "kv slices");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kKvRing * SLOT];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // 4 wavefronts
    const int l16 = lane & 15, kg = lane >> 4;
    const uint16_t *X = static_cast<const uint16_t *>(a.x);
    const uint32_t lds0 = lds_addr(lds);
    const int nitems = min(a.hdr[HDR_NKV], a.kv_cap);
    // this lane's transposed-read row (4 kg + l16 / 4) within a slot
    const int rr = 4 * kg + (l16 >> 2);
    const uint32_t xrow = (uint32_t)((rr >> 1) * PAIR + (rr & 1) * 2 * kKvSlice);

    auto run = [&](auto vslice, int b, int j0, int sl) {
        constexpr bool V = decltype(vslice)::value;
        constexpr int WCOL = V ? VW / 4 : kKvSlice / 4;  // columns per wavefront
        constexpr int NCB = WCOL / 16;
        const int t = __builtin_amdgcn_readfirstlane(a.uniq[b]);
        const int64_t r0 = a.off[t];
        const int d = (int)(a.off[t + 1] - r0);
        const int nr = __builtin_amdgcn_readfirstlane(min(kKvGroup, d - j0));
        const int nrb = (nr + 15) >> 4;
        const int s0 = __builtin_amdgcn_readfirstlane(a.seg_start[b]);
        const int s1 = __builtin_amdgcn_readfirstlane(a.seg_start[b + 1]);
        const int ntile = (s1 - s0 + 15) >> 4;
        const int c0 = (V ? sl - KS : sl) * kKvSlice;  // the slice's first column
        const uint16_t *rows = V ? a.dob : X;
        const int64_t ld = V ? DE : d_in;
        const float *bsrc = V ? a.P : a.dS;
        const int bcol = min(j0 + lane, a.max_d - 1);
        // lane's 16-byte piece of a token row: lanes 0-31 the first row of a pair,
        // 32-63 the second (pieces past the slice repeat its last one)
        const int rc = c0 + min(lane & 31, (V ? VW : kKvSlice) / 8 - 1) * 8;
        // tile k -> slot k % kKvRing: token rows 4w .. 4w + 3 (rows past the block's
        // end repeat its last token; their dS / P are zeroed when read)
        auto issue = [&](int k) {
            const int tb = s0 + 16 * k, last = s1 - 1;
            const uint32_t base = lds0 + (uint32_t)((k % kKvRing) * SLOT);
            int p[4], tok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = min(tb + 4 * w + i, last);
            scalar_ld2(a.perm + p[0], a.perm + p[1], tok[0], tok[1]);
            scalar_ld2(a.perm + p[2], a.perm + p[3], tok[2], tok[3]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tk = lane < 32 ? tok[2 * h] : tok[2 * h + 1];
                async_ld16(rows + (int64_t)tk * ld + rc, base + (uint32_t)((2 * w + h) * PAIR));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                async_ld4(bsrc + (int64_t)p[i] * a.max_d + bcol, base + 8 * PAIR + (uint32_t)((4 * w + i) * TSTR));
        };
        f32x4_t acc[4][NCB];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lds_barrier();  // the previous item's last tile is read by every wavefront
#pragma unroll
        for (int k = 0; k < kKvRing - 1; ++k)
            if (k < ntile) issue(k);
        for (int k = 0; k < ntile; ++k) {
            // this wavefront's 6 copies of tile k have landed (those of k + 1 may not)
            if (k + 1 < ntile) wait_vmcnt<6 * (kKvRing - 2)>();
            else wait_vmcnt<0>();
            lds_barrier();
            // the slot of tile k + 2 was last read in tile k - 1, which every wavefront finished
            if (k + kKvRing - 1 < ntile) issue(k + kKvRing - 1);
            const int nt = min(16, s1 - s0 - 16 * k);
            const unsigned char *slot = lds + (k % kKvRing) * SLOT;
            i16x4_t B[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                if (rb < nrb) {
                    const int row = 16 * rb + l16;
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tk = 4 * kg + i;
                        const float f = *reinterpret_cast<const float *>(slot + 8 * PAIR + tk * TSTR + 4 * row);
                        v[i] = (tk < nt && row < nr) ? f : 0.f;
                    }
                    B[rb] = __builtin_bit_cast(i16x4_t, make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3])));
                }
            }
            const unsigned char *xr = slot + xrow + (w * WCOL + 4 * (l16 & 3)) * 2;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const i16x4_t A = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t *)(xr + 32 * cb));
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    if (rb < nrb) acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, B[rb], acc[rb][cb], 0, 0, 0);
            }
        }
        // lane: columns c0 + w WCOL + 16 cb + 4 kg .. + 3 of row j0 + 16 rb + l16
        float *g = (V ? a.dWV : a.dWK) + (r0 + j0) * ld + c0 + w * WCOL + 4 * kg;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            if (rb < nrb && 16 * rb + l16 < nr) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    float4 *dst = reinterpret_cast<float4 *>(g + (int64_t)(16 * rb + l16) * ld + 16 * cb);
                    float4 v = *dst;
                    v.x += acc[rb][cb][0]; v.y += acc[rb][cb][1]; v.z += acc[rb][cb][2]; v.w += acc[rb][cb][3];
                    *dst = v;
                }
            }
        }
    };
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        const int2 item = a.kv_items[it];
        const int b = __builtin_amdgcn_readfirstlane(item.x);
        const int j0 = __builtin_amdgcn_readfirstlane(item.y >> 4);
        const int sl = __builtin_amdgcn_readfirstlane(item.y & 15);
        if (sl < KS) run(std::false_type{}, b, j0, sl);
        else run(std::true_type{}, b, j0, sl);
    }
}

template <int XQ, int NW, int DE>
void launch_bwd_mfma_de(const BwdArgs &a, int part, hipStream_t s) {
    const dim3 b(64 * NW);
    if (part == 0) {
        hipLaunchKernelGGL((k_attn_bwd_mfma<XQ, DE, NW>), dim3(256), b, 0, s, a);
    } else {
        hipLaunchKernelGGL(k_bwd_normalize, dim3((unsigned)std::min<int64_t>(8192, (a.n * a.max_d + 255) / 256)),
                           dim3(256), 0, s, a.tstat, a.n, a.max_d, a.P, a.dS);
        const int64_t n8 = a.n * DE / 8;
        hipLaunchKernelGGL(k_round_bf16, dim3((unsigned)std::min<int64_t>(4096, (n8 + 255) / 256)), dim3(256), 0,
                           s, reinterpret_cast<const float4 *>(a.dov), n8, reinterpret_cast<uint4 *>(a.dob));
        hipLaunchKernelGGL(k_kv_items_sliced, dim3(64), dim3(256), 0, s, a.off, a.uniq,
                           const_cast<int32_t *>(a.hdr), a.vocab, a.kv_items, a.kv_cap, kv_slices(64 * XQ, DE));
        hipLaunchKernelGGL((k_kv_grad_mfma<XQ, DE>), dim3(1024), dim3(256), 0, s, a);
    }
}

template <int XQ, int NW>
hipError_t launch_bwd_mfma_xq(const BwdArgs &a, int part, hipStream_t s) {
    switch (a.d_emb) {
        case 128:
            if constexpr (NW == 4) {
                launch_bwd_mfma_de<XQ, NW, 128>(a, part, s);
                break;
            }
            return hipErrorInvalidValue;
        case 256: launch_bwd_mfma_de<XQ, NW, 256>(a, part, s); break;
        case 512: launch_bwd_mfma_de<XQ, NW, 512>(a, part, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// d_in 2048 takes eight wavefronts, whose d_emb share must hold a 32-column step
bool bwd_mfma_dims(int64_t d_in, int64_t d_emb, int dtype) {
    if (dtype != L3_BF16) return false;
    if (d_in == 512 || d_in == 1024) return d_emb == 128 || d_emb == 256 || d_emb == 512;
    return d_in == 2048 && (d_emb == 256 || d_emb == 512);
}

}  // namespace

hipError_t launch_transpose(const void *src, int64_t ld_src, int64_t rows, int64_t cols, void *dst,
                            int64_t ld_dst, int64_t rows_pad, int dtype, hipStream_t s) {
    if (rows_pad <= 0 || cols <= 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows_pad + 63) / 64));
    const bool vec = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0) && ld_src % 8 == 0 && ld_dst % 8 == 0;
    if (dtype == L3_BF16 && vec)
        hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, (const uint16_t *)src, ld_src, rows, cols,
                           (uint16_t *)dst, ld_dst, rows_pad);
    else if (dtype == L3_BF16)
        hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)src, ld_src,
                           rows, cols, (uint16_t *)dst, ld_dst, rows_pad);
    else
        hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s, (const float *)src, ld_src, rows,
                           cols, (float *)dst, ld_dst, rows_pad);
    return hipGetLastError();
}

hipError_t launch_ln_bwd(const void *h, const float *stats, const float *gamma, const float *beta,
                         const float *dy, int64_t n, int64_t d_up, void *dh, void *y, float2 *part,
                         float *dgamma, float *dbeta, int dtype, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const dim3 g1((unsigned)((n + 3) / 4)), g2((unsigned)((d_up + 255) / 256), (unsigned)ln_param_chunks(n));
    if (dtype == L3_BF16 && (d_up == 512 || d_up == 1024 || d_up == 2048)) {
        const dim3 gc((unsigned)ln_param_chunks(n));
        const uint16_t *hb = (const uint16_t *)h;
        uint16_t *dhb = (uint16_t *)dh, *yb = (uint16_t *)y;
        switch (d_up / 512) {
            case 1: hipLaunchKernelGGL(k_ln_bwd_bf16<1>, gc, dim3(256), 0, s, hb, stats, gamma, beta, dy, n, dhb, yb, part); break;
            case 2: hipLaunchKernelGGL(k_ln_bwd_bf16<2>, gc, dim3(256), 0, s, hb, stats, gamma, beta, dy, n, dhb, yb, part); break;
            default: hipLaunchKernelGGL(k_ln_bwd_bf16<4>, gc, dim3(256), 0, s, hb, stats, gamma, beta, dy, n, dhb, yb, part); break;
        }
    } else if (dtype == L3_BF16) {
        hipLaunchKernelGGL(k_ln_bwd<uint16_t>, g1, dim3(256), 0, s, (const uint16_t *)h, stats, gamma,
                           beta, dy, n, d_up, (uint16_t *)dh, (uint16_t *)y);
        hipLaunchKernelGGL(k_ln_param_part<uint16_t>, g2, dim3(256), 0, s, (const uint16_t *)h, stats, dy,
                           n, d_up, part);
    } else {
        hipLaunchKernelGGL(k_ln_bwd<float>, g1, dim3(256), 0, s, (const float *)h, stats, gamma, beta, dy,
                           n, d_up, (float *)dh, (float *)y);
        hipLaunchKernelGGL(k_ln_param_part<float>, g2, dim3(256), 0, s, (const float *)h, stats, dy, n,
                           d_up, part);
    }
    hipLaunchKernelGGL(k_ln_param_reduce, dim3((unsigned)((d_up + 15) / 16)), dim3(256), 0, s, part,
                       ln_param_chunks(n), d_up, dgamma, dbeta);
    return hipGetLastError();
}

int kv_item_capacity(int64_t n, int64_t rows, int64_t d_in, int64_t d_emb, int dtype) {
    int64_t c = n + rows / kKvRows + 1;
    if (bwd_mfma_dims(d_in, d_emb, dtype)) c = std::max<int64_t>(c, (n + rows / kKvGroup + 1) * kv_slices(d_in, d_emb));
    return (int)std::min<int64_t>(INT32_MAX, c);
}

int ln_param_chunks(int64_t n) { return (int)std::max<int64_t>(1, (n + kLnRows - 1) / kLnRows); }

int attn_bwd_tokens(int64_t d_in, int64_t d_emb, int dtype) {
    if (bwd_mfma_dims(d_in, d_emb, dtype)) return kBwdT;
    // the kernel's TB for its chunk width: two tokens while a lane's share of d_in
    // (NI * CH elements) is at most 32
    const int64_t ch = dtype == L3_BF16 ? 8 : (d_in % 4 == 0 && d_emb % 4 == 0 ? 4 : 1);
    return d_in <= 256 * ch && 4 * ch <= 32 ? 2 : 1;
}

hipError_t launch_attn_bwd(const BwdArgs &a, int dtype, int part, hipStream_t s) {
    if (a.d_in > 4096 || a.d_emb > 1024) return hipErrorInvalidValue;
    if (bwd_mfma_dims(a.d_in, a.d_emb, dtype)) {
        if (a.d_in == 512) return launch_bwd_mfma_xq<8, 4>(a, part, s);
        if (a.d_in == 1024) return launch_bwd_mfma_xq<16, 4>(a, part, s);
        return launch_bwd_mfma_xq<32, 8>(a, part, s);
    }
    if (dtype == L3_BF16) return launch_token_ch<uint16_t, 8>(a, part, s);  // bf16 dims: multiples of 64
    if (a.d_in % 4 == 0 && a.d_emb % 4 == 0) return launch_token_ch<float, 4>(a, part, s);
    return launch_token_ch<float, 1>(a, part, s);
}

}  // namespace l3
