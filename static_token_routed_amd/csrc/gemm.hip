// The two dense stages of the L^3 layer ("L^3: Large Lookup Layers":
// papernotes.org page, section 整体框架; kimjy99.github.io page, section
// "Method", the layer equation):
//   h   = W_up o            (W_up: d_up x d_emb)
//   out = W_mix [LN(h) ; x]  (W_mix: d_out x (d_up + d_in))
// as bf16 MFMA GEMMs C[M x N] = A[M x K] B[N x K]^T with fp32 accumulation.
//
// Kernel shape (gfx950): 256 threads = 4 wavefronts in 2 x 2, each owning a
// 128 x 128 block of a 256 x 256 output tile as 4 x 4 v_mfma_f32_32x32x16_bf16
// accumulators (256 fp32 per lane).  K advances 64 at a time through two LDS
// stages (A and B tiles, 32 KB each, double-buffered: 128 KB); each 16-byte
// chunk of a 128-byte LDS row is XOR-swizzled by the row index so the
// fragment reads of 32 consecutive rows spread over the banks.  The MFMA takes
// the B tile as its first operand, so each lane ends up holding 4 consecutive
// output columns of one row: the epilogue stores 8-byte row segments directly.
// Tiles are numbered so that the workgroups the dispatcher sends to one XCD
// (workgroup id mod 8) form a contiguous, grouped block of tiles, sharing A
// rows and B columns in that XCD's L2.
//
// Fused work:
//  * W_up epilogue: per output row and 128-column chunk, the mean and the sum
//    of squared deviations (M2) of the bf16-rounded h values (LayerNorm
//    partial statistics).
//  * W_mix prologue: the A operand is built while staging: columns k < d_up
//    are LN(h) = (h - mean) * rstd * gamma + beta, with mean and variance
//    merged from the partials (Chan's pairwise update), columns k >= d_up are
//    x -- the concat [LN(h) ; x] never exists in memory.
#include "l3_internal.h"

namespace l3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int GROUP_M = 8;

struct GemmP {
    const uint16_t *A;   // M x lda, columns [0, K1)
    const uint16_t *A2;  // M x lda2, supplies columns [K1, K) (may be null if K1 == K)
    const uint16_t *B;   // N x K
    uint16_t *C;         // M x N
    int64_t lda, lda2, K1;
    int64_t M, N, K;
    // LayerNorm input statistics (W_mix prologue)
    const float *lnp;  // [M x npart x 2]
    const float *gamma, *beta;
    float eps;
    int npart;
    int64_t ln_width;  // number of normalised features (= K1)
    // LayerNorm output partials (W_up epilogue)
    float *ln_out;  // [M x npart_out x 2]
    int npart_out;
    int tiles_m, tiles_n;
};

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t f2bf(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ inline uint32_t pack2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

// tile id -> (tm, tn): XCD-contiguous, then grouped by GROUP_M tile rows.
__device__ inline void tile_coords(const GemmP &p, int &tm, int &tn) {
    const int nt = p.tiles_m * p.tiles_n;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, q = nt >> 3, r = nt & 7;
    const int tl = xcd * q + min(xcd, r) + (bid >> 3);
    const int per_group = GROUP_M * p.tiles_n;
    const int g = tl / per_group;
    const int first = g * GROUP_M;
    const int gsz = min(p.tiles_m - first, GROUP_M);
    const int in = tl - g * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

template <bool LN_IN, bool LN_OUT>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(GemmP p) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
    __shared__ float s_mean[LN_IN ? BM : 1], s_rstd[LN_IN ? BM : 1];

    int tm, tn;
    tile_coords(p, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = w >> 1, wn = w & 1;

    if constexpr (LN_IN) {
        const int64_t row = m0 + t;
        float mean = 0.f, rstd = 0.f;
        if (row < p.M) {
            const float *pp = p.lnp + row * p.npart * 2;
            float cnt = 0.f, mu = 0.f, m2 = 0.f;
            for (int i = 0; i < p.npart; ++i) {
                const float nb = (float)min<int64_t>(kLnPart, p.ln_width - (int64_t)i * kLnPart);
                const float mb = pp[2 * i], m2b = pp[2 * i + 1];
                const float nn = cnt + nb;
                const float delta = mb - mu;
                mu += delta * (nb / nn);
                m2 += m2b + delta * delta * (cnt * nb / nn);
                cnt = nn;
            }
            mean = mu;
            rstd = 1.f / sqrtf(m2 / cnt + p.eps);
        }
        s_mean[t] = mean;
        s_rstd[t] = rstd;
        __syncthreads();
    }

    // loader mapping: 16-byte chunk c of rows rb + 32 i
    const int lc = t & 7, lr = t >> 3;
    uint4 ra[8], rb[8];

    auto load_stage = [&](int64_t k0) {
        const bool first = k0 < p.K1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = m0 + lr + 32 * i;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < p.M) {
                const uint16_t *src = first ? p.A + row * p.lda + k0 + lc * 8
                                            : p.A2 + row * p.lda2 + (k0 - p.K1) + lc * 8;
                v = *reinterpret_cast<const uint4 *>(src);
            }
            ra[i] = v;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t col = n0 + lr + 32 * i;
            rb[i] = col < p.N ? *reinterpret_cast<const uint4 *>(p.B + col * p.K + k0 + lc * 8)
                              : make_uint4(0, 0, 0, 0);
        }
        if constexpr (LN_IN) {
            if (first) {
                const int64_t k = k0 + lc * 8;
                const float4 g0 = *reinterpret_cast<const float4 *>(p.gamma + k);
                const float4 g1 = *reinterpret_cast<const float4 *>(p.gamma + k + 4);
                const float4 b0 = *reinterpret_cast<const float4 *>(p.beta + k);
                const float4 b1 = *reinterpret_cast<const float4 *>(p.beta + k + 4);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float mu = s_mean[lr + 32 * i], rs = s_rstd[lr + 32 * i];
                    uint4 v = ra[i];
                    v.x = pack2((bf_lo(v.x) - mu) * rs * g0.x + b0.x, (bf_hi(v.x) - mu) * rs * g0.y + b0.y);
                    v.y = pack2((bf_lo(v.y) - mu) * rs * g0.z + b0.z, (bf_hi(v.y) - mu) * rs * g0.w + b0.w);
                    v.z = pack2((bf_lo(v.z) - mu) * rs * g1.x + b1.x, (bf_hi(v.z) - mu) * rs * g1.y + b1.y);
                    v.w = pack2((bf_lo(v.w) - mu) * rs * g1.z + b1.z, (bf_hi(v.w) - mu) * rs * g1.w + b1.w);
                    ra[i] = v;
                }
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = lr + 32 * i;
            const int pc = lc ^ (r & 7);
            *reinterpret_cast<uint4 *>(&As[buf][r * BK + pc * 8]) = ra[i];
            *reinterpret_cast<uint4 *>(&Bs[buf][r * BK + pc * 8]) = rb[i];
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nst = (int)(p.K / BK);
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) load_stage((int64_t)(st + 1) * BK);
        const uint16_t *as = As[buf];
        const uint16_t *bs = Bs[buf];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int ch = kk * 2 + (lane >> 5);
            bf16x8_t fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 128 + i * 32 + (lane & 31);
                fa[i] = *reinterpret_cast<const bf16x8_t *>(&as[r * BK + ((ch ^ (r & 7)) * 8)]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wn * 128 + j * 32 + (lane & 31);
                fb[j] = *reinterpret_cast<const bf16x8_t *>(&bs[r * BK + ((ch ^ (r & 7)) * 8)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
        if (st + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  acc[i][j] element e of lane l: output row m = m0 + wm*128 + i*32 + (l&31),
    // column n = n0 + wn*128 + j*32 + 8*(e/4) + 4*(l/32) + (e%4).
    const int64_t nbase = n0 + wn * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
        float hv[4][16];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n = nbase + j * 32 + 8 * g + 4 * (lane >> 5);
                const uint32_t lo = pack2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
                const uint32_t hi = pack2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                if (m < p.M && n < p.N)
                    *reinterpret_cast<uint2 *>(p.C + m * p.N + n) = make_uint2(lo, hi);
                if constexpr (LN_OUT) {
                    const bool ok = n < p.N;
                    hv[j][4 * g + 0] = ok ? bf_lo(lo) : 0.f;
                    hv[j][4 * g + 1] = ok ? bf_hi(lo) : 0.f;
                    hv[j][4 * g + 2] = ok ? bf_lo(hi) : 0.f;
                    hv[j][4 * g + 3] = ok ? bf_hi(hi) : 0.f;
                }
            }
        if constexpr (LN_OUT) {
            const int64_t width = min<int64_t>(kLnPart, p.N - nbase);
            if (width > 0) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) s += hv[j][e];
                s += __shfl_xor(s, 32);
                const float mean = s / (float)width;
                float q = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int64_t n = nbase + j * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
                        const float dv = hv[j][e] - mean;
                        q += n < p.N ? dv * dv : 0.f;
                    }
                q += __shfl_xor(q, 32);
                if (lane < 32 && m < p.M) {
                    float *dst = p.ln_out + (m * p.npart_out + nbase / kLnPart) * 2;
                    dst[0] = mean;
                    dst[1] = q;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 (any dims)

// C = A B^T with an optional LayerNorm+concat A operand (mix mode): for k < K1,
// A[m][k] = (h[m][k] - mean[m]) * rstd[m] * gamma[k] + beta[k]; else x[m][k - K1].
template <bool MIX>
__global__ __launch_bounds__(256) void k_gemm_f32(const float *__restrict__ A,
                                                  const float *__restrict__ A2,
                                                  const float *__restrict__ B,
                                                  float *__restrict__ C, int64_t M, int64_t N,
                                                  int64_t K, int64_t K1,
                                                  const float *__restrict__ stats,
                                                  const float *__restrict__ gamma,
                                                  const float *__restrict__ beta) {
    __shared__ float as[16][65], bs[16][65];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        for (int i = threadIdx.x; i < 64 * 16; i += 256) {
            const int r = i / 16, kk = i % 16;
            const int64_t m = m0 + r, n = n0 + r, k = k0 + kk;
            float av = 0.f, bv = 0.f;
            if (m < M && k < K) {
                if (!MIX) av = A[m * K + k];
                else if (k < K1) av = (A[m * K1 + k] - stats[2 * m]) * stats[2 * m + 1] * gamma[k] + beta[k];
                else av = A2[m * (K - K1) + (k - K1)];
            }
            if (n < N && k < K) bv = B[n * K + k];
            as[kk][r] = av;
            bs[kk][r] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = as[kk][ty * 4 + i]; b[i] = bs[kk][tx * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < M && n < N) C[m * N + n] = acc[i][j];
        }
}

// Per-row mean and 1/sqrt(var + eps) of h (M x W), two passes, one wavefront per row.
__global__ __launch_bounds__(256) void k_ln_stats_f32(const float *__restrict__ h, int64_t M,
                                                      int64_t W, float eps,
                                                      float *__restrict__ stats) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const float *r = h + row * W;
    float s = 0.f;
    for (int64_t c = lane; c < W; c += 64) s += r[c];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    const float mean = s / (float)W;
    float q = 0.f;
    for (int64_t c = lane; c < W; c += 64) { const float d = r[c] - mean; q = fmaf(d, d, q); }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) q += __shfl_xor(q, o);
    if (lane == 0) {
        stats[2 * row] = mean;
        stats[2 * row + 1] = 1.f / sqrtf(q / (float)W + eps);
    }
}

GemmP make_plain(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M, int64_t N, int64_t K) {
    GemmP p{};
    p.A = A; p.A2 = nullptr; p.B = B; p.C = C;
    p.lda = K; p.lda2 = 0; p.K1 = K;
    p.M = M; p.N = N; p.K = K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    return p;
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M, int64_t N,
                            int64_t K, float *ln_out, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    GemmP p = make_plain(A, B, C, M, N, K);
    const dim3 grid(p.tiles_m * p.tiles_n);
    if (ln_out) {
        p.ln_out = ln_out;
        p.npart_out = (int)((N + kLnPart - 1) / kLnPart);
        hipLaunchKernelGGL((k_gemm_bf16<false, true>), grid, dim3(256), 0, s, p);
    } else {
        hipLaunchKernelGGL((k_gemm_bf16<false, false>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_mix_bf16(const uint16_t *h, const uint16_t *x, const float *lnp,
                                const float *gamma, const float *beta, float eps,
                                const uint16_t *W_mix, uint16_t *out, int64_t M, int64_t d_up,
                                int64_t d_in, int64_t d_out, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    GemmP p = make_plain(h, W_mix, out, M, d_out, d_up + d_in);
    p.lda = d_up;
    p.A2 = x;
    p.lda2 = d_in;
    p.K1 = d_up;
    p.lnp = lnp;
    p.gamma = gamma;
    p.beta = beta;
    p.eps = eps;
    p.npart = (int)((d_up + kLnPart - 1) / kLnPart);
    p.ln_width = d_up;
    hipLaunchKernelGGL((k_gemm_bf16<true, false>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const float *A, const float *B, float *C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL((k_gemm_f32<false>), grid, dim3(256), 0, s, A, (const float *)nullptr, B, C,
                       M, N, K, K, (const float *)nullptr, (const float *)nullptr,
                       (const float *)nullptr);
    return hipGetLastError();
}

hipError_t launch_gemm_mix_f32(const float *h, const float *x, float *stats, const float *gamma,
                               const float *beta, float eps, const float *W_mix, float *out,
                               int64_t M, int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_ln_stats_f32, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, h, M, d_up,
                       eps, stats);
    const dim3 grid((unsigned)((d_out + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL((k_gemm_f32<true>), grid, dim3(256), 0, s, h, x, W_mix, out, M, d_out,
                       d_up + d_in, d_up, (const float *)stats, gamma, beta);
    return hipGetLastError();
}

}  // namespace l3
