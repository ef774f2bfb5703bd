// The dense stages of the L^3 layer ("L^3: Large Lookup Layers": papernotes.org
// page, section 整体框架; kimjy99.github.io page, section "Method", the layer
// equation) when the batch is small, as in decoding:
//   h   = W_up o              C[M x N] = A[M x K] B[N x K]^T, bf16 in, fp32 sums
//   out = W_mix [LN(h) ; x]
// With M of a few dozen rows the work is bound by streaming the weights B, and a
// 256 x 256 output tile would leave most of the chip idle.  Here a workgroup owns
// 64 rows x (64 NB) columns over 256 of the K columns (split K):
//  * its four wavefronts load their B fragments for the whole K slice straight
//    from global memory into registers first (16 rows x 512 contiguous bytes per
//    16-column block), so every load of the slice is in flight at once;
//  * meanwhile the workgroup stages the 64 x 256 slice of A in LDS, applying the
//    LayerNorm of h on the way for the W_mix stage (the concatenation [LN(h) ; x]
//    is formed only in LDS, in bf16, and needs no folded weights);
//  * v_mfma_f32_16x16x32_bf16 with the B fragment as first operand leaves each
//    lane 4 consecutive output columns of one row: fp32 partial sums are stored
//    as 16-byte vectors, one slab per K slice.
// A second kernel adds the slabs in a fixed order (deterministic), rounds to bf16
// and, for the W_up stage, writes the LayerNorm partial statistics of each row's
// stored values per 64 columns (mean and sum of squared deviations).  The W_mix
// stage merges those partials into (mean, rstd) per row itself (Chan's pairwise
// update), so no separate statistics pass runs.
#include "cdna4.h"
#include "l3_internal.h"

namespace l3 {
namespace {

constexpr int SK_BM = 64;            // rows per workgroup
constexpr int SK_KC = 256;           // K columns per split
constexpr int SK_KCP = SK_KC + 8;    // LDS row stride (bf16): 528 bytes, conflict-free 16-byte reads
constexpr int SK_KB = SK_KC / 32;    // MFMA k-blocks per split

struct SkinnyP {
    const uint16_t *A1, *A2;   // A columns [0, K1) from A1 (row stride lda1), [K1, K) from A2 (lda2)
    int64_t lda1, lda2, K1;
    const float *lnp;          // LayerNorm partials of the A1 rows ([M x K1/64 x 2]) or null
    const float *gamma, *beta;
    float eps;
    const uint16_t *B;         // N x K, row stride K
    int64_t M, N, K;
    int S;                     // K splits
    float *part;               // [S x M x N] fp32 partial sums
};

template <int NB>
__global__ __launch_bounds__(256) void k_gemm_skinny(SkinnyP p) {
    __shared__ __attribute__((aligned(16))) uint16_t la[SK_BM * SK_KCP];
    __shared__ float2 rowst[SK_BM];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int s = (int)(blockIdx.x % (unsigned)p.S);
    const int64_t tn = blockIdx.x / (unsigned)p.S;
    const int64_t m0 = (int64_t)blockIdx.y * SK_BM, n0 = tn * (64 * NB), k0 = (int64_t)s * SK_KC;

    // B fragments of the whole slice: lane -> row n = block + lane % 16, columns
    // k0 + 32 kb + 8 (lane / 16) + [0, 8)
    bf16x8_t bf[NB][SK_KB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t n = n0 + 16 * (w * NB + j) + (lane & 15);
        const bool nok = n < p.N;
        const uint16_t *src = p.B + (nok ? n : 0) * p.K + k0 + 8 * (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < SK_KB; ++kb) {
            const bool ok = nok && (k0 + 32 * kb < p.K);
            bf[j][kb] = ok ? *reinterpret_cast<const bf16x8_t *>(src + 32 * kb) : bf16x8_t{};
        }
    }

    // row statistics for the LayerNorm of the A1 columns
    const bool ln = p.lnp != nullptr && k0 < p.K1;
    if (ln && t < SK_BM) {
        const int64_t m = min<int64_t>(m0 + t, p.M - 1);
        const int npart = (int)(p.K1 / kLnPart);
        const float *pp = p.lnp + m * npart * 2;
        float cnt = 0.f, mu = 0.f, m2 = 0.f;
        for (int i = 0; i < npart; ++i) {
            const float nb = (float)kLnPart, mb = pp[2 * i], m2b = pp[2 * i + 1];
            const float nn = cnt + nb, delta = mb - mu;
            mu += delta * (nb / nn);
            m2 += m2b + delta * delta * (cnt * nb / nn);
            cnt = nn;
        }
        rowst[t] = make_float2(mu, 1.f / sqrtf(m2 / cnt + p.eps));
    }
    __syncthreads();

    // stage A[m0 .. m0 + 64) x [k0 .. k0 + 256) (zero outside M x K) into LDS
#pragma unroll
    for (int i = 0; i < SK_BM * SK_KC / 8 / 256; ++i) {
        const int c = t + 256 * i, r = c >> 5, cc = c & 31;
        const int64_t m = m0 + r, k = k0 + 8 * cc;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < p.M && k < p.K) {
            if (k < p.K1) {
                v = *reinterpret_cast<const uint4 *>(p.A1 + m * p.lda1 + k);
                if (ln) {
                    const float2 st = rowst[r];
                    const float4 g0 = *reinterpret_cast<const float4 *>(p.gamma + k);
                    const float4 g1 = *reinterpret_cast<const float4 *>(p.gamma + k + 4);
                    const float4 b0 = *reinterpret_cast<const float4 *>(p.beta + k);
                    const float4 b1 = *reinterpret_cast<const float4 *>(p.beta + k + 4);
                    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                    const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                    uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xffff0000u);
                        u[e] = pack2((lo - st.x) * st.y * g[2 * e] + b[2 * e],
                                     (hi - st.x) * st.y * g[2 * e + 1] + b[2 * e + 1]);
                    }
                    v = make_uint4(u[0], u[1], u[2], u[3]);
                }
            } else {
                v = *reinterpret_cast<const uint4 *>(p.A2 + m * p.lda2 + (k - p.K1));
            }
        }
        *reinterpret_cast<uint4 *>(&la[r * SK_KCP + 8 * cc]) = v;
    }
    __syncthreads();

    f32x4_t acc[4][NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < SK_KB; ++kb) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                &la[(mb * 16 + (lane & 15)) * SK_KCP + 32 * kb + 8 * (lane >> 4)]);
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j][kb], a, acc[mb][j], 0, 0, 0);
        }
    }

    // lane holds columns 4 (lane / 16) + [0, 4) of its block, row lane % 16
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int64_t m = m0 + mb * 16 + (lane & 15);
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t n = n0 + 16 * (w * NB + j) + 4 * (lane >> 4);
            if (n < p.N)
                *reinterpret_cast<f32x4_t *>(p.part + ((int64_t)s * p.M + m) * p.N + n) = acc[mb][j];
        }
    }
}

// out[m][n] = bf16(sum over the S slabs, in slab order); with LN_OUT also the
// partial statistics of the stored values of row m over columns [64 c, 64 c + 64).
// One wavefront per (row, 64 columns).
template <bool LN_OUT>
__global__ __launch_bounds__(256) void k_skinny_reduce(const float *__restrict__ part, int S, int64_t M,
                                                       int64_t N, uint16_t *__restrict__ out,
                                                       float *__restrict__ ln_out) {
    const int lane = threadIdx.x & 63;
    const int64_t chunks = N / 64;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= M * chunks) return;
    const int64_t m = wid / chunks, c = wid - m * chunks, n = 64 * c + lane;
    float sum = 0.f;
    for (int s = 0; s < S; ++s) sum += part[((int64_t)s * M + m) * N + n];
    const uint32_t b = f2bf(sum);
    out[m * N + n] = (uint16_t)b;
    if constexpr (LN_OUT) {
        const float v = __uint_as_float(b << 16);
        float a = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) a += __shfl_xor(a, o);
        const float mean = a * (1.f / 64.f);
        float q = (v - mean) * (v - mean);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) q += __shfl_xor(q, o);
        if (lane == 0) {
            ln_out[(m * chunks + c) * 2] = mean;
            ln_out[(m * chunks + c) * 2 + 1] = q;
        }
    }
}

int skinny_splits(int64_t K) { return (int)((K + SK_KC - 1) / SK_KC); }

hipError_t launch_skinny(SkinnyP &p, hipStream_t s) {
    p.S = skinny_splits(p.K);
    const int64_t tm = (p.M + SK_BM - 1) / SK_BM;
    // widest column tile that still gives the chip a few hundred workgroups
    int nb = 1;
    for (int c : {4, 2}) {
        if (tm * ((p.N + 64 * c - 1) / (64 * c)) * p.S >= 256) { nb = c; break; }
    }
    const dim3 grid((unsigned)(((p.N + 64 * nb - 1) / (64 * nb)) * p.S), (unsigned)tm);
    if (nb == 4) hipLaunchKernelGGL(k_gemm_skinny<4>, grid, dim3(256), 0, s, p);
    else if (nb == 2) hipLaunchKernelGGL(k_gemm_skinny<2>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(k_gemm_skinny<1>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_reduce(const float *part, int S, int64_t M, int64_t N, uint16_t *out, float *ln_out,
                         hipStream_t s) {
    const int64_t waves = M * (N / 64);
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (ln_out) hipLaunchKernelGGL(k_skinny_reduce<true>, grid, dim3(256), 0, s, part, S, M, N, out, ln_out);
    else hipLaunchKernelGGL(k_skinny_reduce<false>, grid, dim3(256), 0, s, part, S, M, N, out, ln_out);
    return hipGetLastError();
}

}  // namespace

size_t skinny_part_bytes(int64_t M, int64_t N, int64_t K) {
    return (size_t)skinny_splits(K) * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_gemm_skinny_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M,
                                   int64_t N, int64_t K, float *ln_out, float *part, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    SkinnyP p{};
    p.A1 = A; p.A2 = A; p.lda1 = K; p.lda2 = K; p.K1 = K;
    p.B = B; p.M = M; p.N = N; p.K = K; p.part = part;
    const hipError_t e = launch_skinny(p, s);
    if (e != hipSuccess) return e;
    return launch_reduce(part, p.S, M, N, C, ln_out, s);
}

hipError_t launch_gemm_mix_skinny_bf16(const uint16_t *h, const uint16_t *x, const float *lnp,
                                       const float *gamma, const float *beta, float eps,
                                       const uint16_t *W_mix, uint16_t *out, int64_t M, int64_t d_up,
                                       int64_t d_in, int64_t d_out, float *part, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    SkinnyP p{};
    p.A1 = h; p.lda1 = d_up; p.K1 = d_up;
    p.A2 = x; p.lda2 = d_in;
    p.lnp = lnp; p.gamma = gamma; p.beta = beta; p.eps = eps;
    p.B = W_mix; p.M = M; p.N = d_out; p.K = d_up + d_in; p.part = part;
    const hipError_t e = launch_skinny(p, s);
    if (e != hipSuccess) return e;
    return launch_reduce(part, p.S, M, d_out, out, nullptr, s);
}

}  // namespace l3
