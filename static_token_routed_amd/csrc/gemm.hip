// The two dense stages of the L^3 layer ("L^3: Large Lookup Layers":
// papernotes.org page, section 整体框架; kimjy99.github.io page, section
// "Method", the layer equation):
//   h   = W_up o            (W_up: d_up x d_emb)
//   out = W_mix [LN(h) ; x]  (W_mix: d_out x (d_up + d_in))
// as bf16 MFMA GEMMs C[M x N] = A[M x K] B[N x K]^T with fp32 accumulation.
//
// Kernel shape (gfx950): 512 threads = 8 wavefronts in 2 x 4, each owning a
// 128 x 64 block of a 256 x 256 output tile as 4 x 2 v_mfma_f32_32x32x16_bf16
// accumulators (128 fp32 per lane), so two wavefronts share each SIMD and one's
// MFMAs cover the other's LDS reads.  K advances 64 at a time.  Both operand
// tiles (256 x 64 bf16 each) go global -> LDS by asynchronous 16-byte copies
// (no register staging) into a double buffer: the copies of stage s+1 are in
// flight while stage s is multiplied, and barriers wait for LDS traffic only.
// Each 16-byte chunk of a 128-byte LDS row is XOR-swizzled by the row index
// (the swizzle is applied to the source address, since a copy lands at a fixed
// lane-linear LDS slot) so fragment reads of 32 consecutive rows spread over the
// banks.  The MFMA takes the B tile as its first operand, so each lane holds 4
// consecutive output columns of one row: the epilogue stores 8-byte segments.
// Tiles are numbered so that the workgroups the dispatcher sends to one XCD
// (workgroup id mod 8) form a contiguous, grouped block of tiles, sharing A
// rows and B columns in that XCD's L2.
//
// LayerNorm and the concat [LN(h) ; x] are fused into the W_mix operand path.
// For the first d_up columns the A tile is h, loaded into registers one stage
// ahead, turned into (h - mean) * rstd * gamma + beta (each element once per
// workgroup) and written into the swizzled LDS layout; mean and rstd per row
// come from the W_up epilogue's partial statistics (per row and 64-column
// chunk, the mean and the sum of squared deviations of the stored bf16 values),
// merged with Chan's pairwise update.  The remaining columns are x, copied
// asynchronously like B.  The concatenated operand never exists in memory.
#include <type_traits>

#include "cdna4.h"
#include "l3_internal.h"

namespace l3 {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int GROUP_M = 8;

struct GemmP {
    const uint16_t *A, *A2;  // A columns [0, K1) from A (row stride lda), [K1, K) from A2 (lda2)
    const uint16_t *B;       // N x K, row stride ldb
    uint16_t *C;             // M x N, row stride N
    int64_t lda, lda2, ldb, K1;
    int64_t M, N, K;
    const float *row_stats;  // [M x 2] (mean, rstd) of the A rows in [0, K1)  (LN_IN)
    const float *gamma, *beta;  // [K1]                                         (LN_IN)
    float *ln_out;           // [M x npart_out x 2] partial statistics of the stored rows
    int npart_out;
    int tiles_m, tiles_n;
};

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
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(GemmP p) {
    __shared__ __attribute__((aligned(1024))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(1024))) uint16_t Bs[2][BN * BK];

    int tm, tn;
    tile_coords(p, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = w >> 2, wn = w & 3;

    // Copy mapping: wave w issues 4 copies per operand and stage; copy q covers tile
    // rows [8q, 8q + 8) (1 KB of LDS).  Lane l fills physical chunk l % 8 of row
    // 8q + l / 8 with global chunk (l % 8) ^ (row & 7).  Rows past M (N) are clamped:
    // they only feed accumulators that are never stored.
    const int crow = lane >> 3, cphys = lane & 7;
    const uint32_t a_lds0 = lds_addr(&As[0][0]), b_lds0 = lds_addr(&Bs[0][0]);
    auto issue = [&](int64_t k0, int buf, bool a_async) {
        const bool first = k0 < p.K1;
        const uint16_t *abase = first ? p.A + k0 : p.A2 + (k0 - p.K1);
        const int64_t lda = first ? p.lda : p.lda2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = w * 4 + i;
            const int row = q * 8 + crow;
            const int gch = cphys ^ (row & 7);
            const int64_t ar = min<int64_t>(m0 + row, p.M - 1);
            const int64_t br = min<int64_t>(n0 + row, p.N - 1);
            const uint32_t off = (uint32_t)(buf * BM * BK * 2 + q * 1024);
            if (a_async) async_ld16(abase + ar * lda + gch * 8, a_lds0 + off);
            async_ld16(p.B + br * p.ldb + k0 + gch * 8, b_lds0 + off);
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // LayerNorm staging (LN_IN): thread t owns chunk t % 8 of tile rows t / 8 + 64 i
    const int sc = t & 7, sr = t >> 3;
    float mu[4] = {0.f, 0.f, 0.f, 0.f}, rs[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (LN_IN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = min<int64_t>(m0 + sr + 64 * i, p.M - 1);
            mu[i] = p.row_stats[2 * m];
            rs[i] = p.row_stats[2 * m + 1];
        }
    }
    uint4 hreg[4];
    float4 gam0, gam1, bet0, bet1;
    auto load_h = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = min<int64_t>(m0 + sr + 64 * i, p.M - 1);
            hreg[i] = *reinterpret_cast<const uint4 *>(p.A + m * p.lda + k0 + sc * 8);
        }
        gam0 = *reinterpret_cast<const float4 *>(p.gamma + k0 + sc * 8);
        gam1 = *reinterpret_cast<const float4 *>(p.gamma + k0 + sc * 8 + 4);
        bet0 = *reinterpret_cast<const float4 *>(p.beta + k0 + sc * 8);
        bet1 = *reinterpret_cast<const float4 *>(p.beta + k0 + sc * 8 + 4);
    };
    auto store_h = [&](int buf) {  // y = (h - mean) * rstd * gamma + beta, into the swizzled tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = sr + 64 * i;
            uint4 u = hreg[i];
            const float m_ = mu[i], r_ = rs[i];
            u.x = pack2((bf_lo(u.x) - m_) * r_ * gam0.x + bet0.x, (bf_hi(u.x) - m_) * r_ * gam0.y + bet0.y);
            u.y = pack2((bf_lo(u.y) - m_) * r_ * gam0.z + bet0.z, (bf_hi(u.y) - m_) * r_ * gam0.w + bet0.w);
            u.z = pack2((bf_lo(u.z) - m_) * r_ * gam1.x + bet1.x, (bf_hi(u.z) - m_) * r_ * gam1.y + bet1.y);
            u.w = pack2((bf_lo(u.w) - m_) * r_ * gam1.z + bet1.z, (bf_hi(u.w) - m_) * r_ * gam1.w + bet1.w);
            *reinterpret_cast<uint4 *>(&As[buf][r * BK + ((sc ^ (r & 7)) * 8)]) = u;
        }
    };

    // Fragments of k-substep kk (16 columns): A rows wm*128 + i*32 + lane%32 and B rows
    // wn*64 + j*32 + lane%32, 8 columns each (chunk 2kk + lane/32 of the 128-byte row).
    auto load_frags = [&](int buf, int kk, bf16x8_t (&fa)[4], bf16x8_t (&fb)[2]) {
        const uint16_t *as = As[buf];
        const uint16_t *bs = Bs[buf];
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + (lane & 31);
            fa[i] = *reinterpret_cast<const bf16x8_t *>(&as[r * BK + ((ch ^ (r & 7)) * 8)]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wn * 64 + j * 32 + (lane & 31);
            fb[j] = *reinterpret_cast<const bf16x8_t *>(&bs[r * BK + ((ch ^ (r & 7)) * 8)]);
        }
    };
    auto compute = [&](int buf) {
        bf16x8_t fa[2][4], fb[2][2];
        load_frags(buf, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int cur = kk & 1;
            // the next substep's fragments are read while this substep's MFMAs run
            if (kk < 3) load_frags(buf, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
        }
    };
    // Pipelined stages: wait for this stage's copies (the only loads in flight), start
    // the next stage's, multiply; an h stage is staged through registers and written
    // (normalised) into the other buffer after the multiply.
    const int nst = (int)(p.K / BK);
    const int nst1 = LN_IN ? (int)(p.K1 / BK) : 0;  // stages whose A operand is normalised h
    if (0 < nst1) {
        load_h(0);
        issue(0, 0, false);
        store_h(0);
    } else {
        issue(0, 0, true);
    }
    for (int st = 0; st < nst; ++st) {
        wait_vmcnt<0>();
        lds_barrier();
        const bool next = st + 1 < nst;
        const bool next_h = st + 1 < nst1;
        if (next) {
            if (next_h) load_h((int64_t)(st + 1) * BK);
            issue((int64_t)(st + 1) * BK, (st + 1) & 1, !next_h);
        }
        compute(st & 1);
        if (next_h) store_h((st + 1) & 1);
    }

    // Epilogue.  acc[i][j] element e of lane l: output row m = m0 + wm*128 + i*32 + (l&31),
    // column n = n0 + wn*64 + j*32 + 8*(e/4) + 4*(l/32) + (e%4).
    const int64_t nbase = n0 + wn * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
        float hv[2][16];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t n = nbase + j * 32 + 8 * g + 4 * (lane >> 5);
                const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                const uint32_t lo = pack2(v0, v1), hi = pack2(v2, v3);
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
            // partial statistics of this row over the wavefront's 64 columns
            const int64_t width = min<int64_t>(kLnPart, p.N - nbase);
            if (width > 0) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) s += hv[j][e];
                s += __shfl_xor(s, 32);
                const float mean = s / (float)width;
                float q = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
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

// Row statistics of h from the W_up epilogue's partials: one thread per row,
// Chan's pairwise merge of (count, mean, M2), then rstd = 1 / sqrt(M2/width + eps).
__global__ __launch_bounds__(256) void k_ln_finalize(const float *__restrict__ lnp, int64_t M,
                                                     int npart, int64_t width, float eps,
                                                     float *__restrict__ stats) {
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= M) return;
    const float *pp = lnp + row * npart * 2;
    float cnt = 0.f, mu = 0.f, m2 = 0.f;
    for (int i = 0; i < npart; ++i) {
        const float nb = (float)min<int64_t>(kLnPart, width - (int64_t)i * kLnPart);
        const float mb = pp[2 * i], m2b = pp[2 * i + 1];
        const float nn = cnt + nb;
        const float delta = mb - mu;
        mu += delta * (nb / nn);
        m2 += m2b + delta * delta * (cnt * nb / nn);
        cnt = nn;
    }
    stats[2 * row] = mu;
    stats[2 * row + 1] = 1.f / sqrtf(m2 / cnt + eps);
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
    p.A = A; p.A2 = A; p.B = B; p.C = C;
    p.lda = K; p.lda2 = K; p.ldb = K; p.K1 = K;
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
        hipLaunchKernelGGL((k_gemm_bf16<false, true>), grid, dim3(512), 0, s, p);
    } else {
        hipLaunchKernelGGL((k_gemm_bf16<false, false>), grid, dim3(512), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_ln_finalize(const float *lnp, int64_t M, int64_t d_up, float eps, float *stats,
                              hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_ln_finalize, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, lnp, M,
                       (int)((d_up + kLnPart - 1) / kLnPart), d_up, eps, stats);
    return hipGetLastError();
}

hipError_t launch_gemm_mix_bf16(const uint16_t *h, const uint16_t *x, const float *stats,
                                const float *gamma, const float *beta, const uint16_t *W_mix,
                                uint16_t *out, int64_t M, int64_t d_up, int64_t d_in, int64_t d_out,
                                hipStream_t s) {
    if (M <= 0) return hipSuccess;
    GemmP p = make_plain(h, W_mix, out, M, d_out, d_up + d_in);
    p.lda = d_up;
    p.A2 = x;
    p.lda2 = d_in;
    p.K1 = d_up;
    p.row_stats = stats;
    p.gamma = gamma;
    p.beta = beta;
    hipLaunchKernelGGL((k_gemm_bf16<true, false>), dim3(p.tiles_m * p.tiles_n), dim3(512), 0, s, p);
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
