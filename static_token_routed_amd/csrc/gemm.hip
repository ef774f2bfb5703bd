// The two dense stages of the L^3 layer ("L^3: Large Lookup Layers":
// papernotes.org page, section 整体框架; kimjy99.github.io page, section
// "Method", the layer equation):
//   h   = W_up o            (W_up: d_up x d_emb)
//   out = W_mix [LN(h) ; x]  (W_mix: d_out x (d_up + d_in))
// as bf16 MFMA GEMMs C[M x N] = A[M x K] B[N x K]^T with fp32 accumulation.
//
// Kernel shape (gfx950): 256 threads = 4 wavefronts in 2 x 2, each owning a
// 128 x 128 block of a 256 x 256 output tile as 8 x 8 v_mfma_f32_16x16x32_bf16
// accumulators (256 fp32 per lane, in AGPRs): 64 MFMAs per 16 fragment reads.  A
// second shape, 8 wavefronts in 2 x 4 (128 x 64 each, two per SIMD), serves the
// W_up GEMM, whose short K (d_emb) leaves more of each stage's start exposed.
// K advances 64 columns per stage through two LDS buffers filled by
// asynchronous global -> LDS copies (buffer_load ... lds: no register staging;
// each operand is read through a buffer resource that ends with the matrix, so
// the rows of a ragged edge tile read as zeros instead of being clamped).  The
// copies of stage s + 1 are issued one at a time between stage s's MFMA rows,
// as are the second 32-column step's fragment reads, so neither holds up the
// MFMA issue for long; barriers wait for LDS traffic only, and the loops are
// peeled where the kind of copy changes, so no stage carries a branch.  LDS rows
// are 128 bytes (64 bf16); 16-byte chunk c of row r sits at physical chunk
// c ^ (r & 7) (applied to the copy's source address, since a copy lands at a
// fixed lane-linear slot), so the 16 rows a fragment read touches fall on
// distinct banks.  Per-lane address offsets live in a small LDS table that each
// stage re-reads: kept in registers across the LayerNorm rescale they get
// spilled, and a scratch reload inside the stage loop would wait for every copy
// in flight.  The MFMA takes the B tile as its first operand, so each lane
// holds 4 consecutive output columns of one row: the epilogue stores 8-byte
// segments.  Tiles are numbered so that the workgroups the dispatcher sends to
// one XCD (workgroup id mod 8) form a contiguous, grouped block of tiles,
// sharing A rows and B columns in that XCD's L2.
//
// LayerNorm and the concat [LN(h) ; x] are folded into the W_mix GEMM.  With
// W_mix = [W1 | W2] (columns acting on LN(h) and on x), LN(h) = (h - mean) * rstd
// * gamma + beta per row, W1' = W1 diag(gamma), c1 = W1' 1 and c2 = W1 beta:
//   W_mix [LN(h) ; x] = rstd * (W1' h - mean * c1) + c2 + W2 x.
// A small kernel forms W1' (bf16), c1 and c2 from W_mix, gamma and beta; the GEMM
// then runs over [h | x] against [W1' | W2], rescales its accumulators once,
// when the h columns are done, and adds c2 in the epilogue.  mean and rstd per
// row come from the W_up epilogue's partial statistics (per row and 64-column
// chunk, the mean and the sum of squared deviations of the stored bf16 values),
// merged with Chan's pairwise update.  The concatenated operand never exists in
// memory and the inner loop carries no LayerNorm arithmetic.
#include <algorithm>
#include <type_traits>

#include "cdna4.h"
#include "l3_internal.h"

namespace l3 {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE = BM * BK * 2;          // bytes of one operand tile of a stage
constexpr int SLOT = 2 * TILE;             // one stage (double-buffered)
constexpr int GROUP_M = 4;

struct GemmP {
    const uint16_t *A, *A2;  // A columns [0, K1) from A (row stride lda), [K1, K) from A2 (lda2)
    const uint16_t *B, *B2;  // B columns [0, K1) from B (ldb), [K1, K) from B2 (ldb2)
    uint16_t *C;             // M x N, row stride N (bf16 output)
    float *Cf;               // M x N, row stride N (fp32 output, OUT = 1 write, 2 add)
    int64_t lda, lda2, ldb, ldb2, K1;
    int64_t M, N, K;
    const float *row_stats;  // [M x 2] (mean, rstd) of the A rows in [0, K1)  (LN_IN)
    // (LN_IN, instead of row_stats) per-row shares of o^T G o, [M x quad_npart]: the row's
    // mean is 0 and rstd = 1 / sqrt(max(sum / quad_width, 0) + quad_eps), shares added in order
    const float *quad_parts;
    int quad_npart;
    float quad_width, quad_eps;
    const float *c1, *c2;    // [N] LayerNorm fold terms                         (LN_IN)
    float *ln_out;           // [M x npart_out x 2] partial statistics of the stored rows
    int npart_out;
    int tiles_m, tiles_n;
    int splits;       // OUT == 1: K cut in `splits` ranges of ksplit columns, one output slab each
    int64_t ksplit;
};

// tile id -> (tm, tn): XCD-contiguous, then grouped by GROUP_M tile rows.
__device__ inline void tile_coords(const GemmP &p, int bid, int &tm, int &tn) {
    const int nt = p.tiles_m * p.tiles_n;
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

template <bool LN_IN, bool LN_OUT, int OUT = 0, int NW = 4>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm_bf16(GemmP p) {
    // NW wavefronts: 4 in 2 x 2 (128 x 128 each) or 8 in 2 x 4 (128 x 64 each)
    static_assert(NW == 4 || NW == 8, "wavefronts");
    constexpr int WN = NW == 4 ? 128 : 64;  // output columns per wavefront
    constexpr int NJ = WN / 16;              // their 16-column blocks
    constexpr int CPW = 32 / NW;             // copies per operand, wavefront and stage
    __shared__ __attribute__((aligned(1024))) unsigned char ring[2 * SLOT];
    // LN_IN: (mean, rstd) of the tile's rows; c1 and c2 of its columns
    __shared__ float2 rowst[LN_IN ? BM : 1];
    __shared__ __attribute__((aligned(16))) float c1s[LN_IN ? BN : 1];
    __shared__ __attribute__((aligned(16))) float c2s[LN_IN ? BN : 1];
    // each thread's lane offsets (LaneOffs below), written once, re-read per stage
    __shared__ uint4 lane_tab[64 * NW][2];

    int bid = blockIdx.x;
    if constexpr (OUT == 1) {
        // split K: workgroup bid / tiles takes columns [k0, k0 + ksplit) into slab sp
        if (p.splits > 1) {
            const int nt = p.tiles_m * p.tiles_n;
            const int sp = bid / nt;
            bid -= sp * nt;
            const int64_t k0 = (int64_t)sp * p.ksplit;
            p.A += k0;
            p.B += k0;
            p.A2 = p.A;
            p.B2 = p.B;
            p.K = min(p.ksplit, p.K - k0);
            p.K1 = p.K;
            p.Cf += (int64_t)sp * p.M * p.N;
        }
    }
    int tm, tn;
    tile_coords(p, bid, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wm = NW == 4 ? w >> 1 : w >> 2, wn = NW == 4 ? w & 1 : w & 3;
    const uint32_t ring0 = lds_addr(ring);
    const int nst = (int)(p.K / BK);
    const int nst1 = LN_IN ? (int)(p.K1 / BK) : 0;  // stages over the h columns

    // Copies: 32 per operand and stage, 1 KB = 8 rows x 128 bytes each; wave w issues
    // q = 8w + i.  Lane l fills row 8q + l/8, physical chunk l % 8, with global chunk
    // (l % 8) ^ (l / 8) (= row & 7).  Each operand is read through a buffer resource
    // whose base is the tile's first row and whose size ends with the matrix's last
    // row, so rows past M (N) read as zeros (they only feed accumulators that are
    // never stored).  The lane's row and chunk go in the 32-bit vector offset, the
    // stage's column offset in the scalar offset.  With LN_IN the columns [K1, K)
    // come from A2 and B2 (second pair of resources).
    auto rsrc = [&](const uint16_t *base, int64_t rows_left, int64_t ld, int64_t len) {
        const uint64_t nb = rows_left > 0 ? (uint64_t)(rows_left - 1) * ld * 2 + (uint64_t)len * 2 : 0;
        return make_rsrc(base, (uint32_t)min<uint64_t>(nb, 0xffffffffull));
    };
    const int64_t Ka = LN_IN ? p.K1 : p.K;
    const i32x4_t rA = rsrc(p.A + m0 * p.lda, p.M - m0, p.lda, Ka);
    const i32x4_t rB = rsrc(p.B + n0 * p.ldb, p.N - n0, p.ldb, Ka);
    i32x4_t rA2{}, rB2{};
    if constexpr (LN_IN) {
        rA2 = rsrc(p.A2 + m0 * p.lda2, p.M - m0, p.lda2, p.K - p.K1);
        rB2 = rsrc(p.B2 + n0 * p.ldb2, p.N - n0, p.ldb2, p.K - p.K1);
    }

    // Per-lane offsets: fragment reads (16-row block rb, 32-column step ks: row
    // 16 rb + (l & 15) of the wave's rows, logical chunk 4 ks + l/16 at physical chunk
    // (4 ks + l/16) ^ (l & 7)) and copy sources of the columns [0, K1) (vA, vB) and
    // [K1, K) (vA2, vB2).  Computed once into LDS and read back at the start of every
    // stage: kept in registers they would live across the LayerNorm rescale, whose
    // register pressure gets them spilled to scratch, and scratch reloads inside the
    // stage loop wait for every copy in flight.
    struct LaneOffs { uint32_t fA[2], fB[2], vA, vB, vA2, vB2; };
    {
        const uint32_t l = threadIdx.x & 63;
        uint32_t fa[2], fb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint32_t c = 16 * ((4 * ks + (l >> 4)) ^ (l & 7));
            fa[ks] = (uint32_t)(wm * 128 + (l & 15)) * 128 + c;
            fb[ks] = TILE + (uint32_t)(wn * WN + (l & 15)) * 128 + c;
        }
        const uint32_t gch = (l & 7) ^ (l >> 3), rl = 8 * CPW * w + (l >> 3);
        lane_tab[threadIdx.x][0] = make_uint4(fa[0], fa[1], fb[0], fb[1]);
        lane_tab[threadIdx.x][1] = make_uint4(rl * (uint32_t)(p.lda * 2) + gch * 16,
                                              rl * (uint32_t)(p.ldb * 2) + gch * 16,
                                              rl * (uint32_t)(p.lda2 * 2) + gch * 16,
                                              rl * (uint32_t)(p.ldb2 * 2) + gch * 16);
    }
    auto lane_offs = [&]() {
        const uint32_t t = 64 * w + fresh_lane_id();  // = threadIdx.x, not kept live
        const uint4 a = lane_tab[t][0], b = lane_tab[t][1];
        LaneOffs o;
        o.fA[0] = a.x; o.fA[1] = a.y; o.fB[0] = a.z; o.fB[1] = a.w;
        o.vA = b.x; o.vB = b.y; o.vA2 = b.z; o.vB2 = b.w;
        return o;
    };
    const uint32_t sA = (uint32_t)(16 * p.lda), sB = (uint32_t)(16 * p.ldb);  // 8 rows
    const uint32_t sA2 = (uint32_t)(16 * p.lda2), sB2 = (uint32_t)(16 * p.ldb2);

    // Copy c (0..15: operand c & 1, index c >> 1) of stage st.  KIND 1: columns
    // [0, K1); 2: columns [K1, K) if st >= nst1, else [0, K1) (scalar selects, no
    // branch); 0: none (last stage).  The empty asm keeps the 16 per-copy offsets from
    // being hoisted out of the stage loop as 16 more live registers.
    auto issue_one = [&](auto kind, int st, int c, const LaneOffs &o) {
        constexpr int KIND = decltype(kind)::value;
        const uint32_t base = ring0 + (uint32_t)((st & 1) * SLOT);
        const int i = c >> 1;
        const uint32_t off = (uint32_t)((CPW * w + i) * 1024) + ((c & 1) ? TILE : 0);
        if constexpr (KIND == 1) {
            uint32_t v = (c & 1) ? o.vB : o.vA;
            __asm__ volatile("" : "+v"(v));
            const uint32_t so = (uint32_t)st * (BK * 2);
            if (c & 1) async_buf16(rB, v + i * sB, so, base + off);
            else async_buf16(rA, v + i * sA, so, base + off);
        } else if constexpr (KIND == 2 && LN_IN) {
            const bool sec = st >= nst1;
            uint32_t v = (c & 1) ? (sec ? o.vB2 : o.vB) : (sec ? o.vA2 : o.vA);
            __asm__ volatile("" : "+v"(v));
            const uint32_t so = (uint32_t)(sec ? st - nst1 : st) * (BK * 2);
            if (c & 1) async_buf16(sec ? rB2 : rB, v + i * (sec ? sB2 : sB), so, base + off);
            else async_buf16(sec ? rA2 : rA, v + i * (sec ? sA2 : sA), so, base + off);
        }
    };

    f32x4_t acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // LN_IN: the tile's row statistics and column terms, loaded while the first stage's
    // copies are in flight (the wait for these loads also covers the copies, which were
    // issued first); the first stage's barrier publishes them
    auto load_ln = [&]() {
        if constexpr (LN_IN) {
        const int t = threadIdx.x;
        if (t < 256) {
            const int64_t m = min<int64_t>(m0 + t, p.M - 1), n = min<int64_t>(n0 + t, p.N - 1);
            const float c1v = p.c1[n], c2v = p.c2[n];
            if (p.quad_parts) {
                // the shares in groups of 8 loads, added in order
                const float *qp = p.quad_parts + m * p.quad_npart;
                float q = 0.f;
                for (int i0 = 0; i0 < p.quad_npart; i0 += 8) {
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = i0 + i < p.quad_npart ? qp[i0 + i] : 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (i0 + i < p.quad_npart) q += v[i];
                }
                rowst[t] = make_float2(0.f, 1.f / sqrtf(fmaxf(q / p.quad_width, 0.f) + p.quad_eps));
            } else {
                rowst[t] = make_float2(p.row_stats[2 * m], p.row_stats[2 * m + 1]);
            }
            c1s[t] = c1v;
            c2s[t] = c2v;
        }
        }
    };
    // the accumulators pinned to AGPRs around the rescale, so the stage loops on either
    // side keep them in place instead of shuffling them between registers
    auto pin_acc = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) __asm__ volatile("" : "+a"(acc[i][j]));
    };
    // after the h columns: acc = rstd * (acc - mean * c1) per element, one 16-row
    // block at a time (few live VGPRs)
    auto fold = [&]() {
        const uint32_t l = fresh_lane_id();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float2 st2 = rowst[wm * 128 + 16 * i + (l & 15)];
            const float rm = st2.x * st2.y;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float4 c4 = *reinterpret_cast<const float4 *>(&c1s[wn * WN + 16 * j + 4 * (l >> 4)]);
                acc[i][j][0] = fmaf(-rm, c4.x, st2.y * acc[i][j][0]);
                acc[i][j][1] = fmaf(-rm, c4.y, st2.y * acc[i][j][1]);
                acc[i][j][2] = fmaf(-rm, c4.z, st2.y * acc[i][j][2]);
                acc[i][j][3] = fmaf(-rm, c4.w, st2.y * acc[i][j][3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One stage: wait for its copies (the only global loads in flight), barrier, then
    // two 32-column steps of 64 MFMAs.  Between the MFMA rows of the first step the
    // second step's fragments are read (the first step's come first, in the order the
    // MFMAs use them), and between all rows the next stage's copies (of kind KIND) are
    // issued, one at a time, so neither blocks the MFMA issue for long.
    auto stage = [&](auto kind, int st) {
        const LaneOffs o = lane_offs();
        wait_vmcnt<0>();
        lds_barrier();
        const unsigned char *sb = ring + (st & 1) * SLOT;
        auto rd = [&](uint32_t a) { return *reinterpret_cast<const bf16x8_t *>(sb + a); };
        bf16x8_t fa0[8], fb0[NJ], fa1[8], fb1[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb0[j] = rd(o.fB[0] + 2048 * j);
        fa0[0] = rd(o.fA[0]);
        fa0[1] = rd(o.fA[0] + 2048);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0);
            if (i + 2 < 8) fa0[i + 2] = rd(o.fA[0] + 2048 * (i + 2));
            if (i < NJ) fb1[i] = rd(o.fB[1] + 2048 * i);
            fa1[i] = rd(o.fA[1] + 2048 * i);
            // 2 CPW copies per stage over the 16 MFMA rows: every row (4 wavefronts) or
            // every other row (8)
            if constexpr (NW == 4) issue_one(kind, st + 1, 2 * i, o);
            else if (i % 2 == 0) issue_one(kind, st + 1, i / 2, o);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb1[j], fa1[i], acc[i][j], 0, 0, 0);
            if constexpr (NW == 4) issue_one(kind, st + 1, 2 * i + 1, o);
            else if (i % 2 == 0) issue_one(kind, st + 1, 4 + i / 2, o);
            __builtin_amdgcn_sched_barrier(0);
        }
        pin_acc();
    };
    using KNone = std::integral_constant<int, 0>;
    using KFirst = std::integral_constant<int, 1>;
    using KSel = std::integral_constant<int, 2>;
    if constexpr (!LN_IN) {
        // the last stage is peeled so no stage carries a branch
        {
            const LaneOffs o = lane_offs();
#pragma unroll
            for (int c = 0; c < 2 * CPW; ++c) issue_one(KFirst{}, 0, c, o);
        }
        for (int st = 0; st < nst - 1; ++st) stage(KFirst{}, st);
        stage(KNone{}, nst - 1);
    } else {
        // the h stages (the last one issues the first x stage's copies), the rescale
        // while those are in flight, then the x stages (nst > nst1: d_in >= 64)
        {
            const LaneOffs o = lane_offs();
#pragma unroll
            for (int c = 0; c < 2 * CPW; ++c) issue_one(KFirst{}, 0, c, o);
        }
        load_ln();
        for (int st = 0; st < nst1; ++st) stage(KSel{}, st);
        pin_acc();
        fold();
        pin_acc();
        for (int st = nst1; st < nst - 1; ++st) stage(KSel{}, st);
        stage(KNone{}, nst - 1);
    }

    pin_acc();
    // Epilogue.  acc[i][j] element e of lane l: row m0 + wm*128 + 16i + (l & 15),
    // column n0 + wn*128 + 16j + 4(l/16) + e.
    const uint32_t lane = fresh_lane_id();
    const int64_t nbase = n0 + wn * WN;
    auto epilogue = [&](auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        // OUT 3: the A values at this lane's output positions (A is M x K with K = N),
        // all loads issued before the first use
        uint2 av[OUT == 3 ? 8 : 1][OUT == 3 ? NJ : 1];
        if constexpr (OUT == 3) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t m = m0 + wm * 128 + 16 * i + (lane & 15);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int64_t n = nbase + 16 * j + 4 * (lane >> 4);
                    av[i][j] = (FULL || (m < p.M && n < p.N))
                                   ? *reinterpret_cast<const uint2 *>(p.A + m * p.lda + n)
                                   : make_uint2(0u, 0u);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t m = m0 + wm * 128 + 16 * i + (lane & 15);
            uint32_t pk[LN_OUT ? NJ : 1][2];  // the stored bf16 values (all kept for LN_OUT)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int64_t n = nbase + 16 * j + 4 * (lane >> 4);
                if constexpr (LN_IN) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(&c2s[wn * WN + 16 * j + 4 * (lane >> 4)]);
                    acc[i][j][0] += c4.x;
                    acc[i][j][1] += c4.y;
                    acc[i][j][2] += c4.z;
                    acc[i][j][3] += c4.w;
                }
                if constexpr (OUT == 0) {
                    pk[j & (LN_OUT ? NJ - 1 : 0)][0] = pack2(acc[i][j][0], acc[i][j][1]);
                    pk[j & (LN_OUT ? NJ - 1 : 0)][1] = pack2(acc[i][j][2], acc[i][j][3]);
                }
                if (OUT != 3 && (FULL || (m < p.M && n < p.N))) {
                    if constexpr (OUT == 0) {
                        *reinterpret_cast<uint2 *>(p.C + m * p.N + n) =
                            make_uint2(pk[j & (LN_OUT ? NJ - 1 : 0)][0], pk[j & (LN_OUT ? NJ - 1 : 0)][1]);
                    } else if constexpr (OUT != 3) {
                        float4 *dst = reinterpret_cast<float4 *>(p.Cf + m * p.N + n);
                        float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
                        if constexpr (OUT == 2) {
                            const float4 c = *dst;
                            v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
                        }
                        *dst = v;
                    }
                }
            }
            if constexpr (OUT == 3) {
                // the wavefront's share of row m's quadratic form sum_n C[m][n] A[m][n]
                // (its WN columns; zero-filled A past the edges)
                float q = 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    q = fmaf(acc[i][j][0], bf_lo(av[i][j].x), q);
                    q = fmaf(acc[i][j][1], bf_hi(av[i][j].x), q);
                    q = fmaf(acc[i][j][2], bf_lo(av[i][j].y), q);
                    q = fmaf(acc[i][j][3], bf_hi(av[i][j].y), q);
                }
                q += __shfl_xor(q, 16);
                q += __shfl_xor(q, 32);
                if (lane < 16 && (FULL || (m < p.M && nbase < p.N)))
                    p.ln_out[m * p.npart_out + nbase / WN] = q;
            }
            if constexpr (LN_OUT && OUT == 0) {
                // partial statistics over each 64 columns (4 blocks of 16) of this row's
                // stored (bf16) values
                auto stored = [&](int j, int e) {
                    const uint32_t w2 = pk[j][e >> 1];
                    const float v = __uint_as_float((e & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
                    if constexpr (FULL) return v;
                    const int64_t n = nbase + 16 * j + 4 * (lane >> 4) + e;
                    return n < p.N ? v : 0.f;
                };
#pragma unroll
                for (int part = 0; part < NJ / 4; ++part) {
                    const int64_t c0 = nbase + 64 * part;
                    const int64_t width = FULL ? kLnPart : min<int64_t>(kLnPart, p.N - c0);
                    if (!FULL && width <= 0) continue;
                    float sum = 0.f;
#pragma unroll
                    for (int j = 4 * part; j < 4 * part + 4; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sum += stored(j, e);
                    sum += __shfl_xor(sum, 16);
                    sum += __shfl_xor(sum, 32);
                    // kLnPart is a power of two: the product is the exact quotient
                    const float mean = FULL ? sum * (1.f / kLnPart) : sum / (float)width;
                    float q = 0.f;
#pragma unroll
                    for (int j = 4 * part; j < 4 * part + 4; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float dv = stored(j, e) - mean;
                            if constexpr (FULL) {
                                q += dv * dv;
                            } else {
                                const int64_t n = nbase + 16 * j + 4 * (lane >> 4) + e;
                                q += n < p.N ? dv * dv : 0.f;
                            }
                        }
                    q += __shfl_xor(q, 16);
                    q += __shfl_xor(q, 32);
                    if (lane < 16 && (FULL || m < p.M)) {
                        float *dst = p.ln_out + (m * p.npart_out + c0 / kLnPart) * 2;
                        dst[0] = mean;
                        dst[1] = q;
                    }
                }
            }
        }
    };
    // (only the GEMMs that reduce their rows in the epilogue, whose per-element work
    // that doubles, get the unchecked copy; the others keep one copy of the code)
    if ((LN_OUT || OUT == 3) && m0 + BM <= p.M && n0 + BN <= p.N) epilogue(std::true_type{});
    else epilogue(std::false_type{});
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
                                                  const float *__restrict__ beta, int accum) {
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
            if (m < M && n < N) C[m * N + n] = accum ? C[m * N + n] + acc[i][j] : acc[i][j];
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

// LayerNorm fold terms of W_mix (one workgroup per output row n):
// W1'[n][k] = bf16(W_mix[n][k] * gamma[k]) for k < d_up, c1[n] = sum_k W1'[n][k],
// c2[n] = sum_k W_mix[n][k] * beta[k]  (fp32 sums).
__global__ __launch_bounds__(256) void k_mix_fold(const uint16_t *__restrict__ W_mix,
                                                  const float *__restrict__ gamma,
                                                  const float *__restrict__ beta, int64_t d_up,
                                                  int64_t ld, uint16_t *__restrict__ w1p,
                                                  float *__restrict__ c1, float *__restrict__ c2) {
    __shared__ float red[2][4];
    const int64_t n = blockIdx.x;
    const uint16_t *row = W_mix + n * ld;
    float s1 = 0.f, s2 = 0.f;
    for (int64_t k = 8 * threadIdx.x; k < d_up; k += 8 * 256) {
        const uint4 u = *reinterpret_cast<const uint4 *>(row + k);
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float w0 = bf_lo(uu[e]), w1 = bf_hi(uu[e]);
            o[e] = pack2(w0 * gamma[k + 2 * e], w1 * gamma[k + 2 * e + 1]);
            s1 += bf_lo(o[e]) + bf_hi(o[e]);
            s2 = fmaf(w0, beta[k + 2 * e], s2);
            s2 = fmaf(w1, beta[k + 2 * e + 1], s2);
        }
        *reinterpret_cast<uint4 *>(w1p + n * d_up + k) = make_uint4(o[0], o[1], o[2], o[3]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s1 += __shfl_xor(s1, o);
        s2 += __shfl_xor(s2, o);
    }
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = s1;
        red[1][threadIdx.x >> 6] = s2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        c1[n] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        c2[n] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    }
}

size_t mix_fold_w1p_bytes(int64_t d_up, int64_t d_out) {
    return ((size_t)d_out * d_up * 2 + 255) & ~(size_t)255;
}

// C[i] += sum of the split-K slabs at i, in slab order (float4 per thread)
__global__ __launch_bounds__(256) void k_split_add(const float4 *__restrict__ part, int splits, int64_t n4,
                                                   float4 *__restrict__ C) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 acc = part[i];
    for (int sp = 1; sp < splits; ++sp) {
        const float4 v = part[(int64_t)sp * n4 + i];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float4 c = C[i];
    c.x += acc.x; c.y += acc.y; c.z += acc.z; c.w += acc.w;
    C[i] = c;
}

GemmP make_plain(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M, int64_t N, int64_t K) {
    GemmP p{};
    p.A = A; p.A2 = A; p.B = B; p.B2 = B; p.C = C;
    p.lda = K; p.lda2 = K; p.ldb = K; p.ldb2 = K; p.K1 = K;
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
        // W_up: K = d_emb is short, so two wavefronts per SIMD (8 per tile) hide more of
        // each stage's start than one
        hipLaunchKernelGGL((k_gemm_bf16<false, true, 0, 8>), grid, dim3(512), 0, s, p);
    } else {
        hipLaunchKernelGGL((k_gemm_bf16<false, false>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- factored W_mix
//
// With h = W_up o, LayerNorm's centred row is h - mean(h) 1 = W_c o, where W_c is W_up
// with each column's mean over the rows taken away (mean(h) = wbar . o, wbar the
// column means), and W_mix [LN(h) ; x] = W1 diag(gamma) (h - mean) rstd + W1 beta + W2 x
//   = rstd * (F o) + c2 + W2 x,   F = W1 diag(gamma) W_c  (d_out x d_emb),  c2 = W1 beta.
// So the W_mix GEMM runs over [o | x] (K = d_emb + d_in) instead of [h | x]
// (K = d_up + d_in).  h itself is never formed: LayerNorm needs only its variance,
// var = |W_c o|^2 / d_up = o^T G o / d_up with the Gram matrix G = W_c^T W_c
// (d_emb x d_emb), and the GEMM o G^T with a quadratic-form epilogue gives
// o^T G o per row at a quarter of W_up's work when d_up = 4 d_emb.  F and G are
// formed per call from the weights: W_c^T (W_up transposed, each row less its
// mean, bf16) is written right after W1' = W1 diag(gamma) (from k_mix_fold), so
// the rows [W1' ; W_c^T] are one (d_out + d_emb) x d_up matrix, and one GEMM of it
// against W_c^T gives [F ; G] in the layouts the two GEMMs read.
// Centring first means no mean * (row sum) term is subtracted later, so a large
// mean cancels nothing in bf16.

// W_up^T [d_emb x d_up] (bf16, from the transpose) centred in place: one wavefront
// per row c subtracts the row's mean (the mean of W_up's column c) and rounds to bf16;
// lanes take 8 consecutive elements at a time (cols is a multiple of 64).  The first
// workgroup also zeroes `zero` [nz] (the factored GEMM's mean coefficients).
__global__ __launch_bounds__(256) void k_center_rows(uint16_t *__restrict__ WT, int64_t rows, int64_t cols,
                                                     float *__restrict__ zero, int64_t nz) {
    if (blockIdx.x == 0)
        for (int64_t i = threadIdx.x; i < nz; i += 256) zero[i] = 0.f;
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    uint4 *row = reinterpret_cast<uint4 *>(WT + r * cols);
    const int64_t nv = cols / 8;
    float sum = 0.f;
    for (int64_t c = lane; c < nv; c += 64) {
        const uint4 u = row[c];
        sum += ((bf_lo(u.x) + bf_hi(u.x)) + (bf_lo(u.y) + bf_hi(u.y))) +
               ((bf_lo(u.z) + bf_hi(u.z)) + (bf_lo(u.w) + bf_hi(u.w)));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    const float mean = sum / (float)cols;
    for (int64_t c = lane; c < nv; c += 64) {
        const uint4 u = row[c];
        row[c] = make_uint4(pack2(bf_lo(u.x) - mean, bf_hi(u.x) - mean), pack2(bf_lo(u.y) - mean, bf_hi(u.y) - mean),
                            pack2(bf_lo(u.z) - mean, bf_hi(u.z) - mean), pack2(bf_lo(u.w) - mean, bf_hi(u.w) - mean));
    }
}

// (mean, rstd) per row from the quadratic-form partials: var = (sum of the row's
// npart partials) / width, clamped at zero (G's rounding can leave a tiny negative
// value for a row whose variance is zero).  The mean is not needed (the factored
// GEMM's mean coefficients are zero) and is written as 0.
constexpr int kQuadWN = 64;  // output columns per wavefront of k_gemm_bf16<.., 3, 8>

int ln_quad_parts(int64_t d_emb) { return (int)((d_emb + kQuadWN - 1) / kQuadWN); }

hipError_t launch_ln_quad_stats_bf16(const uint16_t *o, const void *factor_ws, int64_t M, int64_t d_emb,
                                     int64_t d_up, int64_t d_out, float *qp, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const uint16_t *G = reinterpret_cast<const uint16_t *>(
                            static_cast<const char *>(factor_ws) + al((size_t)(d_out + d_emb) * d_up * 2)) +
                        d_out * d_emb;
    GemmP p = make_plain(o, G, nullptr, M, d_emb, d_emb);
    p.ln_out = qp;
    p.npart_out = ln_quad_parts(d_emb);
    // 8 wavefronts in 2 x 4, each kQuadWN columns wide
    hipLaunchKernelGGL((k_gemm_bf16<false, false, 3, 8>), dim3(p.tiles_m * p.tiles_n), dim3(512), 0, s, p);
    return hipGetLastError();
}

// factor_ws: [W1' ; W_c^T] ((d_out + d_emb) x d_up bf16), [F ; G] ((d_out + d_emb) x
// d_emb bf16), the d_out zeros; each region 256-byte aligned.
size_t mix_factor_bytes(int64_t d_emb, int64_t d_up, int64_t d_out) {
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    return al((size_t)(d_out + d_emb) * d_up * 2) + al((size_t)(d_out + d_emb) * d_emb * 2) +
           al((size_t)d_out * 4);
}

// [F ; G] = [W1' ; W_c^T] W_c runs on the 256 x 256 tile kernel over the whole K = d_up
// (bf16 output): few workgroups and no partial sums in memory, so it leaves the chip
// and its memory to the route it runs beside; it is needed only after the gather.
hipError_t launch_mix_factor(const uint16_t *W_up, const uint16_t *W_mix, const float *gamma,
                             const float *beta, void *fold_ws, void *factor_ws, int64_t d_emb,
                             int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s) {
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    char *f = static_cast<char *>(factor_ws);
    uint16_t *stack = reinterpret_cast<uint16_t *>(f);  // W1' rows, then W_c^T rows
    uint16_t *wct = stack + d_out * d_up;
    uint16_t *fg = reinterpret_cast<uint16_t *>(f + al((size_t)(d_out + d_emb) * d_up * 2));
    float *zero = reinterpret_cast<float *>(reinterpret_cast<char *>(fg) + al((size_t)(d_out + d_emb) * d_emb * 2));
    // W_c^T: W_up transposed, then each row less its mean
    hipError_t e = launch_transpose(W_up, d_emb, d_up, d_emb, wct, d_up, d_up, L3_BF16, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_center_rows, dim3((unsigned)((d_emb + 3) / 4)), dim3(256), 0, s, wct, d_emb, d_up,
                       zero, d_out);
    // W1' into the stack's first d_out rows; c1, c2 into fold_ws
    float *c1 = reinterpret_cast<float *>(static_cast<char *>(fold_ws) + mix_fold_w1p_bytes(d_up, d_out));
    hipLaunchKernelGGL(k_mix_fold, dim3((unsigned)d_out), dim3(256), 0, s, W_mix, gamma, beta, d_up,
                       d_up + d_in, stack, c1, c1 + d_out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // [F ; G] = [W1' ; W_c^T] W_c  (row i of the product: stack row i against each W_c^T row)
    return launch_gemm_bf16(stack, wct, fg, d_out + d_emb, d_emb, d_up, nullptr, s);
}

hipError_t launch_gemm_mix_factored_bf16(const uint16_t *o, const uint16_t *x, const float *qp, float eps,
                                         const uint16_t *W_mix, uint16_t *out, const void *fold_ws,
                                         const void *factor_ws, int64_t M, int64_t d_emb, int64_t d_up,
                                         int64_t d_in, int64_t d_out, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const char *f = static_cast<const char *>(factor_ws);
    const uint16_t *fm = reinterpret_cast<const uint16_t *>(f + al((size_t)(d_out + d_emb) * d_up * 2));
    const float *zero = reinterpret_cast<const float *>(reinterpret_cast<const char *>(fm) +
                                                        al((size_t)(d_out + d_emb) * d_emb * 2));
    const float *c2 = reinterpret_cast<const float *>(static_cast<const char *>(fold_ws) +
                                                      mix_fold_w1p_bytes(d_up, d_out)) + d_out;
    GemmP p = make_plain(o, fm, out, M, d_out, d_emb + d_in);
    p.lda = d_emb;
    p.ldb = d_emb;
    p.A2 = x;
    p.lda2 = d_in;
    p.B2 = W_mix + d_up;
    p.ldb2 = d_up + d_in;
    p.K1 = d_emb;
    p.quad_parts = qp;  // rstd per row from the statistics GEMM's shares, in the prologue
    p.quad_npart = ln_quad_parts(d_emb);
    p.quad_width = (float)d_up;
    p.quad_eps = eps;
    p.c1 = zero;  // F acts on the centred row: no mean term
    p.c2 = c2;
    hipLaunchKernelGGL((k_gemm_bf16<true, false>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16_f32out(const uint16_t *A, const uint16_t *B, float *C, int64_t M,
                                   int64_t N, int64_t K, bool accumulate, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    GemmP p = make_plain(A, B, nullptr, M, N, K);
    p.Cf = C;
    const dim3 grid(p.tiles_m * p.tiles_n);
    if (accumulate) hipLaunchKernelGGL((k_gemm_bf16<false, false, 2>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_gemm_bf16<false, false, 1>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

int gemm_f32_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return (int)std::max<int64_t>(1, std::min<int64_t>(256 / std::max<int64_t>(tiles, 1), K / 2048));
}

size_t gemm_f32_split_bytes(int64_t M, int64_t N, int64_t K) {
    const int sp = gemm_f32_splits(M, N, K);
    return sp > 1 ? (size_t)sp * M * N * 4 : 0;
}

hipError_t launch_gemm_bf16_f32acc_split(const uint16_t *A, const uint16_t *B, float *C, int64_t M,
                                         int64_t N, int64_t K, float *part, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int sp = gemm_f32_splits(M, N, K);
    if (sp <= 1 || !part) return launch_gemm_bf16_f32out(A, B, C, M, N, K, true, s);
    GemmP p = make_plain(A, B, nullptr, M, N, K);
    p.Cf = part;
    p.splits = sp;
    p.ksplit = ((K + sp - 1) / sp + BK - 1) / BK * BK;
    p.splits = (int)((K + p.ksplit - 1) / p.ksplit);
    hipLaunchKernelGGL((k_gemm_bf16<false, false, 1>), dim3(p.tiles_m * p.tiles_n * p.splits), dim3(256), 0,
                       s, p);
    const int64_t n4 = M * N / 4;
    hipLaunchKernelGGL(k_split_add, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       (const float4 *)part, p.splits, n4, (float4 *)C);
    return hipGetLastError();
}

hipError_t launch_ln_finalize(const float *lnp, int64_t M, int64_t d_up, float eps, float *stats,
                              hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_ln_finalize, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, lnp, M,
                       (int)((d_up + kLnPart - 1) / kLnPart), d_up, eps, stats);
    return hipGetLastError();
}

hipError_t launch_mix_fold(const uint16_t *W_mix, const float *gamma, const float *beta,
                           void *fold_ws, int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s) {
    uint16_t *w1p = static_cast<uint16_t *>(fold_ws);
    float *c1 = reinterpret_cast<float *>(static_cast<char *>(fold_ws) + mix_fold_w1p_bytes(d_up, d_out));
    hipLaunchKernelGGL(k_mix_fold, dim3((unsigned)d_out), dim3(256), 0, s, W_mix, gamma, beta, d_up,
                       d_up + d_in, w1p, c1, c1 + d_out);
    return hipGetLastError();
}

hipError_t launch_gemm_mix_bf16(const uint16_t *h, const uint16_t *x, const float *stats,
                                const uint16_t *W_mix, uint16_t *out, const void *fold_ws, int64_t M,
                                int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const uint16_t *w1p = static_cast<const uint16_t *>(fold_ws);
    const float *c1 = reinterpret_cast<const float *>(static_cast<const char *>(fold_ws) +
                                                      mix_fold_w1p_bytes(d_up, d_out));
    GemmP p = make_plain(h, w1p, out, M, d_out, d_up + d_in);
    p.lda = d_up;
    p.ldb = d_up;
    p.A2 = x;
    p.lda2 = d_in;
    p.B2 = W_mix + d_up;
    p.ldb2 = d_up + d_in;
    p.K1 = d_up;
    p.row_stats = stats;
    p.c1 = c1;
    p.c2 = c1 + d_out;
    hipLaunchKernelGGL((k_gemm_bf16<true, false>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
    return hipGetLastError();
}

size_t mix_fold_bytes(int64_t d_up, int64_t d_out) {
    return mix_fold_w1p_bytes(d_up, d_out) + (size_t)d_out * 2 * 4;
}

hipError_t launch_gemm_f32(const float *A, const float *B, float *C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL((k_gemm_f32<false>), grid, dim3(256), 0, s, A, (const float *)nullptr, B, C,
                       M, N, K, K, (const float *)nullptr, (const float *)nullptr,
                       (const float *)nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_gemm_f32_acc(const float *A, const float *B, float *C, int64_t M, int64_t N,
                               int64_t K, bool accumulate, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL((k_gemm_f32<false>), grid, dim3(256), 0, s, A, (const float *)nullptr, B, C,
                       M, N, K, K, (const float *)nullptr, (const float *)nullptr,
                       (const float *)nullptr, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_ln_stats_f32(const float *h, int64_t M, int64_t d_up, float eps, float *stats,
                               hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_ln_stats_f32, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, h, M, d_up, eps,
                       stats);
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
                       d_up + d_in, d_up, (const float *)stats, gamma, beta, 0);
    return hipGetLastError();
}

}  // namespace l3
