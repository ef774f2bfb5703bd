// Internal declarations of the L^3 forward library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/l3.h"

#define L3_HIP_TRY(expr)                                   \
    do {                                                   \
        hipError_t e_ = (expr);                            \
        if (e_ != hipSuccess) return L3_ERR_HIP;           \
    } while (0)

namespace l3 {

constexpr int kSortTile = 512;     // keys ranked per workgroup and pass
constexpr int kSortPer = kSortTile / 256;  // keys per thread of a 256-thread tile
static_assert(kSortTile % 256 == 0 && kSortPer <= 32, "sort tile");
constexpr int kRouteSmallMax = 1024;  // batches up to this size are routed by one workgroup
constexpr int kSmallThreads = 1024;   // its threads (one token each)
constexpr int kRadixBits = 9;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kLnPart = 64;        // LayerNorm partial statistics cover 64 features
constexpr int kHeavyTile = 32;     // tokens per MFMA gather-attention work item
constexpr int kHeavyMinTokens = 8; // blocks with at least this many tokens use the MFMA path
constexpr int kHeavyMinRows = 64;  // ... and so do blocks with at least this many rows
// Streaming items are taken longest first, in three classes by the block's rows: at least
// kHeavyLongRows (the heavy list's front), at least kHeavyMidRows (its back), the rest
// (the back of the dense list, whose front holds the dense items: the two never meet, as
// every item holds at least one token of the batch)
constexpr int kHeavyLongRows = 256;
constexpr int kHeavyMidRows = 128;
// Radix scatter: up to this many 512-key tiles each workgroup forms its own digit
// offsets from the whole histogram; past it a scan launch forms them all first (from
// 32 tiles on, the extra launch costs less than every workgroup reading the histogram)
constexpr int kScatterDirectTiles = 16;
constexpr int kHeavyMinTokensWide = 64;  // the token threshold at d_in 4096
constexpr int kDenseTile = 64;     // tokens per dense work item (long blocks of the Zipf head)
constexpr int kDenseMinTokens = 33;  // blocks with at least this many tokens ...
constexpr int kDenseMaxD = 512;    // ... and at most this many rows take dense items
constexpr int kDenseMinD = 64;     // ... and at least this many (a dense item's stages over
                                   // d_in cost the same for any d_t, so few rows waste them)

// Workspace header (int32 words), zeroed at the start of every call.
enum { HDR_ERR = 0, HDR_NSEG = 1, HDR_NLIGHT = 2, HDR_NHEAVY = 3, HDR_NDENSE = 4, HDR_NKV = 5,
       HDR_NSPLIT = 6, HDR_NLIGHT_LONG = 7,
       HDR_QUEUE = 8,           // 8 per-XCD counters of the matrix-core gather, then its dense counter
       HDR_NLIGHT_MID = 17,
       HDR_NHEAVY_SHORT = 18,   // streaming items of blocks in [kHeavyMidRows, kHeavyLongRows) rows
       HDR_NHEAVY_TAIL = 19,    // streaming items of blocks under kHeavyMidRows rows
       HDR_NLIGHT_SHORT = 20,   // light items of blocks under kLightShortRows rows (light's back)
       HDR_WORDS = 64 };
// Light items of blocks with at least kLightLongRows rows, then those with at least
// kLightMidRows, are listed apart and taken first, so the longest start first: the
// former from the front of the light_long region, the latter from its back.
constexpr int kLightLongRows = 32;
constexpr int kLightMidRows = 16;
// The other light items: those of blocks with at least kLightShortRows rows from the
// front of the light list, the rest from its back, so the wavefronts' shares (dealt in
// snake order) start with the longer ones and even out.
constexpr int kLightShortRows = 8;

struct Dims {
    int64_t d_in, d_emb, d_up, d_out;
    int dtype;
    float eps;
};
// bf16 plans with d_emb above 512 (1024, 2048; d_in = d_emb) serve tied tables only: the
// forward requires W_V to be the W_K buffer, and the wavefront gather kernel takes
// every block
inline bool tied_only(const Dims &d) { return d.dtype == L3_BF16 && d.d_emb > 512; }

// Byte offsets of the workspace regions for n_max tokens.
struct WsLayout {
    size_t hdr, keys_a, vals_a, keys_b, vals_b, rank, hist, tile_cnt;
    size_t inv_perm, uniq, counts, seg_start, light, light_long, heavy, dense;
    size_t scores;  // fp32 path only: n x max_d
    size_t o, h, lnp;
    size_t stats;  // LayerNorm row statistics (mean, rstd)
    size_t fold;   // LayerNorm fold of W_mix (bf16 path)
    size_t factor; // the factored W_mix's F and its temporaries (bf16, n > kSkinnyMaxM)
    size_t part;   // split-K partial slabs of the small-M path (bf16 path, n <= kSkinnyMaxM)
    // split-row gather-attention of small batches (split_slots() > 0): row-chunk
    // items, per-block {slot base, chunks, tokens, first sorted position}, each sorted
    // position's block, and per (token, chunk) partial (max, sum) and output rows
    size_t sitems, blkinfo, blk_of, pml, po;
    int64_t slots;  // 0: the small-batch split path is off for this size
    size_t total;
    int64_t ntiles;
};

WsLayout ws_layout(const Dims &d, int64_t n_max, int32_t max_d);

template <typename T>
inline T *ws_ptr(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

// Route outputs inside (or outside) the workspace.
struct RouteBufs {
    int32_t *hdr;
    int32_t *keys_a, *vals_a, *keys_b, *vals_b, *rank, *hist, *tile_cnt;
    int32_t *sorted_ids;  // final keys
    int32_t *perm;        // final values
    int32_t *inv_perm, *uniq, *counts, *seg_start;
};

// ---- launchers (all enqueue on `s`; return hipError_t of the last launch)
hipError_t launch_zero_i32(int32_t *p, int64_t count, hipStream_t s);
// The multi-kernel route; it also clears the header (the first sort pass) and
// sets the out-of-range flag (the block writer), so no separate clear is needed.  Its
// block writer also forms the blocks' sizes and, with light non-null, their work items
// (the lists and thresholds of launch_worklist).  tile_cnt holds 2 ntiles words.
hipError_t launch_route(const int32_t *ids, int64_t n, int64_t vocab, RouteBufs &b, int64_t ntiles,
                        const int64_t *off, int heavy_min_tokens, int dense_min_tokens, int light_tokens,
                        int4 *light, int2 *heavy, int2 *dense, int4 *light_long, hipStream_t s);
// Work lists for the gather-attention kernels (reads the route outputs).
// Blocks go to the dense list (>= dense_min_tokens tokens, kDenseMinD <= d_t <= kDenseMaxD, items of
// kDenseTile tokens), else the heavy list (>= heavy_min_tokens tokens or >= kHeavyMinRows
// rows, items of kHeavyTile tokens), else the light list (items of light_tokens tokens,
// written out as {first sorted position, tokens, first row, d_t (-1: ID out of range)});
// with light_long non-null (n entries), light items of blocks with >= kLightLongRows rows
// go to light_long from the front (count in HDR_NLIGHT_LONG) and those with >=
// kLightMidRows from its back, entry n - 1 first (count in HDR_NLIGHT_MID).
hipError_t launch_worklist(const RouteBufs &b, int64_t n, const int64_t *off, int64_t vocab,
                           int heavy_min_tokens, int dense_min_tokens, int light_tokens,
                           int4 *light, int2 *heavy, int2 *dense, hipStream_t s,
                           int4 *light_long = nullptr);
// The header zeroing, the route and the work lists of a batch of 1 .. kRouteSmallMax
// tokens in one single-workgroup launch (same outputs; sorted keys and permutation
// in keys_a / vals_a).
hipError_t launch_route_small(const int32_t *ids, int64_t n, int64_t vocab, const int64_t *off,
                              int heavy_min_tokens, int dense_min_tokens, int light_tokens, RouteBufs &b,
                              int4 *light, int2 *heavy, int2 *dense, hipStream_t s);

// Split-row gather-attention for small bf16 batches: each block's rows are cut into
// chunks of split_rows(d_in) rows and its tokens into groups of split_tokens(d_in);
// one wavefront per (chunk, group) item forms the chunk's softmax partials, and one
// wavefront per token merges its block's chunks.  Used when n <= kSplitMaxN and the
// partial slots (<= n * ceil(max_d / split_rows)) stay within kSplitMaxSlots.
constexpr int kSplitMaxN = 512;
constexpr int64_t kSplitMaxSlots = 32768;
int split_rows(int64_t d_in);
int split_tokens(int64_t d_in);
int64_t split_slots(const Dims &d, int64_t n, int32_t max_d);  // 0: path off
struct SplitLists {
    int4 *items, *blkinfo;
    int32_t *blk_of;
};
// The single-workgroup route that also writes the split-row items (instead of the
// light / heavy / dense lists).
hipError_t launch_route_small_split(const int32_t *ids, int64_t n, int64_t vocab, const int64_t *off,
                                    int rows, int tokens, RouteBufs &b, const SplitLists &sl,
                                    hipStream_t s);
struct SplitArgs {
    const void *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *perm, *hdr, *blk_of;
    const int4 *items, *blkinfo;
    int64_t n, d_in, d_emb;
    float2 *pml;
    float *po;
    void *o;
};
hipError_t launch_attn_split(const SplitArgs &a, hipStream_t s);

struct AttnArgs {
    const void *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    int32_t *queue;  // per-XCD work counters of the MFMA path (in the header)
    const int4 *light, *light_long;  // light items (short blocks), then those of long blocks
    const int2 *heavy, *dense;
    int64_t n, d_in, d_emb, vocab;
    void *o;
    float *scores;  // fp32 path scratch
    int32_t max_d;
};
int attn_light_tokens(int64_t d_in, int64_t d_emb, int dtype);   // tokens per light work item
int attn_heavy_min_tokens(int64_t d_in, int64_t d_emb, int dtype, int32_t max_d);  // INT32_MAX = none
int attn_dense_min_tokens(int64_t d_in, int64_t d_emb, int dtype);                  // INT32_MAX = none
// the MFMA kernel over the heavy work list (bf16, when attn_heavy_min_tokens allows it),
// and the wavefront-per-item kernel over the light list (any dtype)
hipError_t launch_attn_heavy(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_light(const AttnArgs &a, int dtype, hipStream_t s);

// out[M x N] = A[M x K] B[N x K]^T, bf16 in / bf16 out, fp32 accumulate.
// Optional LayerNorm partial statistics of the stored (bf16-rounded) rows of C
// (ln_out [M x ceil(N/128) x 2] = per 128-column chunk (mean, M2)).
hipError_t launch_gemm_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M, int64_t N,
                            int64_t K, float *ln_out, hipStream_t s);
// stats [M x 2] = (mean, 1/sqrt(var + eps)) per row from the W_up partials.
hipError_t launch_ln_finalize(const float *lnp, int64_t M, int64_t d_up, float eps, float *stats,
                              hipStream_t s);
// out = W_mix [LN(h) ; x] with LayerNorm folded into the h columns of W_mix;
// fold_ws holds the folded weights and terms (mix_fold_bytes).
hipError_t launch_gemm_mix_bf16(const uint16_t *h, const uint16_t *x, const float *stats,
                                const uint16_t *W_mix, uint16_t *out, const void *fold_ws, int64_t M,
                                int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s);
// the fold terms of W_mix (W1' = W1 diag(gamma), c1, c2) into fold_ws
hipError_t launch_mix_fold(const uint16_t *W_mix, const float *gamma, const float *beta,
                           void *fold_ws, int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s);
size_t mix_fold_bytes(int64_t d_up, int64_t d_out);
// Factored W_mix (batches of more than kSkinnyMaxM tokens): F = W1 diag(gamma) W_c and
// G = W_c^T W_c of the centred W_up into factor_ws (mix_factor_bytes; the fold terms
// into fold_ws),
// the per-row shares of o^T G o (qp: [M x ln_quad_parts(d_emb)] fp32), and out = rstd *
// (F o) + c2 + W2 x, the W_mix GEMM forming each row's rstd = 1 / sqrt(o^T G o / d_up +
// eps) from the shares.
size_t mix_factor_bytes(int64_t d_emb, int64_t d_up, int64_t d_out);
int ln_quad_parts(int64_t d_emb);
hipError_t launch_mix_factor(const uint16_t *W_up, const uint16_t *W_mix, const float *gamma,
                             const float *beta, void *fold_ws, void *factor_ws, int64_t d_emb,
                             int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s);
hipError_t launch_ln_quad_stats_bf16(const uint16_t *o, const void *factor_ws, int64_t M, int64_t d_emb,
                                     int64_t d_up, int64_t d_out, float *qp, hipStream_t s);
hipError_t launch_gemm_mix_factored_bf16(const uint16_t *o, const uint16_t *x, const float *qp, float eps,
                                         const uint16_t *W_mix, uint16_t *out, const void *fold_ws,
                                         const void *factor_ws, int64_t M, int64_t d_emb, int64_t d_up,
                                         int64_t d_in, int64_t d_out, hipStream_t s);
// Decode staging: destination row r of the compact tables belongs to compact ID i
// with coff[i] <= r < coff[i+1] and comes from table row src[i] + (r - coff[i]) of
// the pinned host tables (device mappings WK_dev / WV_dev), or, for src[i] < 0, from
// row -1 - src[i] + (r - coff[i]) of the device cache cK / cV.
hipError_t launch_stage_rows(const int64_t *coff, const int64_t *src, int64_t m, int64_t rows,
                             const void *WK_dev, const void *WV_dev, const void *cK, const void *cV,
                             void *dK, void *dV, int64_t row_k_bytes, int64_t row_v_bytes,
                             hipStream_t s);
// Small-M path (split K, fp32 partial slabs in `part`, skinny_part_bytes of them):
// the plain GEMM (with the same optional LayerNorm partials as launch_gemm_bf16),
// and out = W_mix [LN(h) ; x] with LayerNorm applied to h while it is staged,
// its row statistics merged from the W_up partials `lnp` (no fold terms needed).
constexpr int64_t kSkinnyMaxM = 512;  // batches up to this many tokens take the small-M path
size_t skinny_part_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_skinny_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C, int64_t M,
                                   int64_t N, int64_t K, float *ln_out, float *part, hipStream_t s);
hipError_t launch_gemm_mix_skinny_bf16(const uint16_t *h, const uint16_t *x, const float *lnp,
                                       const float *gamma, const float *beta, float eps,
                                       const uint16_t *W_mix, uint16_t *out, int64_t M, int64_t d_up,
                                       int64_t d_in, int64_t d_out, float *part, hipStream_t s);
// fp32 variants (any dims): plain GEMM, and the mix GEMM with LayerNorm computed in a
// separate per-row statistics pass.
hipError_t launch_gemm_f32(const float *A, const float *B, float *C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s);
hipError_t launch_gemm_mix_f32(const float *h, const float *x, float *stats, const float *gamma,
                               const float *beta, float eps, const float *W_mix, float *out,
                               int64_t M, int64_t d_up, int64_t d_in, int64_t d_out, hipStream_t s);

// ---- backward pass
// fp32 GEMMs with fp32 output, written or added to C (C = A B^T as above)
// C[M x N] (fp32) += A B^T with K cut into gemm_f32_splits(M, N, K) ranges when the
// output has too few tiles to fill the chip: one launch writes a slab per range into
// `part` (gemm_f32_split_bytes), a second adds the slabs to C in range order.
int gemm_f32_splits(int64_t M, int64_t N, int64_t K);
size_t gemm_f32_split_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_bf16_f32acc_split(const uint16_t *A, const uint16_t *B, float *C, int64_t M,
                                         int64_t N, int64_t K, float *part, hipStream_t s);
hipError_t launch_gemm_bf16_f32out(const uint16_t *A, const uint16_t *B, float *C, int64_t M,
                                   int64_t N, int64_t K, bool accumulate, hipStream_t s);
hipError_t launch_gemm_f32_acc(const float *A, const float *B, float *C, int64_t M, int64_t N,
                               int64_t K, bool accumulate, hipStream_t s);
// stats [M x 2] = (mean, 1/sqrt(var + eps)) per row of an fp32 h
hipError_t launch_ln_stats_f32(const float *h, int64_t M, int64_t d_up, float eps, float *stats,
                               hipStream_t s);
// dst [cols x ld_dst] = src^T (rows >= `rows` up to rows_pad zero-filled), element
// type by dtype
hipError_t launch_transpose(const void *src, int64_t ld_src, int64_t rows, int64_t cols, void *dst,
                            int64_t ld_dst, int64_t rows_pad, int dtype, hipStream_t s);
// LayerNorm backward: dh and y = LN(h) per row, and dgamma += sum dy*yhat, dbeta +=
// sum dy (column partials of ln_param_chunks(n) row chunks, reduced in order)
int ln_param_chunks(int64_t n);
hipError_t launch_ln_bwd(const void *h, const float *stats, const float *gamma, const float *beta,
                         const float *dy, int64_t n, int64_t d_up, void *dh, void *y, float2 *part,
                         float *dgamma, float *dbeta, int dtype, hipStream_t s);
struct BwdArgs {
    const void *x, *WK, *WV;
    const int64_t *off;
    const int32_t *uniq, *seg_start, *perm, *hdr;
    const int4 *items;   // attn_bwd_tokens tokens per item (first sorted position, count, first row, d_t)
    const float *dov;    // dL/do [n x d_emb]
    const void *o;       // the forward's o [n x d_emb] (recomputed), for <dO, o>
    int64_t d_in, d_emb, vocab;
    int max_d;
    float *dx;           // [n x d_in], holds W2^T dout; the attention term is added
    float *P, *dS;       // [n x max_d] per sorted position
    float *dWK, *dWV;    // accumulated
    int2 *kv_items;      // items of the key / value gradients
    int kv_cap;          // their capacity (kv_item_capacity)
    int64_t n;           // tokens
    uint16_t *dob;       // [n x d_emb] dO rounded to bf16 (matrix-core key / value gradients)
    float4 *tstat;       // [n] per sorted position: (lse, <dO, o>, d_t as int bits, 0) (matrix cores)
};
// items of the key / value gradients: at most one per block plus one per 16 rows, or
// for the matrix-core kernel (one per block plus one per 64 rows) per column slice
int kv_item_capacity(int64_t n, int64_t rows, int64_t d_in, int64_t d_emb, int dtype);
// tokens per attention-backward work item (all of one block) for these dims
int attn_bwd_tokens(int64_t d_in, int64_t d_emb, int dtype);
// part 0: attention backward per work item; part 1: the key / value gradients per
// ID block (after part 0)
hipError_t launch_attn_bwd(const BwdArgs &a, int dtype, int part, hipStream_t s);

}  // namespace l3
