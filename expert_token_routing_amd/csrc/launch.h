// Host-side launchers of the library's kernels (internal; the C ABI is in
// include/occ.h).  Each queues its kernels on `stream` and returns the launch
// status.  Shapes have been validated by the caller.
#pragma once

#include "common.h"

namespace occ {

// Compute units of the current device (read once per device; 256 on MI355X).
int compute_units();

// --- routing (route.hip) ---
// prune_rule 0 none, 1 TRAVERSE, 2 GROUPSUM, 3 similarity (sim_rank: Ne x Ne
// ranked table, used only by rule 3).
hipError_t launch_route(const float *logits, int T, int Ne, int k, int prune_rule, int G,
                        const PlaceTab &tab, const int32_t *sim_rank, int32_t *ids, float *w,
                        hipStream_t s);
// Copies caller routing into ids/w, replacing out-of-range or repeated ids of
// a token by the lowest unused experts with weight 0.
hipError_t launch_sanitize_ids(const int32_t *ids_in, const float *w_in, int T, int k, int Ne,
                               int32_t *ids, float *w, hipStream_t s);

// --- gate projection (gate.hip) ---
// logits (T x Ne fp32) = x (T x d) . w_router (Ne x d)^T, bf16 or fp32 inputs.
hipError_t launch_gate(const void *x, const void *w_router, int T, int d, int Ne, int bf16,
                       float *logits, hipStream_t s);

// --- expert similarity table (similarity.hip) ---
// gram += H^T H (fp64, tokens ascending); H is T x Ne fp32.
hipError_t launch_sim_gram(const float *H, int T, int Ne, double *gram, hipStream_t s);
// Squared cosine similarities (t2 may be NULL) and each row's ranking.
hipError_t launch_sim_rank(const double *gram, int Ne, double *t2, int32_t *rank, hipStream_t s);

// --- BRIM (brim.hip) ---
constexpr int kBrimChunk = 128;  // tokens per BRIM workgroup
// Batches of at most kBrimSmallT tokens and kBrimSmallEntries routing
// entries build the BRIM in one workgroup (more entries are faster over
// the three kernels' several workgroups).
constexpr int kBrimSmallT = 512, kBrimSmallEntries = 1024;
struct BrimBufs {
    int32_t *brim0, *sfd_off, *epd_off, *tile_off, *epd_src, *tok_epd, *brim1;
    float *epd_w;
    int32_t *down_rows, *first_cnt, *tile_off_first, *tile_off_rest;
    int32_t *chunk_cnt, *chunk_base;
};
// tile_rows: the grouped GEMMs' row-tile capacity.  fill_cols > 0: the
// up-projection's column tiles; the experts then take extra row tiles (at
// most kBrimMaxFill) until the up-projection's tiles fill their last round
// of the CUs.
constexpr int kBrimMaxFill = 64;
hipError_t launch_brim(const int32_t *ids, const float *w, int T, int k, const PlaceTab &tab,
                       int tile_rows, int fill_cols, int dense_brim1, const BrimBufs &b,
                       hipStream_t s);

// --- row movers (rows.hip) ---
// x_sfd[brim0[g, t]] = x[t] for every group the token uses; with zero_out,
// also zero_out[brim0[g, t]][0 .. zero_cols) = 0 (fp32, zero_cols % 4 == 0).
hipError_t launch_dispatch(const void *x, int T, int Nd, size_t row_bytes, const int32_t *brim0,
                           void *x_sfd, hipStream_t s, float *zero_out = nullptr,
                           int zero_cols = 0);
// Deterministic stage one: each SFD row holds its first contributor's result
// (the token's lowest-position expert in the group) and y_epd[tok_epd[t, j]]
// holds the others'; sfd_out[brim0[g, t]] becomes the sum over the token's
// experts in group g in ascending placement position (fp32), written back
// only for groups with several experts.  With y, also stage two, as
// launch_combine would compute it (same order).
hipError_t launch_merge_slots(const float *y_epd, const int32_t *ids, const int32_t *tok_epd,
                              const int32_t *brim0, const PlaceTab &tab, int T, int k, int d,
                              float *sfd_out, const float *y_sh, void *y, int y_bf16,
                              hipStream_t s);
// y[t] = dtype( sum over g of sfd_out[brim0[g, t]] (+ y_sh[t]) ), fp32 sums in
// ascending group order.
hipError_t launch_combine(const float *sfd_out, const int32_t *brim0, const float *y_sh, int T,
                          int Nd, int d, int out_bf16, void *y, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, size_t n, int32_t v, hipStream_t s);

// --- grouped GEMMs, bf16 MFMA (gemm_bf16.hip) ---
// Up-projection with SwiGLU and routing-weight modulation:
//   out[r, f] = bf16( row_w[r] * silu(a_r . Wg[e][f]) * (a_r . Wu[e][f]) )
// a_r = A[a_rows[r]] (or A[r] when a_rows is NULL).  Routed mode walks the
// segments [seg_off[p], seg_off[p+1]) of each placement position p with the
// tile schedule tile_off; shared mode (seg_off NULL) is one segment of M rows.
// gu_out (optional, training): the pre-activations are also stored, row r
// holding bf16 g = a_r . Wg[e] in columns [0, N) and u in [N, 2N).
struct UpArgs {
    const void *A;
    const int32_t *a_rows;
    const void *Wg, *Wu;
    const int32_t *seg_off, *tile_off;
    const float *row_w;
    void *out;
    void *gu_out;
    int M, K, N, Ne;
    PlaceTab tab;
    int m_tiles;  // dense mode: row tiles (set by the bf16 launchers)
};
hipError_t launch_gemm_up_bf16(const UpArgs &a, size_t max_m_tiles, hipStream_t s);

// Down-projection.  Routed: the EPD rows of expert position p are
// rows[seg_off[p] ..  seg_off[p+1]), first_cnt[p] of them first contributors
// to their SFD row; phase 1 multiplies those and stores
// out[dst_rows[r], :] = A[r] . W[e]^T, which writes every SFD row once;
// phase 2 multiplies the others and adds with fp32 atomics (several experts
// of one group share an SFD row).  tile_off is the phase's row-tile schedule.
// Phase 3 (the deterministic merge's first half) multiplies every row, with
// the all-rows schedule: first contributors store into their SFD rows, the
// others into epd_out at their own EPD rows.
// Shared (seg_off NULL): out[r, :] = A[r] . W^T with W = n_sh blocks of
// (N x k_split) laid end to end along K.
struct DownArgs {
    const void *A;
    const void *W;
    const int32_t *seg_off, *tile_off;
    const int32_t *rows, *first_cnt;
    const int32_t *dst_rows;
    float *out;
    float *epd_out;  // phase 3
    int M, K, N, Ne, k_split, phase;
    PlaceTab tab;
    int m_tiles;  // dense mode: row tiles (set by the bf16 launchers)
};
hipError_t launch_gemm_down_bf16(const DownArgs &a, size_t max_m_tiles, hipStream_t s);
// The same with 128-row tiles (gemm_bf16_m128.hip), taken by bf16 batches
// whose experts average fewer than kSmallTileRows rows.
constexpr int kGemmBmBf16Small = 128;
constexpr int kSmallTileRows = 96;
hipError_t launch_gemm_up_bf16_m128(const UpArgs &a, size_t max_m_tiles, hipStream_t s);
hipError_t launch_gemm_down_bf16_m128(const DownArgs &a, size_t max_m_tiles, hipStream_t s);
// The same, four-wave and software-pipelined with 256 x 256 tiles
// (gemm_bf16_dense.hip), for dense products only (seg_off NULL; a routed
// launch returns hipErrorInvalidValue).  Taken by dense products of at least
// kDensePipeRounds rounds of tiles on the CUs.
constexpr int kDensePipeRounds = 4;
hipError_t launch_gemm_up_bf16_dense(const UpArgs &a, size_t max_m_tiles, hipStream_t s);
hipError_t launch_gemm_down_bf16_dense(const DownArgs &a, size_t max_m_tiles, hipStream_t s);

// --- the same two GEMMs in fp32 on the vector ALUs (gemm_f32.hip) ---
hipError_t launch_gemm_up_f32(const UpArgs &a, size_t max_m_tiles, hipStream_t s);
hipError_t launch_gemm_down_f32(const DownArgs &a, size_t max_m_tiles, hipStream_t s);

// --- backward grouped GEMMs, bf16 MFMA (gemm_bwd.hip) ---
// Input-gradient GEMM over row tiles of up to kBwdRowTile rows (tile_off over the segments
// seg_off of placement positions; first_cnt and phase select rows as in
// DownArgs):  C[pos, :] = A_row . B_e, K contracted, with A_row the K values
// at column a_col of row a_rows[pos] (or pos) of A (rows lda apart), and row
// k of B_e = B1[e] row k for k < ksplit, else B2[e] row k - ksplit (both N
// wide, so B is read K-major; e = tab.expert[p]).  N >= 256.  With b_kcontig
// (SWIGLU only, no B2, ksplit = K) B1 holds the weights transposed instead:
// expert e's block of N rows of K contiguous values, B_e[k][n] = B1[(e N + n) K + k].
// Epilogue SWIGLU: C is dh; with g = gu[pos*gu_ld + gu_col + f], u at
// + gu_uoff, and w = row_w[pos] (1 if NULL), writes bf16 dg, du to
// out[pos*out_ld + out_col + f] and + out_uoff, and (dw_part non-NULL)
// dw_part[pos * dw_stride + q] = this tile half's sum of dh * silu(g) u.
// Epilogue MERGE: C goes to merge_out[dst_rows[a_rows[pos]]] (identity
// without dst_rows / a_rows), N wide fp32: stored (merge_store) or added;
// with split (phase 0), the rows of a segment after its first_cnt first
// contributors are stored to epd_out[a_rows[pos]] instead.
enum { BWD_EPI_SWIGLU = 0, BWD_EPI_MERGE = 1 };
// Row capacity of the input-gradient tiles: the row schedules tile_off are
// built with it (ceil(rows / kBwdRowTile) tiles per segment, the all-rows
// schedule filled to whole rounds of the CUs; rows shared out evenly in
// 16-row blocks).
constexpr int kBwdRowTile = 320;
struct BwdDgradArgs {
    const void *A;
    const int32_t *a_rows;
    const void *B1, *B2;
    const int32_t *seg_off, *tile_off, *first_cnt, *dst_rows;
    const void *gu;
    const float *row_w;
    void *out;
    float *dw_part;
    float *merge_out;
    float *epd_out;
    int N, K, ksplit, Ne, phase, epilogue, dw_stride, merge_store, split, b_kcontig;
    int lda, a_col, gu_ld, gu_col, gu_uoff, out_ld, out_col, out_uoff;
    PlaceTab tab;
};
hipError_t launch_bwd_dgrad(const BwdDgradArgs &a, size_t max_m_tiles, hipStream_t s);

// Weight-gradient GEMM, one group of K rows per expert (routed: the expert
// segments seg_off, placement position order, e = tab.expert[p]; dense:
// seg_off NULL, n_groups blocks of `rows` rows, e = block):
//   C_e[m, n] = sum over the group's rows pos of A[a_rows[pos]][a_col + m] *
//               B[b_rows[pos]][b_col + n],   a_col = a_col0 + group * a_col_grp
// both operands K-major (rows lda / ldb elements apart); at most one of
// a_rows, b_rows is given (hipErrorInvalidValue otherwise).  Rows m < msplit go
// to C1[e] (msplit x N), the rest to C2[e].  M, N >= 256; tail rows of a
// group read zero_row (at least 256 zero elements).
// Dense launches (seg_off NULL) may split K (the rows) into k_parts chunks
// of k_chunk rows: each chunk's fp32 tiles go to `part` (k_parts x n_groups
// x M x N) and a second kernel adds them in chunk order into C1 / C2, so
// the result stays deterministic.
struct BwdWgradArgs {
    const void *A, *B;
    const int32_t *a_rows, *b_rows, *seg_off;
    const void *zero_row;
    float *C1, *C2;
    int M, N, msplit, lda, ldb, a_col0, a_col_grp, b_col0, b_col_grp, n_groups, rows;
    PlaceTab tab;
    int k_parts, k_chunk;
    float *part;
};
hipError_t launch_bwd_wgrad(const BwdWgradArgs &a, hipStream_t s);
// K chunks for a dense weight-gradient product of n_groups x M x N outputs
// over `rows` rows (1: no split), chosen from the shape alone; rows per
// chunk for that count.
int wgrad_k_parts(int n_groups, int M, int N, int rows);
int wgrad_k_chunk(int rows, int parts);

// Row-tile schedules for `tile_rows`-row tiles from the expert segments
// epd_off and first-contributor counts first_cnt (all rows, first, rest).
hipError_t launch_tile_sched(const int32_t *epd_off, const int32_t *first_cnt, int Ne,
                             int tile_rows, int fill_cols, int32_t *tile_off,
                             int32_t *tile_off_first, int32_t *tile_off_rest, hipStream_t s);
// A one-segment schedule for a dense GEMM over T rows: seg_off = {0, T},
// tile_off = {0, m_tiles} (the rows shared out evenly over m_tiles tiles).
hipError_t launch_dense_sched(int T, int m_tiles, int32_t *seg_off, int32_t *tile_off,
                              hipStream_t s);
// nz bf16 matrices of R x C, the z-th at src + z * src_z (elements), each
// written transposed: dst[z * dst_z + c * ldd + r] = src[z * src_z + r * C + c].
// R and C multiples of 64, ldd >= R, 16-byte aligned rows.
hipError_t launch_transpose_bf16(const void *src, int R, int C, size_t src_z, void *dst, int ldd,
                                 size_t dst_z, int nz, hipStream_t s);
// Routing-weight and logit gradients: dw[t, j] = sum of dw_part over the
// EPD row tok_epd[t*k + j]'s nparts partials (in order); dlogits through the
// full softmax of the logits (logits may be NULL: dw only).
hipError_t launch_route_backward(const float *logits, const int32_t *ids, const int32_t *tok_epd,
                                 const float *dw_part, int nparts, int dw_stride, int T, int Ne,
                                 int k, float *dw, float *dlogits, hipStream_t s);

// --- co-activation statistics (coact.hip) ---
hipError_t launch_coact(const int32_t *ids, int T, int k, const PlaceTab &tab, int32_t *C,
                        float *P, int64_t *n_sfd, double *ct, double *intra, hipStream_t s);

}  // namespace occ
