// BRIM_0 and BRIM_1 (Occult paper, appendix A.2, Algorithms 3 and 5) as a
// parallel counting sort.
//
// Both algorithms run a counter over a 2-D grid in row-major order, so every
// entry is (start of its row) + (rank of the token inside the row).  Rows are
// "bins": Nd group bins for BRIM_0 (a token enters bin g once if any of its
// experts lives on group g) and Ne expert bins, in placement order, for
// BRIM_1 (the group-local counter of Algorithm 5 is the global EPD row minus
// the group's first EPD row, because groups' EPD blocks are laid end to end).
// A third family of Ne bins counts, per expert, the EPD rows that are the
// first contributor to their SFD row (the token's lowest-slot expert in that
// group); it orders each expert's rows for the down-projection merge: first
// contributors, then the rest, each in token order.
//
//   k_brim_count  per chunk of kBrimChunk tokens, the token count of every bin
//                 (stored bin-major: a bin's counts are contiguous);
//   k_brim_scan   one workgroup: exclusive scans over chunks and over bins,
//                 giving each (bin, chunk) its first row, plus sfd_off,
//                 epd_off, first-contributor counts and GEMM tile schedules;
//   k_brim_fill   per chunk: a token's rank inside a bin is the popcount of
//                 the lower tokens' bits in its 64-token block's mask for
//                 that bin (built with LDS atomic OR, so the result does not
//                 depend on timing) plus the counts of the earlier blocks.
// Count and fill give each routing entry (token, j) its own thread, so a
// thread's work is one entry, not a token's k of them.
// The result is identical, entry by entry, to the serial counters.
#include "launch.h"

namespace occ {
namespace {

constexpr int kBlocksPerChunk = kBrimChunk / kWave;  // 64-token blocks of a chunk
constexpr int kBrimThreads = 1024;  // count and fill: one thread per routing entry
constexpr int kScanLds = 14336;     // (bin, chunk) counts the scan keeps in LDS
constexpr int kScanBatch = 8;       // 64-chunk scan steps whose counts are loaded together
constexpr int kRegBins = 8;        // bins per wave whose scans the scan can keep in registers
constexpr int kLoadBatch = 8;      // loads a thread keeps in flight in the scan's copy loops

// Is any position in [lo, hi) set in the 256-bit position mask em?
__device__ __forceinline__ bool any_in(const uint64_t *em, int lo, int hi) {
    bool any = false;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const int a = max(lo - 64 * w, 0), b = min(hi - 64 * w, 64);
        if (a < b) {
            const uint64_t hi_mask = b == 64 ? ~0ull : (1ull << b) - 1ull;
            any |= (em[w] & hi_mask & ~((1ull << a) - 1ull)) != 0ull;
        }
    }
    return any;
}

__device__ __forceinline__ bool has_pos(const uint64_t *em, int p) {
    return (em[p >> 6] >> (p & 63)) & 1ull;
}

// Shared state of a chunk of at most NTOK tokens: its ids (id[token * k +
// j]), placement tables, and per token the 256-bit mask of its placement
// positions and the mask of its groups.
template <int NTOK>
struct ChunkIds {
    uint8_t id[NTOK * kMaxK];
    uint64_t em[NTOK][4];
    uint64_t gm[NTOK];
    uint8_t grp[kMaxNe];
    int16_t pos[kMaxNe];
};

// Coalesced load of the chunk's ids and the placement tables; then, one
// thread per token, the position and group masks.  Ends with a barrier.
template <int NTOK>
__device__ __forceinline__ void load_chunk(const int32_t *__restrict__ ids, int t0, int nt, int k,
                                           const PlaceTab &tab, ChunkIds<NTOK> &c) {
    const int n = tab.n;
    const size_t base = static_cast<size_t>(t0) * k;
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x)
        c.id[i] = static_cast<uint8_t>(ids[base + i]);
    for (int e = threadIdx.x; e < tab.Ne; e += blockDim.x) {
        c.grp[e] = tab.grp[e];
        c.pos[e] = static_cast<int16_t>(tab.grp[e] * n + tab.slot[e]);
    }
    __syncthreads();
    for (int tok = threadIdx.x; tok < nt; tok += blockDim.x) {
        uint64_t em[4] = {0, 0, 0, 0}, gm = 0;
        for (int j = 0; j < k; j++) {
            const int e = c.id[tok * k + j];
            const int q = c.pos[e];
            em[q >> 6] |= 1ull << (q & 63);
            gm |= 1ull << c.grp[e];
        }
#pragma unroll
        for (int w = 0; w < 4; w++) c.em[tok][w] = em[w];
        c.gm[tok] = gm;
    }
    __syncthreads();
}

// Entry (tok, j) with placement position q is its token's first contributor
// to its group's SFD row when no lower position of that group is set.
template <int NTOK>
__device__ __forceinline__ bool first_contrib(const ChunkIds<NTOK> &c, int tok, int q, int n) {
    return !any_in(c.em[tok], (q / n) * n, q);
}

// Adds the chunk's tokens to the bin counts cnt (LDS, zeroed; no barrier).
template <int NTOK>
__device__ __forceinline__ void count_bins(const ChunkIds<NTOK> &c, int nt, int k,
                                           const PlaceTab &tab, int *cnt) {
    const int Nd = tab.Nd, Ne = tab.Ne, n = tab.n;
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int tok = i / k, q = c.pos[c.id[i]];
        atomicAdd(&cnt[Nd + q], 1);
        if (first_contrib(c, tok, q, n)) atomicAdd(&cnt[Nd + Ne + q], 1);
    }
    for (int i = threadIdx.x; i < nt * Nd; i += blockDim.x) {
        const int g = i / nt, tok = i - g * nt;
        if ((c.gm[tok] >> g) & 1ull) atomicAdd(&cnt[g], 1);
    }
}

__global__ __launch_bounds__(kBrimThreads) void k_brim_count(const int32_t *__restrict__ ids,
                                                             int T, int k, PlaceTab tab,
                                                             int32_t *__restrict__ chunk_cnt) {
    __shared__ int cnt[kMaxBins];
    __shared__ ChunkIds<kBrimChunk> c;
    const int NB = tab.Nd + 2 * tab.Ne;
    const int t0 = blockIdx.x * kBrimChunk, nt = min(kBrimChunk, T - t0);
    for (int b = threadIdx.x; b < NB; b += blockDim.x) cnt[b] = 0;
    load_chunk(ids, t0, nt, k, tab, c);
    count_bins(c, nt, k, tab, cnt);
    __syncthreads();
    for (int b = threadIdx.x; b < NB; b += blockDim.x)
        chunk_cnt[static_cast<size_t>(b) * gridDim.x + blockIdx.x] = cnt[b];
}

// Across bins, from the bins' totals (run by one wave): groups give
// sfd_off; experts (placement order) give epd_off; first-contributor bins
// start at their expert's first EPD row (binoff: each bin's first row).
// ceil(rows / tile_rows) gives the GEMM row-tile schedules: all rows
// (up-projection, raised by fill_rounds when fill_cols > 0), first
// contributors and the rest (merge).  s_vt: LDS scratch of Ne entries.
__device__ void bin_offsets(const int *total, int Nd, int Ne, int tile_rows, int fill_cols,
                            int slots, int *s_vt, int *binoff, int32_t *__restrict__ sfd_off,
                            int32_t *__restrict__ epd_off, int32_t *__restrict__ tile_off,
                            int32_t *__restrict__ first_cnt, int32_t *__restrict__ tile_off_first,
                            int32_t *__restrict__ tile_off_rest) {
    const int lane = lane_id();
    const int vg = lane < Nd ? total[lane] : 0;
    const int ig = wave_incl_scan(vg);
    if (lane < Nd) {
        binoff[lane] = ig - vg;
        sfd_off[lane] = ig - vg;
    }
    if (lane == kWave - 1) sfd_off[Nd] = ig;
    // row tiles per expert: ceil(rows / tile_rows), raised by fill_rounds
    for (int p = lane; p < Ne; p += kWave) s_vt[p] = (total[Nd + p] + tile_rows - 1) / tile_rows;
    if (fill_cols > 0) fill_rounds(total + Nd, s_vt, Ne, fill_cols, slots, kBrimMaxFill);
    int run = 0, run_t = 0, run_f = 0, run_r = 0;
    for (int p0 = 0; p0 < Ne; p0 += kWave) {
        const int p = p0 + lane;
        const int v = p < Ne ? total[Nd + p] : 0;
        const int f = p < Ne ? total[Nd + Ne + p] : 0;
        const int vt = p < Ne ? s_vt[p] : 0;
        const int vf = (f + tile_rows - 1) / tile_rows;
        const int vr = (v - f + tile_rows - 1) / tile_rows;
        const int inc = wave_incl_scan(v), inc_t = wave_incl_scan(vt);
        const int inc_f = wave_incl_scan(vf), inc_r = wave_incl_scan(vr);
        if (p < Ne) {
            binoff[Nd + p] = run + inc - v;
            binoff[Nd + Ne + p] = run + inc - v;
            epd_off[p] = run + inc - v;
            tile_off[p] = run_t + inc_t - vt;
            tile_off_first[p] = run_f + inc_f - vf;
            tile_off_rest[p] = run_r + inc_r - vr;
            first_cnt[p] = f;
        }
        run += __shfl(inc, kWave - 1);
        run_t += __shfl(inc_t, kWave - 1);
        run_f += __shfl(inc_f, kWave - 1);
        run_r += __shfl(inc_r, kWave - 1);
    }
    if (lane == 0) {
        epd_off[Ne] = run;
        tile_off[Ne] = run_t;
        tile_off_first[Ne] = run_f;
        tile_off_rest[Ne] = run_r;
    }
}

__global__ __launch_bounds__(1024) void k_brim_scan(const int32_t *__restrict__ chunk_cnt,
                                                    int nchunks, int Nd, int Ne, int tile_rows,
                                                    int fill_cols, int slots,
                                                    int32_t *__restrict__ chunk_base,
                                                    int32_t *__restrict__ sfd_off,
                                                    int32_t *__restrict__ epd_off,
                                                    int32_t *__restrict__ tile_off,
                                                    int32_t *__restrict__ first_cnt,
                                                    int32_t *__restrict__ tile_off_first,
                                                    int32_t *__restrict__ tile_off_rest) {
    __shared__ int total[kMaxBins];
    __shared__ int binoff[kMaxBins];
    __shared__ int s_vt[kMaxNe];
    __shared__ int s_cc[kScanLds];
    const int NB = Nd + 2 * Ne;
    const int lane = lane_id(), wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
    const size_t n = static_cast<size_t>(nchunks) * NB;
    // the (chunk, bin) counts come in with one coalesced pass when they fit
    const bool staged = n <= static_cast<size_t>(kScanLds);
    if (staged) {
        // kLoadBatch loads in flight per thread, not one round trip each
        for (size_t i0 = threadIdx.x; i0 < n; i0 += static_cast<size_t>(blockDim.x) * kLoadBatch) {
            int v[kLoadBatch];
#pragma unroll
            for (int j = 0; j < kLoadBatch; j++) {
                const size_t i = i0 + static_cast<size_t>(j) * blockDim.x;
                v[j] = i < n ? chunk_cnt[i] : 0;
            }
#pragma unroll
            for (int j = 0; j < kLoadBatch; j++) {
                const size_t i = i0 + static_cast<size_t>(j) * blockDim.x;
                if (i < n) s_cc[i] = v[j];
            }
        }
        __syncthreads();
    }
    // Not staged, but every bin within one batch of scan steps and few bins
    // per wave: the counts of all of a wave's bins are loaded at once and
    // their scans stay in registers until the bin offsets are known, so that
    // step 3 stores them without reading them back.
    const bool in_regs = !staged && nchunks <= kWave * kScanBatch && NB <= nw * kRegBins;
    int rv[kRegBins][kScanBatch];
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kRegBins; i++) {
            const int b = wv + i * nw;
#pragma unroll
            for (int j = 0; j < kScanBatch; j++) {
                const int c = j * kWave + lane;
                rv[i][j] = b < NB && c < nchunks ? chunk_cnt[static_cast<size_t>(b) * nchunks + c] : 0;
            }
        }
#pragma unroll
        for (int i = 0; i < kRegBins; i++) {
            const int b = wv + i * nw;
            if (b >= NB) break;  // wave-uniform
            int run = 0;
#pragma unroll
            for (int j = 0; j < kScanBatch; j++) {
                if (j * kWave >= nchunks) break;  // wave-uniform
                const int incl = wave_incl_scan(rv[i][j]);
                rv[i][j] = run + incl - rv[i][j];
                run += __shfl(incl, kWave - 1);
            }
            if (lane == 0) total[b] = run;
        }
    }

    // 1. per bin, exclusive scan over chunks (64 chunks per wave step).  The
    //    counts are bin-major, so a bin's are contiguous, and a batch of
    //    kScanBatch steps is loaded before it is scanned: one round trip per
    //    batch instead of one per step (at 512 chunks x 124 bins the serial
    //    loads took the scan to 118 us).  Staged scans stay in LDS until step 3.
    for (int b = in_regs ? NB : wv; b < NB; b += nw) {
        int run = 0;
        const size_t row = static_cast<size_t>(b) * nchunks;
        for (int c0 = 0; c0 < nchunks; c0 += kWave * kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; j++) {
                const int c = c0 + j * kWave + lane;
                v[j] = c < nchunks ? (staged ? s_cc[row + c] : chunk_cnt[row + c]) : 0;
            }
#pragma unroll
            for (int j = 0; j < kScanBatch; j++) {
                if (c0 + j * kWave >= nchunks) break;  // wave-uniform: no empty steps
                const int c = c0 + j * kWave + lane;
                const int incl = wave_incl_scan(v[j]);
                if (c < nchunks) {
                    if (staged) s_cc[row + c] = run + incl - v[j];
                    else chunk_base[row + c] = run + incl - v[j];
                }
                run += __shfl(incl, kWave - 1);
            }
        }
        if (lane == 0) total[b] = run;
    }
    __syncthreads();

    // 2. across bins (wave 0)
    if (wv == 0)
        bin_offsets(total, Nd, Ne, tile_rows, fill_cols, slots, s_vt, binoff, sfd_off, epd_off,
                    tile_off, first_cnt, tile_off_first, tile_off_rest);
    __syncthreads();

    // 3. each (bin, chunk) start = start of the bin + rows of earlier chunks
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kRegBins; i++) {
            const int b = wv + i * nw;
            if (b >= NB) break;
#pragma unroll
            for (int j = 0; j < kScanBatch; j++) {
                const int c = j * kWave + lane;
                if (c < nchunks) chunk_base[static_cast<size_t>(b) * nchunks + c] = rv[i][j] + binoff[b];
            }
        }
        return;
    }
    for (size_t i0 = threadIdx.x; i0 < n; i0 += static_cast<size_t>(blockDim.x) * kLoadBatch) {
        int v[kLoadBatch];
#pragma unroll
        for (int j = 0; j < kLoadBatch; j++) {
            const size_t i = i0 + static_cast<size_t>(j) * blockDim.x;
            v[j] = i < n ? (staged ? s_cc[i] : chunk_base[i]) : 0;
        }
#pragma unroll
        for (int j = 0; j < kLoadBatch; j++) {
            const size_t i = i0 + static_cast<size_t>(j) * blockDim.x;
            if (i < n) chunk_base[i] = v[j] + binoff[i / nchunks];
        }
    }
}

// Chunk [t0, t0 + nt) of the batch (NBLK 64-token blocks at most), ids and
// masks in c: its bin rows, s_base[b] being the first row of bin b that the
// chunk fills; s_epd / s_first / s_sfd: epd_off, first_cnt, sfd_off in LDS;
// bmask zeroed, everything visible to the workgroup.  Writes BRIM_0, the
// condensed BRIM_1 (epd_src, epd_w, tok_epd), the merge order and, when
// dense, BRIM_1 as matrices.
template <int NBLK, int NTOK>
__device__ __forceinline__ void fill_chunk(
    const float *__restrict__ w, int T, int k, const PlaceTab &tab, int t0, int nt,
    const ChunkIds<NTOK> &c, unsigned long long (*bmask)[kMaxBins], int (*bpre)[kMaxBins],
    const int *s_base, const int *s_epd, const int *s_first, const int *s_sfd, int dense,
    int32_t *__restrict__ brim0, int32_t *__restrict__ epd_src, float *__restrict__ epd_w,
    int32_t *__restrict__ tok_epd, int32_t *__restrict__ down_rows, int32_t *__restrict__ brim1) {
    const int Nd = tab.Nd, Ne = tab.Ne, n = tab.n, NB = Nd + 2 * Ne;
    const int nblk = (nt + kWave - 1) / kWave;
    // bin membership bits (LDS atomic OR, so the result does not depend on timing)
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int tok = i / k, q = c.pos[c.id[i]];
        const unsigned long long bit = 1ull << (tok & 63);
        atomicOr(&bmask[tok >> 6][Nd + q], bit);
        if (first_contrib(c, tok, q, n)) atomicOr(&bmask[tok >> 6][Nd + Ne + q], bit);
    }
    for (int i = threadIdx.x; i < nt * Nd; i += blockDim.x) {
        const int g = i / nt, tok = i - g * nt;
        if ((c.gm[tok] >> g) & 1ull) atomicOr(&bmask[tok >> 6][g], 1ull << (tok & 63));
    }
    __syncthreads();
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        int run = s_base[b];
        for (int q = 0; q < nblk; q++) {
            bpre[q][b] = run;
            run += __popcll(bmask[q][b]);
        }
    }
    __syncthreads();

    // row of token tok in bin b: tokens of the chunk before it in the bin
    auto slot_of = [&](int tok, int b) {
        const unsigned long long below = (1ull << (tok & 63)) - 1ull;
        return bpre[tok >> 6][b] + __popcll(bmask[tok >> 6][b] & below);
    };

    // BRIM_0: coalesced along tokens
    for (int i = threadIdx.x; i < nt * Nd; i += blockDim.x) {
        const int g = i / nt, tok = i - g * nt;
        brim0[static_cast<size_t>(g) * T + t0 + tok] = ((c.gm[tok] >> g) & 1ull) ? slot_of(tok, g) : -1;
    }
    // one thread per routing entry: its EPD row, SFD row and merge order
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
        const int tok = i / k;
        const size_t o = static_cast<size_t>(t0) * k + i;
        const int q = c.pos[c.id[i]], g = q / n;
        const int srow = slot_of(tok, g);
        const int erow = slot_of(tok, Nd + q);
        epd_src[erow] = srow;
        epd_w[erow] = w[o];
        tok_epd[o] = erow;
        // merge order: first contributors of expert q, then its other rows
        const int e0 = s_epd[q];
        const int f_before = slot_of(tok, Nd + Ne + q);  // e0 + first rows of q before tok
        if (first_contrib(c, tok, q, n)) down_rows[f_before] = erow;
        else down_rows[e0 + s_first[q] + (erow - e0) - (f_before - e0)] = erow;
        if (dense) {
            const int g0 = s_sfd[g], Ng = s_sfd[g + 1] - g0;
            brim1[static_cast<size_t>(n) * g0 + static_cast<size_t>(q - g * n) * Ng + (srow - g0)] =
                erow - s_epd[g * n];
        }
    }
    if (dense) {
        // the positions of a group that a token's SFD row does not use
        for (int i = threadIdx.x; i < nt * Nd; i += blockDim.x) {
            const int g = i / nt, tok = i - g * nt;
            if (!((c.gm[tok] >> g) & 1ull)) continue;
            const int g0 = s_sfd[g], Ng = s_sfd[g + 1] - g0;
            const int srow = slot_of(tok, g);
            for (int j = 0; j < n; j++)
                if (!has_pos(c.em[tok], g * n + j))
                    brim1[static_cast<size_t>(n) * g0 + static_cast<size_t>(j) * Ng + (srow - g0)] = -1;
        }
    }
}

__global__ __launch_bounds__(kBrimThreads) void k_brim_fill(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int T, int k, PlaceTab tab,
    const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ sfd_off,
    const int32_t *__restrict__ epd_off, const int32_t *__restrict__ first_cnt, int dense,
    int32_t *__restrict__ brim0, int32_t *__restrict__ epd_src, float *__restrict__ epd_w,
    int32_t *__restrict__ tok_epd, int32_t *__restrict__ down_rows,
    int32_t *__restrict__ brim1) {
    // bit (tok mod 64) of bmask[tok / 64][b]: token tok is in bin b
    __shared__ unsigned long long bmask[kBlocksPerChunk][kMaxBins];
    __shared__ int bpre[kBlocksPerChunk][kMaxBins];
    __shared__ int s_base[kMaxBins];
    __shared__ int s_epd[kMaxNe + 1], s_first[kMaxNe], s_sfd[kMaxNd + 1];
    __shared__ ChunkIds<kBrimChunk> c;
    const int Nd = tab.Nd, Ne = tab.Ne, NB = Nd + 2 * Ne;
    const int t0 = blockIdx.x * kBrimChunk, nt = min(kBrimChunk, T - t0);
    for (int i = threadIdx.x; i < kBlocksPerChunk * NB; i += blockDim.x)
        bmask[i / NB][i % NB] = 0ull;
    for (int b = threadIdx.x; b < NB; b += blockDim.x)
        s_base[b] = chunk_base[static_cast<size_t>(b) * gridDim.x + blockIdx.x];
    for (int e = threadIdx.x; e < Ne; e += blockDim.x) s_first[e] = first_cnt[e];
    for (int e = threadIdx.x; e <= Ne; e += blockDim.x) s_epd[e] = epd_off[e];
    for (int g = threadIdx.x; g <= Nd; g += blockDim.x) s_sfd[g] = sfd_off[g];
    load_chunk(ids, t0, nt, k, tab, c);
    fill_chunk<kBlocksPerChunk>(w, T, k, tab, t0, nt, c, bmask, bpre, s_base, s_epd, s_first, s_sfd,
                                dense, brim0, epd_src, epd_w, tok_epd, down_rows, brim1);
}

// A small batch (at most kBrimSmallT tokens and kBrimSmallEntries routing
// entries) in one workgroup: the counts, the offsets and schedules across
// bins and the fill of k_brim_count, k_brim_scan and k_brim_fill, with the
// whole batch as one chunk, in one launch (the three launches' fixed
// latencies dominate such batches: 15.5 -> 9.8 us at 256 tokens of top-2;
// at 512 tokens of top-8 one workgroup was 10% slower than the three
// kernels).  Same results, entry by entry.
constexpr int kSmallBlocks = kBrimSmallT / kWave;

__global__ __launch_bounds__(kBrimThreads) void k_brim_small(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int T, int k, PlaceTab tab,
    int tile_rows, int fill_cols, int slots, int dense, int32_t *__restrict__ sfd_off,
    int32_t *__restrict__ epd_off, int32_t *__restrict__ tile_off, int32_t *__restrict__ first_cnt,
    int32_t *__restrict__ tile_off_first, int32_t *__restrict__ tile_off_rest,
    int32_t *__restrict__ brim0, int32_t *__restrict__ epd_src, float *__restrict__ epd_w,
    int32_t *__restrict__ tok_epd, int32_t *__restrict__ down_rows,
    int32_t *__restrict__ brim1) {
    __shared__ unsigned long long bmask[kSmallBlocks][kMaxBins];
    __shared__ int bpre[kSmallBlocks][kMaxBins];
    __shared__ int cnt[kMaxBins], binoff[kMaxBins], s_vt[kMaxNe];
    __shared__ int s_epd[kMaxNe + 1], s_first[kMaxNe], s_sfd[kMaxNd + 1];
    __shared__ ChunkIds<kBrimSmallT> c;
    const int Nd = tab.Nd, Ne = tab.Ne, NB = Nd + 2 * Ne;
    for (int i = threadIdx.x; i < kSmallBlocks * NB; i += blockDim.x)
        bmask[i / NB][i % NB] = 0ull;
    for (int b = threadIdx.x; b < NB; b += blockDim.x) cnt[b] = 0;
    load_chunk(ids, 0, T, k, tab, c);
    count_bins(c, T, k, tab, cnt);
    __syncthreads();
    if (threadIdx.x < kWave)
        bin_offsets(cnt, Nd, Ne, tile_rows, fill_cols, slots, s_vt, binoff, sfd_off, epd_off,
                    tile_off, first_cnt, tile_off_first, tile_off_rest);
    __syncthreads();
    // the fill's LDS copies of the offsets, from the bins' totals and starts
    for (int e = threadIdx.x; e < Ne; e += blockDim.x) {
        s_first[e] = cnt[Nd + Ne + e];
        s_epd[e] = binoff[Nd + e];
    }
    if (threadIdx.x == 0) s_epd[Ne] = binoff[Nd + Ne - 1] + cnt[Nd + Ne - 1];
    for (int g = threadIdx.x; g < Nd; g += blockDim.x) s_sfd[g] = binoff[g];
    if (threadIdx.x == 0) s_sfd[Nd] = binoff[Nd - 1] + cnt[Nd - 1];
    __syncthreads();
    fill_chunk<kSmallBlocks>(w, T, k, tab, 0, T, c, bmask, bpre, binoff, s_epd, s_first, s_sfd,
                             dense, brim0, epd_src, epd_w, tok_epd, down_rows, brim1);
}

}  // namespace

hipError_t launch_brim(const int32_t *ids, const float *w, int T, int k, const PlaceTab &tab,
                       int tile_rows, int fill_cols, int dense_brim1, const BrimBufs &b,
                       hipStream_t s) {
    if (T <= kBrimSmallT && T * k <= kBrimSmallEntries) {
        k_brim_small<<<1, kBrimThreads, 0, s>>>(ids, w, T, k, tab, tile_rows, fill_cols,
                                                compute_units(), dense_brim1, b.sfd_off,
                                                b.epd_off, b.tile_off, b.first_cnt,
                                                b.tile_off_first, b.tile_off_rest, b.brim0,
                                                b.epd_src, b.epd_w, b.tok_epd, b.down_rows, b.brim1);
        return hipGetLastError();
    }
    const int nchunks = static_cast<int>(ceil_div(T, kBrimChunk));
    k_brim_count<<<nchunks, kBrimThreads, 0, s>>>(ids, T, k, tab, b.chunk_cnt);
    k_brim_scan<<<1, 1024, 0, s>>>(b.chunk_cnt, nchunks, tab.Nd, tab.Ne, tile_rows, fill_cols,
                                   compute_units(), b.chunk_base,
                                   b.sfd_off, b.epd_off, b.tile_off, b.first_cnt,
                                   b.tile_off_first, b.tile_off_rest);
    k_brim_fill<<<nchunks, kBrimThreads, 0, s>>>(ids, w, T, k, tab, b.chunk_base, b.sfd_off,
                                               b.epd_off, b.first_cnt, dense_brim1, b.brim0,
                                               b.epd_src, b.epd_w, b.tok_epd, b.down_rows,
                                               b.brim1);
    return hipGetLastError();
}

}  // namespace occ
