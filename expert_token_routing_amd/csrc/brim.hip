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
//   k_brim_count  per chunk of kBrimChunk tokens, the token count of every bin;
//   k_brim_scan   one workgroup: exclusive scans over chunks and over bins,
//                 giving each (chunk, bin) its first row, plus sfd_off,
//                 epd_off, first-contributor counts and GEMM tile schedules;
//   k_brim_fill   per chunk: a token's rank inside a bin is the popcount of
//                 the lower lanes' bits in a per-wave 64-bit mask (built with
//                 LDS atomic OR, so the result does not depend on timing)
//                 plus the counts of the earlier waves.
// The result is identical, entry by entry, to the serial counters.
#include "launch.h"

namespace occ {
namespace {

constexpr int kWavesPerChunk = kBrimChunk / kWave;

__device__ __forceinline__ bool has_pos(const uint64_t (&em)[4], int p) {
    return (em[p >> 6] >> (p & 63)) & 1ull;
}

// Is placement position p (one of the token's experts, mask em) the token's
// lowest position inside p's group?  Positions g*n .. g*n+n-1 form group g.
__device__ __forceinline__ bool first_in_group(const uint64_t (&em)[4], int p, int n) {
    for (int q = (p / n) * n; q < p; q++)
        if (has_pos(em, q)) return false;
    return true;
}

__global__ __launch_bounds__(kBrimChunk) void k_brim_count(const int32_t *__restrict__ ids, int T,
                                                           int k, PlaceTab tab,
                                                           int32_t *__restrict__ chunk_cnt) {
    __shared__ int cnt[kMaxBins];
    __shared__ uint8_t s_grp[kMaxNe];
    __shared__ int16_t s_pos[kMaxNe];
    const int Nd = tab.Nd, Ne = tab.Ne, n = tab.n, NB = Nd + 2 * Ne;
    for (int b = threadIdx.x; b < NB; b += blockDim.x) cnt[b] = 0;
    for (int e = threadIdx.x; e < Ne; e += blockDim.x) {
        s_grp[e] = tab.grp[e];
        s_pos[e] = static_cast<int16_t>(tab.grp[e] * n + tab.slot[e]);
    }
    __syncthreads();
    const int t = blockIdx.x * kBrimChunk + threadIdx.x;
    if (t < T) {
        uint64_t gmask = 0, em[4] = {0, 0, 0, 0};
        for (int j = 0; j < k; j++) {
            const int e = ids[static_cast<size_t>(t) * k + j];
            const int p = s_pos[e];
            em[p >> 6] |= 1ull << (p & 63);
            atomicAdd(&cnt[Nd + p], 1);
            gmask |= 1ull << s_grp[e];
        }
        for (int j = 0; j < k; j++) {
            const int p = s_pos[ids[static_cast<size_t>(t) * k + j]];
            if (first_in_group(em, p, n)) atomicAdd(&cnt[Nd + Ne + p], 1);
        }
        while (gmask) {
            const int g = __ffsll(static_cast<unsigned long long>(gmask)) - 1;
            atomicAdd(&cnt[g], 1);
            gmask &= gmask - 1;
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < NB; b += blockDim.x)
        chunk_cnt[static_cast<size_t>(blockIdx.x) * NB + b] = cnt[b];
}

__global__ __launch_bounds__(1024) void k_brim_scan(const int32_t *__restrict__ chunk_cnt,
                                                    int nchunks, int Nd, int Ne, int tile_rows,
                                                    int32_t *__restrict__ chunk_base,
                                                    int32_t *__restrict__ sfd_off,
                                                    int32_t *__restrict__ epd_off,
                                                    int32_t *__restrict__ tile_off,
                                                    int32_t *__restrict__ first_cnt,
                                                    int32_t *__restrict__ tile_off_first,
                                                    int32_t *__restrict__ tile_off_rest) {
    __shared__ int total[kMaxBins];
    __shared__ int binoff[kMaxBins];
    const int NB = Nd + 2 * Ne;
    const int lane = lane_id(), wv = threadIdx.x / kWave, nw = blockDim.x / kWave;

    // 1. per bin, exclusive scan over chunks (64 chunks per wave step)
    for (int b = wv; b < NB; b += nw) {
        int run = 0;
        for (int c0 = 0; c0 < nchunks; c0 += kWave) {
            const int c = c0 + lane;
            const int v = c < nchunks ? chunk_cnt[static_cast<size_t>(c) * NB + b] : 0;
            const int incl = wave_incl_scan(v);
            if (c < nchunks) chunk_base[static_cast<size_t>(c) * NB + b] = run + incl - v;
            run += __shfl(incl, kWave - 1);
        }
        if (lane == 0) total[b] = run;
    }
    __syncthreads();

    // 2. across bins: groups give sfd_off; experts (placement order) give
    //    epd_off; first-contributor bins start at their expert's first EPD
    //    row.  ceil(rows / tile_rows) gives the GEMM row-tile schedules: all
    //    rows (up-projection), first contributors and the rest (merge).
    if (wv == 0) {
        const int vg = lane < Nd ? total[lane] : 0;
        const int ig = wave_incl_scan(vg);
        if (lane < Nd) {
            binoff[lane] = ig - vg;
            sfd_off[lane] = ig - vg;
        }
        if (lane == kWave - 1) sfd_off[Nd] = ig;
        int run = 0, run_t = 0, run_f = 0, run_r = 0;
        for (int p0 = 0; p0 < Ne; p0 += kWave) {
            const int p = p0 + lane;
            const int v = p < Ne ? total[Nd + p] : 0;
            const int f = p < Ne ? total[Nd + Ne + p] : 0;
            const int vt = (v + tile_rows - 1) / tile_rows;
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
    __syncthreads();

    // 3. each (chunk, bin) start = start of the bin + rows of earlier chunks
    const size_t n = static_cast<size_t>(nchunks) * NB;
    for (size_t i = threadIdx.x; i < n; i += blockDim.x) chunk_base[i] += binoff[i % NB];
}

__global__ __launch_bounds__(kBrimChunk) void k_brim_fill(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int T, int k, PlaceTab tab,
    const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ sfd_off,
    const int32_t *__restrict__ epd_off, const int32_t *__restrict__ first_cnt, int dense,
    int32_t *__restrict__ brim0, int32_t *__restrict__ epd_src, float *__restrict__ epd_w,
    int32_t *__restrict__ tok_epd, int32_t *__restrict__ down_rows,
    int32_t *__restrict__ brim1) {
    __shared__ unsigned long long wmask[kWavesPerChunk][kMaxBins];
    __shared__ int wpre[kWavesPerChunk][kMaxBins];
    __shared__ int s_base[kMaxBins];
    __shared__ uint8_t s_grp[kMaxNe];
    __shared__ int16_t s_pos[kMaxNe];
    const int Nd = tab.Nd, Ne = tab.Ne, n = tab.n, NB = Nd + 2 * Ne;
    for (int i = threadIdx.x; i < kWavesPerChunk * NB; i += blockDim.x)
        wmask[i / NB][i % NB] = 0ull;
    for (int b = threadIdx.x; b < NB; b += blockDim.x)
        s_base[b] = chunk_base[static_cast<size_t>(blockIdx.x) * NB + b];
    for (int e = threadIdx.x; e < Ne; e += blockDim.x) {
        s_grp[e] = tab.grp[e];
        s_pos[e] = static_cast<int16_t>(tab.grp[e] * n + tab.slot[e]);
    }
    __syncthreads();

    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int t = blockIdx.x * kBrimChunk + threadIdx.x;
    const bool valid = t < T;
    const unsigned long long bit = 1ull << lane, lower = bit - 1ull;
    uint64_t gmask = 0, em[4] = {0, 0, 0, 0};
    if (valid) {
        for (int j = 0; j < k; j++) {
            const int e = ids[static_cast<size_t>(t) * k + j];
            const int p = s_pos[e];
            em[p >> 6] |= 1ull << (p & 63);
            gmask |= 1ull << s_grp[e];
            atomicOr(&wmask[wv][Nd + p], bit);
        }
        for (int j = 0; j < k; j++) {
            const int p = s_pos[ids[static_cast<size_t>(t) * k + j]];
            if (first_in_group(em, p, n)) atomicOr(&wmask[wv][Nd + Ne + p], bit);
        }
        for (uint64_t m = gmask; m; m &= m - 1)
            atomicOr(&wmask[wv][__ffsll(static_cast<unsigned long long>(m)) - 1], bit);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        int run = 0;
        for (int q = 0; q < kWavesPerChunk; q++) {
            wpre[q][b] = run;
            run += __popcll(wmask[q][b]);
        }
    }
    __syncthreads();
    if (!valid) return;

    // rank of this token among the chunk-ordered tokens of bin b
    auto slot_of = [&](int b) { return s_base[b] + wpre[wv][b] + __popcll(wmask[wv][b] & lower); };

    for (int g = 0; g < Nd; g++)
        brim0[static_cast<size_t>(g) * T + t] = ((gmask >> g) & 1ull) ? slot_of(g) : -1;
    for (int j = 0; j < k; j++) {
        const size_t o = static_cast<size_t>(t) * k + j;
        const int p = s_pos[ids[o]], g = p / n;
        const int srow = slot_of(g);
        const int erow = slot_of(Nd + p);
        epd_src[erow] = srow;
        epd_w[erow] = w[o];
        tok_epd[o] = erow;
        // merge order: first contributors of expert p, then its other rows
        const int e0 = epd_off[p];
        const int f_before = slot_of(Nd + Ne + p);  // e0 + first rows of p before t
        if (first_in_group(em, p, n)) down_rows[f_before] = erow;
        else down_rows[e0 + first_cnt[p] + (erow - e0) - (f_before - e0)] = erow;
        if (dense) {
            const int g0 = sfd_off[g], Ng = sfd_off[g + 1] - g0;
            brim1[static_cast<size_t>(n) * g0 + static_cast<size_t>(p - g * n) * Ng + (srow - g0)] =
                erow - epd_off[g * n];
        }
    }
    if (dense) {
        for (uint64_t m = gmask; m; m &= m - 1) {
            const int g = __ffsll(static_cast<unsigned long long>(m)) - 1;
            const int g0 = sfd_off[g], Ng = sfd_off[g + 1] - g0;
            const int srow = slot_of(g);
            for (int j = 0; j < n; j++)
                if (!has_pos(em, g * n + j))
                    brim1[static_cast<size_t>(n) * g0 + static_cast<size_t>(j) * Ng + (srow - g0)] = -1;
        }
    }
}

}  // namespace

hipError_t launch_brim(const int32_t *ids, const float *w, int T, int k, const PlaceTab &tab,
                       int tile_rows, int dense_brim1, const BrimBufs &b, hipStream_t s) {
    const int nchunks = static_cast<int>(ceil_div(T, kBrimChunk));
    k_brim_count<<<nchunks, kBrimChunk, 0, s>>>(ids, T, k, tab, b.chunk_cnt);
    k_brim_scan<<<1, 1024, 0, s>>>(b.chunk_cnt, nchunks, tab.Nd, tab.Ne, tile_rows, b.chunk_base,
                                   b.sfd_off, b.epd_off, b.tile_off, b.first_cnt,
                                   b.tile_off_first, b.tile_off_rest);
    k_brim_fill<<<nchunks, kBrimChunk, 0, s>>>(ids, w, T, k, tab, b.chunk_base, b.sfd_off,
                                               b.epd_off, b.first_cnt, dense_brim1, b.brim0,
                                               b.epd_src, b.epd_w, b.tok_epd, b.down_rows,
                                               b.brim1);
    return hipGetLastError();
}

}  // namespace occ
