// The two grouped expert GEMMs of the Occult pipeline in fp32 (same
// semantics as gemm_bf16.hip: SMM scattering with SwiGLU and weight
// modulation, Algorithms 6-7; SMM merging with fp32 accumulation, Algorithm
// 8), on the vector ALUs.  On MI355X fp32 vector FMA and fp32 MFMA have the
// same peak, so a plain LDS-tiled kernel suffices for the fp32 workloads.
//
// A 256-thread workgroup computes 32 rows x 32 output columns; thread
// (ty, tx) owns rows ty + 16*i and columns tx + 16*j (i, j < 2), so the LDS
// reads of a 16-thread row are consecutive.  The fp32 layers here are small
// (hundreds of tokens), where a tile's length, not the CUs' throughput,
// sets the time: 32 x 32 tiles give four times the workgroups of 64 x 64
// ones, each a quarter of the serial FMAs per thread.  K slices of 64 are
// staged K-major in LDS; the next slice's loads go out into registers
// before the current one is multiplied, so that a tile waits for one load
// round trip per 64-deep slice.  Every output accumulates its k in
// ascending order, one fma each.  Tile scheduling follows the same
// per-expert row-tile schedule as the bf16 kernels, with 32-row tiles.
#include "launch.h"

namespace occ {
namespace {

constexpr int BM = kGemmBmF32;  // 32
constexpr int BN = 32;
constexpr int BKS = 64;          // k per LDS slice (K is a multiple of 16)
constexpr int PAD = 4;
constexpr int NT = 256;
static_assert(BM == 32 && BN == 32, "thread (ty, tx) owns 2 x 2 outputs");

struct Tile {
    int e, seg, m0, rows, n0;
    int first;  // phase 3: the tile's first `first` rows are first contributors
};

// Routed tiles walk expert segments [seg_off[p], seg_off[p+1]) -- all rows
// (phases 0 and 3), the first first_cnt[p] rows (phase 1) or the rest
// (phase 2).
__device__ __forceinline__ bool tile_of(const int32_t *seg_off, const int32_t *tile_off, int M,
                                        int Ne, const PlaceTab &tab, int n_tiles, Tile &t,
                                        const int32_t *first_cnt = nullptr, int phase = 0) {
    const int tm = blockIdx.x / n_tiles, tn = blockIdx.x % n_tiles;
    if (seg_off) {
        if (tm >= tile_off[Ne]) return false;
        const int p = tile_owner(tile_off, Ne, tm);
        const int seg0 = seg_off[p], len = seg_off[p + 1] - seg0;
        const int nf = phase == 1 || phase == 2 ? first_cnt[p] : 0;
        t.e = tab.expert[p];
        t.seg = phase == 2 ? seg0 + nf : seg0;
        t.m0 = (tm - tile_off[p]) * BM;
        t.rows = min(BM, (phase == 1 ? nf : len - nf) - t.m0);
        t.first = phase == 3 ? first_cnt[p] - t.m0 : 0;
    } else {
        if (tm * BM >= M) return false;
        t.e = 0;
        t.seg = 0;
        t.m0 = tm * BM;
        t.rows = min(BM, M - t.m0);
        t.first = 0;
    }
    t.n0 = tn * BN;
    return true;
}

// Loads of a 64-deep slice of a 32-row operand (rows K-contiguous): thread
// tid moves 4 consecutive k (k4 = 4 (tid & 15)) of rows (tid >> 4) and
// (tid >> 4) + 16, one 16-byte vector each; put() writes them into the LDS
// slice as [k][row].  A vector past K (a multiple of 16) is not loaded.
__device__ __forceinline__ int k4_of() { return (threadIdx.x & 15) * 4; }
__device__ __forceinline__ f32x4 take(const float *const src_row, int k0) {
    return *reinterpret_cast<const f32x4 *>(src_row + k0 + k4_of());
}
__device__ __forceinline__ void put(float (*dst)[BM + PAD], int h, const f32x4 &v) {
    const int q = k4_of(), r = (threadIdx.x >> 4) + 16 * h;
    dst[q + 0][r] = v.x;
    dst[q + 1][r] = v.y;
    dst[q + 2][r] = v.z;
    dst[q + 3][r] = v.w;
}

__global__ __launch_bounds__(NT) void k_gemm_up_f32(UpArgs a) {
    __shared__ float sA[BKS][BM + PAD], sG[BKS][BN + PAD], sU[BKS][BN + PAD];
    Tile t;
    if (!tile_of(a.seg_off, a.tile_off, a.M, a.Ne, a.tab, (a.N + BN - 1) / BN, t)) return;
    const int K = a.K, N = a.N;
    const int r_ld = threadIdx.x >> 4;
    const float *a_row[2], *g_row[2], *u_row[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int row_ld = t.seg + t.m0 + min(r_ld + 16 * h, t.rows - 1);
        const int src = a.a_rows ? a.a_rows[row_ld] : row_ld;
        a_row[h] = static_cast<const float *>(a.A) + static_cast<size_t>(src) * K;
        const int f_ld = min(t.n0 + r_ld + 16 * h, N - 1);
        const size_t wbase = static_cast<size_t>(t.e) * N * K + static_cast<size_t>(f_ld) * K;
        g_row[h] = static_cast<const float *>(a.Wg) + wbase;
        u_row[h] = static_cast<const float *>(a.Wu) + wbase;
    }

    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float ag[2][2] = {}, au[2][2] = {};
    f32x4 ra[2], rg[2], ru[2];
    auto load = [&](int k0) {
        if (k0 + k4_of() < K) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                ra[h] = take(a_row[h], k0);
                rg[h] = take(g_row[h], k0);
                ru[h] = take(u_row[h], k0);
            }
        }
    };
    load(0);
    for (int k0 = 0; k0 < K; k0 += BKS) {
        __syncthreads();
        if (k0 + k4_of() < K) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                put(sA, h, ra[h]);
                put(sG, h, rg[h]);
                put(sU, h, ru[h]);
            }
        }
        __syncthreads();
        if (k0 + BKS < K) load(k0 + BKS);
        const int kn = min(BKS, K - k0);  // a multiple of 16
#pragma unroll
        for (int s16 = 0; s16 < BKS; s16 += 16) {
            if (s16 >= kn) break;
#pragma unroll
            for (int kk = s16; kk < s16 + 16; kk++) {
                float av[2], gv[2], uv[2];
#pragma unroll
                for (int i = 0; i < 2; i++) av[i] = sA[kk][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    gv[j] = sG[kk][tx + 16 * j];
                    uv[j] = sU[kk][tx + 16 * j];
                }
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        ag[i][j] = fmaf(av[i], gv[j], ag[i][j]);
                        au[i][j] = fmaf(av[i], uv[j], au[i][j]);
                    }
            }
        }
    }
    float *out = static_cast<float *>(a.out);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = ty + 16 * i;
        if (r >= t.rows) continue;
        const size_t row = static_cast<size_t>(t.seg) + t.m0 + r;
        const float wr = a.row_w ? a.row_w[row] : 1.f;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int f = t.n0 + tx + 16 * j;
            if (f >= N) continue;
            const float g = ag[i][j];
            out[row * N + f] = g / (1.f + expf(-g)) * au[i][j] * wr;
        }
    }
}

__global__ __launch_bounds__(NT) void k_gemm_down_f32(DownArgs a) {
    __shared__ float sA[BKS][BM + PAD], sB[BKS][BN + PAD];
    Tile t;
    if (!tile_of(a.seg_off, a.tile_off, a.M, a.Ne, a.tab, (a.N + BN - 1) / BN, t, a.first_cnt,
                 a.phase))
        return;
    const int K = a.K, N = a.N, ksp = a.k_split;
    const int r_ld = threadIdx.x >> 4;
    const float *a_row[2];
    size_t b_row[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int row_ld = t.seg + t.m0 + min(r_ld + 16 * h, t.rows - 1);
        a_row[h] = static_cast<const float *>(a.A) +
                   static_cast<size_t>(a.rows ? a.rows[row_ld] : row_ld) * K;
        b_row[h] = static_cast<size_t>(min(t.n0 + r_ld + 16 * h, N - 1)) * ksp;
    }
    const float *W = static_cast<const float *>(a.W) + static_cast<size_t>(t.e) * N * K;
    const size_t blk = static_cast<size_t>(N) * ksp;

    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[2][2] = {};
    f32x4 ra[2], rb[2];
    auto load = [&](int k0) {
        const int k = k0 + k4_of();
        if (k < K) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                ra[h] = take(a_row[h], k0);
                // k lies in block k / ksp (ksp is a multiple of 16, so the
                // thread's 4 k do too)
                rb[h] = *reinterpret_cast<const f32x4 *>(W + (k / ksp) * blk + b_row[h] + k % ksp);
            }
        }
    };
    load(0);
    for (int k0 = 0; k0 < K; k0 += BKS) {
        __syncthreads();
        if (k0 + k4_of() < K) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                put(sA, h, ra[h]);
                put(sB, h, rb[h]);
            }
        }
        __syncthreads();
        if (k0 + BKS < K) load(k0 + BKS);
        const int kn = min(BKS, K - k0);  // a multiple of 16
#pragma unroll
        for (int s16 = 0; s16 < BKS; s16 += 16) {
            if (s16 >= kn) break;
#pragma unroll
            for (int kk = s16; kk < s16 + 16; kk++) {
                float av[2], bv[2];
#pragma unroll
                for (int i = 0; i < 2; i++) av[i] = sA[kk][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 2; j++) bv[j] = sB[kk][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = ty + 16 * i;
        if (r >= t.rows) continue;
        const size_t row = static_cast<size_t>(t.seg) + t.m0 + r;
        const int erow = a.rows ? a.rows[row] : static_cast<int>(row);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int c = t.n0 + tx + 16 * j;
            if (c >= N) continue;
            if (!a.dst_rows) a.out[row * N + c] = acc[i][j];
            else if (a.phase == 3 && r >= t.first) a.epd_out[static_cast<size_t>(erow) * N + c] = acc[i][j];
            else if (a.phase == 1 || a.phase == 3) a.out[static_cast<size_t>(a.dst_rows[erow]) * N + c] = acc[i][j];
            else unsafeAtomicAdd(a.out + static_cast<size_t>(a.dst_rows[erow]) * N + c, acc[i][j]);
        }
    }
}

}  // namespace

hipError_t launch_gemm_up_f32(const UpArgs &a, size_t max_m_tiles, hipStream_t s) {
    const size_t grid = max_m_tiles * ceil_div(a.N, BN);
    if (grid == 0) return hipSuccess;
    k_gemm_up_f32<<<static_cast<unsigned>(grid), NT, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemm_down_f32(const DownArgs &a, size_t max_m_tiles, hipStream_t s) {
    const size_t grid = max_m_tiles * ceil_div(a.N, BN);
    if (grid == 0) return hipSuccess;
    k_gemm_down_f32<<<static_cast<unsigned>(grid), NT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace occ
