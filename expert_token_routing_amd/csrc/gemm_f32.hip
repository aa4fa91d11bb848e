// The two grouped expert GEMMs of the Occult pipeline in fp32 (same
// semantics as gemm_bf16.hip: SMM scattering with SwiGLU and weight
// modulation, Algorithms 6-7; SMM merging with fp32 accumulation, Algorithm
// 8), on the vector ALUs.  On MI355X fp32 vector FMA and fp32 MFMA have the
// same peak, so a plain LDS-tiled kernel suffices for the fp32 workloads.
//
// A 256-thread workgroup computes 64 rows x 64 output columns; thread
// (ty, tx) owns rows ty + 16*i and columns tx + 16*j (i, j < 4), so the LDS
// reads of a 16-thread row are consecutive.  K slices of 64 are staged
// K-major in LDS; the next slice's loads go out into registers before the
// current one is multiplied, so that a tile waits for one load round trip
// per 64-deep slice (16-deep slices loaded one at a time left the small
// fp32 layers' GEMMs waiting on a round trip every 16 k).  Every output
// accumulates its k in ascending order, one fma each.  Tile scheduling
// follows the same per-expert row-tile schedule as the bf16 kernels, with
// 64-row tiles.
#include "launch.h"

namespace occ {
namespace {

constexpr int BM = kGemmBmF32;  // 64
constexpr int BN = 64;
constexpr int BK = 16;           // k per load step (K is a multiple of 16)
constexpr int NS = 4;            // load steps per LDS slice
constexpr int BKS = BK * NS;     // 64-deep LDS slices
constexpr int PAD = 4;

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

// A 64 x 16 step of an operand (rows K-contiguous): thread tid holds 4
// consecutive k of row tid / 4, loaded as one 16-byte vector; put() writes
// it into the LDS slice as [k][row].
__device__ __forceinline__ f32x4 take(const float *const src_row, int k0) {
    return *reinterpret_cast<const f32x4 *>(src_row + k0 + (threadIdx.x & 3) * 4);
}
__device__ __forceinline__ void put(float (*dst)[BM + PAD], int kk0, const f32x4 &v) {
    const int q = kk0 + (threadIdx.x & 3) * 4, r = threadIdx.x >> 2;
    dst[q + 0][r] = v.x;
    dst[q + 1][r] = v.y;
    dst[q + 2][r] = v.z;
    dst[q + 3][r] = v.w;
}

__global__ __launch_bounds__(256) void k_gemm_up_f32(UpArgs a) {
    __shared__ float sA[BKS][BM + PAD], sG[BKS][BN + PAD], sU[BKS][BN + PAD];
    Tile t;
    if (!tile_of(a.seg_off, a.tile_off, a.M, a.Ne, a.tab, (a.N + BN - 1) / BN, t)) return;
    const int K = a.K, N = a.N;
    const int r_ld = threadIdx.x >> 2;
    const int row_ld = t.seg + t.m0 + min(r_ld, t.rows - 1);
    const int src = a.a_rows ? a.a_rows[row_ld] : row_ld;
    const float *a_row = static_cast<const float *>(a.A) + static_cast<size_t>(src) * K;
    const int f_ld = min(t.n0 + r_ld, N - 1);
    const size_t wbase = static_cast<size_t>(t.e) * N * K + static_cast<size_t>(f_ld) * K;
    const float *g_row = static_cast<const float *>(a.Wg) + wbase;
    const float *u_row = static_cast<const float *>(a.Wu) + wbase;

    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float ag[4][4] = {}, au[4][4] = {};
    f32x4 ra[NS], rg[NS], ru[NS];
    auto load = [&](int k0) {
#pragma unroll
        for (int s = 0; s < NS; s++)
            if (k0 + BK * s < K) {
                ra[s] = take(a_row, k0 + BK * s);
                rg[s] = take(g_row, k0 + BK * s);
                ru[s] = take(u_row, k0 + BK * s);
            }
    };
    load(0);
    for (int k0 = 0; k0 < K; k0 += BKS) {
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NS; s++)
            if (k0 + BK * s < K) {
                put(sA, BK * s, ra[s]);
                put(sG, BK * s, rg[s]);
                put(sU, BK * s, ru[s]);
            }
        __syncthreads();
        if (k0 + BKS < K) load(k0 + BKS);
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (k0 + BK * s >= K) break;
#pragma unroll
            for (int kk = BK * s; kk < BK * (s + 1); kk++) {
                float av[4], gv[4], uv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) av[i] = sA[kk][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    gv[j] = sG[kk][tx + 16 * j];
                    uv[j] = sU[kk][tx + 16 * j];
                }
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        ag[i][j] = fmaf(av[i], gv[j], ag[i][j]);
                        au[i][j] = fmaf(av[i], uv[j], au[i][j]);
                    }
            }
        }
    }
    float *out = static_cast<float *>(a.out);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = ty + 16 * i;
        if (r >= t.rows) continue;
        const size_t row = static_cast<size_t>(t.seg) + t.m0 + r;
        const float wr = a.row_w ? a.row_w[row] : 1.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int f = t.n0 + tx + 16 * j;
            if (f >= N) continue;
            const float g = ag[i][j];
            out[row * N + f] = g / (1.f + expf(-g)) * au[i][j] * wr;
        }
    }
}

__global__ __launch_bounds__(256) void k_gemm_down_f32(DownArgs a) {
    __shared__ float sA[BKS][BM + PAD], sB[BKS][BN + PAD];
    Tile t;
    if (!tile_of(a.seg_off, a.tile_off, a.M, a.Ne, a.tab, (a.N + BN - 1) / BN, t, a.first_cnt,
                 a.phase))
        return;
    const int K = a.K, N = a.N, ksp = a.k_split;
    const int r_ld = threadIdx.x >> 2;
    const int row_ld = t.seg + t.m0 + min(r_ld, t.rows - 1);
    const float *a_row = static_cast<const float *>(a.A) +
                         static_cast<size_t>(a.rows ? a.rows[row_ld] : row_ld) * K;
    const int n_ld = min(t.n0 + r_ld, N - 1);
    const float *W = static_cast<const float *>(a.W) + static_cast<size_t>(t.e) * N * K;
    const size_t blk = static_cast<size_t>(N) * ksp;

    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    f32x4 ra[NS], rb[NS];
    auto load = [&](int k0) {
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const int k = k0 + BK * s;
            if (k < K) {
                ra[s] = take(a_row, k);
                // step k lies in block k / ksp (ksp is a multiple of 16)
                rb[s] = take(W + (k / ksp) * blk + static_cast<size_t>(n_ld) * ksp, k % ksp);
            }
        }
    };
    load(0);
    for (int k0 = 0; k0 < K; k0 += BKS) {
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NS; s++)
            if (k0 + BK * s < K) {
                put(sA, BK * s, ra[s]);
                put(sB, BK * s, rb[s]);
            }
        __syncthreads();
        if (k0 + BKS < K) load(k0 + BKS);
#pragma unroll
        for (int s = 0; s < NS; s++) {
            if (k0 + BK * s >= K) break;
#pragma unroll
            for (int kk = BK * s; kk < BK * (s + 1); kk++) {
                float av[4], bv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) av[i] = sA[kk][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 4; j++) bv[j] = sB[kk][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = ty + 16 * i;
        if (r >= t.rows) continue;
        const size_t row = static_cast<size_t>(t.seg) + t.m0 + r;
        const int erow = a.rows ? a.rows[row] : static_cast<int>(row);
#pragma unroll
        for (int j = 0; j < 4; j++) {
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
    k_gemm_up_f32<<<static_cast<unsigned>(grid), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemm_down_f32(const DownArgs &a, size_t max_m_tiles, hipStream_t s) {
    const size_t grid = max_m_tiles * ceil_div(a.N, BN);
    if (grid == 0) return hipSuccess;
    k_gemm_down_f32<<<static_cast<unsigned>(grid), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace occ
