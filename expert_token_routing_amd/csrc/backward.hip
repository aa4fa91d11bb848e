// Small kernels of the backward pass: the row-tile schedules of the
// input-gradient GEMMs, and the router's backward (routing-weight and logit
// gradients through Eq. 2's full softmax).
#include "launch.h"

namespace occ {
namespace {

// One workgroup, thread p owns placement position p; a serial scan over the
// (at most 256) positions by thread 0 keeps it trivially deterministic.  The
// all-rows schedule is filled to whole rounds of the CUs for fill_cols
// column tiles (fill_rounds), as the forward's is.
__global__ __launch_bounds__(kMaxNe) void k_tile_sched(const int32_t *__restrict__ epd_off,
                                                       const int32_t *__restrict__ first_cnt,
                                                       int Ne, int bm, int fill_cols, int slots,
                                                       int32_t *__restrict__ t_all,
                                                       int32_t *__restrict__ t_first,
                                                       int32_t *__restrict__ t_rest) {
    __shared__ int s_len[kMaxNe], s_all[kMaxNe], s_first[kMaxNe], s_rest[kMaxNe];
    const int p = threadIdx.x;
    if (p < Ne) {
        const int len = epd_off[p + 1] - epd_off[p], f = first_cnt[p];
        s_len[p] = len;
        s_all[p] = (len + bm - 1) / bm;
        s_first[p] = (f + bm - 1) / bm;
        s_rest[p] = (len - f + bm - 1) / bm;
    }
    __syncthreads();
    if (fill_cols > 0 && p < kWave) fill_rounds(s_len, s_all, Ne, fill_cols, slots, kBrimMaxFill);
    __syncthreads();
    if (p == 0) {
        int a = 0, f = 0, r = 0;
        for (int q = 0; q < Ne; q++) {
            t_all[q] = a;
            t_first[q] = f;
            t_rest[q] = r;
            a += s_all[q];
            f += s_first[q];
            r += s_rest[q];
        }
        t_all[Ne] = a;
        t_first[Ne] = f;
        t_rest[Ne] = r;
    }
}

__global__ void k_dense_sched(int T, int m_tiles, int32_t *seg_off, int32_t *tile_off) {
    if (threadIdx.x == 0) {
        seg_off[0] = 0;
        seg_off[1] = T;
        tile_off[0] = 0;
        tile_off[1] = m_tiles;
    }
}

// dst[c * ldd + r] = src[r * C + c] for 64 x 64 tiles of bf16 bits staged
// through LDS: each thread loads two 16-byte row pieces and stores two
// 16-byte pieces of the transposed rows; blockIdx.z selects the matrix.
constexpr int kTr = 64;
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t *__restrict__ src, int C,
                                                       size_t src_z, uint16_t *__restrict__ dst,
                                                       int ldd, size_t dst_z) {
    __shared__ uint16_t s[kTr][kTr + 2];
    const int r0 = blockIdx.y * kTr, c0 = blockIdx.x * kTr, t = threadIdx.x, ch = t & 7;
    src += blockIdx.z * src_z;
    dst += blockIdx.z * dst_z;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = (t >> 3) + 32 * i;
        const u16x8_t v =
            *reinterpret_cast<const u16x8_t *>(src + static_cast<size_t>(r0 + r) * C + c0 + ch * 8);
#pragma unroll
        for (int j = 0; j < 8; j++) s[r][ch * 8 + j] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int c = (t >> 3) + 32 * i;
        u16x8_t v;
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = s[ch * 8 + j][c];
        *reinterpret_cast<u16x8_t *>(dst + static_cast<size_t>(c0 + c) * ldd + r0 + ch * 8) = v;
    }
}

constexpr int kRbWaves = 4;  // tokens per workgroup

// One wave per token.  Lane j < k sums its EPD row's dw partials in order;
// the softmax is recomputed from the logits (lane l holds experts l, l+64..).
//   dlogits[e] = p_e ([e chosen] dw_(j of e) - sum_j dw_j p_(e_j))
template <int NI>
__global__ __launch_bounds__(kRbWaves *kWave) void k_route_backward(
    const float *__restrict__ logits, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ tok_epd, const float *__restrict__ dw_part, int nparts,
    int dw_stride, int T, int Ne, int k, float *__restrict__ dw, float *__restrict__ dlogits) {
    const int lane = lane_id();
    const int t = blockIdx.x * kRbWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const float *lt = logits ? logits + static_cast<size_t>(t) * Ne : nullptr;
    float lv[NI];
    float m = -INFINITY, s = 1.f;
    if (lt) {
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const int e = lane + kWave * i;
            lv[i] = e < Ne ? lt[e] : -INFINITY;
            m = fmaxf(m, lv[i]);
        }
        m = wave_max(m);
        s = 0.f;
#pragma unroll
        for (int i = 0; i < NI; i++)
            if (lane + kWave * i < Ne) s += expf(lv[i] - m);
        s = wave_sum(s);
    }

    int my_e = -1;
    float my_dw = 0.f, contrib = 0.f;
    if (lane < k) {
        const size_t o = static_cast<size_t>(t) * k + lane;
        my_e = ids[o];
        const float *dp = dw_part + static_cast<size_t>(tok_epd[o]) * dw_stride;
        for (int q = 0; q < nparts; q++) my_dw += dp[q];
        if (dw) dw[o] = my_dw;
        if (lt) contrib = my_dw * (expf(lt[my_e] - m) / s);
    }
    if (!dlogits || !lt) return;
    const float acc = wave_sum(contrib);
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const int e = lane + kWave * i;
        float chosen = 0.f;
        for (int j = 0; j < k; j++) {
            const int ej = __shfl(my_e, j);
            const float dj = __shfl(my_dw, j);
            if (ej == e) chosen = dj;
        }
        if (e < Ne) {
            const float p = expf(lv[i] - m) / s;
            dlogits[static_cast<size_t>(t) * Ne + e] = p * (chosen - acc);
        }
    }
}

}  // namespace

hipError_t launch_tile_sched(const int32_t *epd_off, const int32_t *first_cnt, int Ne,
                             int tile_rows, int fill_cols, int32_t *tile_off,
                             int32_t *tile_off_first, int32_t *tile_off_rest, hipStream_t s) {
    k_tile_sched<<<1, kMaxNe, 0, s>>>(epd_off, first_cnt, Ne, tile_rows, fill_cols, compute_units(),
                                      tile_off, tile_off_first, tile_off_rest);
    return hipGetLastError();
}

hipError_t launch_dense_sched(int T, int m_tiles, int32_t *seg_off, int32_t *tile_off,
                              hipStream_t s) {
    k_dense_sched<<<1, kWave, 0, s>>>(T, m_tiles, seg_off, tile_off);
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void *src, int R, int C, size_t src_z, void *dst, int ldd,
                                 size_t dst_z, int nz, hipStream_t s) {
    if (R % kTr || C % kTr || ldd < R || nz < 1) return hipErrorInvalidValue;
    if (R == 0 || C == 0) return hipSuccess;
    k_transpose_bf16<<<dim3(C / kTr, R / kTr, nz), 256, 0, s>>>(
        static_cast<const uint16_t *>(src), C, src_z, static_cast<uint16_t *>(dst), ldd, dst_z);
    return hipGetLastError();
}

hipError_t launch_route_backward(const float *logits, const int32_t *ids, const int32_t *tok_epd,
                                 const float *dw_part, int nparts, int dw_stride, int T, int Ne,
                                 int k, float *dw, float *dlogits, hipStream_t s) {
    const dim3 grid(ceil_div(T, kRbWaves)), block(kRbWaves * kWave);
    const int ni = (Ne + kWave - 1) / kWave;
#define OCC_RB(N)                                                                                 \
    k_route_backward<N><<<grid, block, 0, s>>>(logits, ids, tok_epd, dw_part, nparts, dw_stride, \
                                               T, Ne, k, dw, dlogits)
    switch (ni) {
        case 1: OCC_RB(1); break;
        case 2: OCC_RB(2); break;
        case 3: OCC_RB(3); break;
        default: OCC_RB(4); break;
    }
#undef OCC_RB
    return hipGetLastError();
}

}  // namespace occ
