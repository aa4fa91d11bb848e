// Memory-bound row movers of the Occult pipeline (paper, appendix A.2):
//   dispatch  ORI -> SFD (Algorithm 4): each token row is read once and
//             written once per group it uses, at BRIM_0[g, t]; optionally
//             the same rows of an fp32 buffer are zeroed on the way (the
//             accumulator of a merge done entirely with atomic adds);
//   merge     the deterministic stage one of Algorithm 8: sfd_out[BRIM_0[g,
//             t]] = sum, in ascending placement position, of the fp32 results
//             y_epd of the token's EPD rows in group g (no atomics);
//   combine   SFD -> ORI (Algorithm 9): y[t] = sum over g of
//             sfd_out[BRIM_0[g, t]], entries -1 skipped, summed in fp32 in
//             ascending group order, plus the shared experts' fp32 output,
//             cast once to the output dtype.
// One 64-lane wave per token row; lanes move 16-byte vectors, so a wave
// touches whole contiguous rows (fully coalesced).  BRIM_0's column for the
// token is read by lanes 0..Nd-1 and broadcast with shuffles.
#include <algorithm>

#include "launch.h"

namespace occ {
namespace {

constexpr int kRowWaves = 4;  // token rows per workgroup

template <int VPL>
__global__ __launch_bounds__(kRowWaves *kWave) void k_dispatch(const u32x4 *__restrict__ x, int T,
                                                               int Nd, int row_vec,
                                                               const int32_t *__restrict__ brim0,
                                                               u32x4 *__restrict__ x_sfd,
                                                               f32x4 *__restrict__ zero_out,
                                                               int zero_vec) {
    const int lane = lane_id();
    const int t = blockIdx.x * kRowWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const int br = lane < Nd ? brim0[static_cast<size_t>(lane) * T + t] : -1;
    u32x4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = min(lane + kWave * i, row_vec - 1);
        v[i] = x[static_cast<size_t>(t) * row_vec + c];
    }
    for (int g = 0; g < Nd; g++) {
        const int r = __shfl(br, g);
        if (r < 0) continue;
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = lane + kWave * i;
            if (c < row_vec) x_sfd[static_cast<size_t>(r) * row_vec + c] = v[i];
        }
        if (zero_out)
            for (int c = lane; c < zero_vec; c += kWave)
                zero_out[static_cast<size_t>(r) * zero_vec + c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *__restrict__ p, size_t n, int32_t v) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = v;
}

// A row that is read once (the combine's SFD rows and shared-expert rows):
// non-temporal loads keep it out of the caches the GEMMs rely on.
template <int VPL>
__device__ __forceinline__ void load_row(const f32x4 *__restrict__ src, int lane, int row_vec4,
                                         f32x4 (&v)[VPL]) {
#pragma unroll
    for (int i = 0; i < VPL; i++)
        v[i] = __builtin_nontemporal_load(src + min(lane + kWave * i, row_vec4 - 1));
}

// The groups holding a replica of the token are the set bits of `mask`;
// rows are summed in ascending group order, two rows' loads in flight at a
// time.
template <int VPL, bool BF16>
__global__ __launch_bounds__(kRowWaves *kWave) void k_combine(const f32x4 *__restrict__ sfd_out,
                                                              const int32_t *__restrict__ brim0,
                                                              const f32x4 *__restrict__ y_sh,
                                                              int T, int Nd, int row_vec4,
                                                              void *__restrict__ y) {
    const int lane = lane_id();
    const int t = blockIdx.x * kRowWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const int br = lane < Nd ? brim0[static_cast<size_t>(lane) * T + t] : -1;
    uint64_t mask = __ballot(br >= 0);
    f32x4 acc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (VPL > 8) {  // wide rows: one row at a time keeps registers in bounds
        for (; mask; mask &= mask - 1) {
            const int r = __shfl(br, __ffsll(static_cast<unsigned long long>(mask)) - 1);
            const f32x4 *src = sfd_out + static_cast<size_t>(r) * row_vec4;
#pragma unroll
            for (int i = 0; i < VPL; i++) acc[i] += src[min(lane + kWave * i, row_vec4 - 1)];
        }
        if (y_sh) {
            const f32x4 *src = y_sh + static_cast<size_t>(t) * row_vec4;
#pragma unroll
            for (int i = 0; i < VPL; i++) acc[i] += src[min(lane + kWave * i, row_vec4 - 1)];
        }
    } else {
    f32x4 a[VPL], b[VPL];
    while (mask) {
        const int g0 = __ffsll(static_cast<unsigned long long>(mask)) - 1;
        mask &= mask - 1;
        const int r0 = __shfl(br, g0);
        load_row<VPL>(sfd_out + static_cast<size_t>(r0) * row_vec4, lane, row_vec4, a);
        if (mask) {
            const int g1 = __ffsll(static_cast<unsigned long long>(mask)) - 1;
            mask &= mask - 1;
            const int r1 = __shfl(br, g1);
            load_row<VPL>(sfd_out + static_cast<size_t>(r1) * row_vec4, lane, row_vec4, b);
#pragma unroll
            for (int i = 0; i < VPL; i++) acc[i] = (acc[i] + a[i]) + b[i];
        } else {
#pragma unroll
            for (int i = 0; i < VPL; i++) acc[i] += a[i];
        }
    }
    if (y_sh) {
        load_row<VPL>(y_sh + static_cast<size_t>(t) * row_vec4, lane, row_vec4, a);
#pragma unroll
        for (int i = 0; i < VPL; i++) acc[i] += a[i];
    }
    }
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane + kWave * i;
        if (c >= row_vec4) continue;
        const size_t o = static_cast<size_t>(t) * row_vec4 + c;
        if constexpr (BF16) {
            uint2 packed;
            packed.x = static_cast<uint32_t>(f32_to_bf16_bits(acc[i].x)) |
                       (static_cast<uint32_t>(f32_to_bf16_bits(acc[i].y)) << 16);
            packed.y = static_cast<uint32_t>(f32_to_bf16_bits(acc[i].z)) |
                       (static_cast<uint32_t>(f32_to_bf16_bits(acc[i].w)) << 16);
            reinterpret_cast<uint2 *>(y)[o] = packed;
        } else {
            reinterpret_cast<f32x4 *>(y)[o] = acc[i];
        }
    }
}

// SPLIT waves per token, each owning VPL * 64 consecutive float4 columns of
// the row (rows of more than 1024 fp32 values are split, which keeps a
// wave's registers, and so the waves in flight per CU, within bounds).
// Lane j < k holds the token's j-th expert: placement
// position p_j and EPD row erow_j; after a sort by position (the positions
// are distinct), lane r holds the r-th.  The walk visits each group's
// experts together, in slot order (a group's positions are contiguous).  A
// group's first expert (its first contributor) left its result in the
// group's SFD row, the others at their EPD rows: the walk starts each group
// from the SFD row, adds the others in turn and writes the row back when
// there were any (a single-expert group's row is final as it is).
// With Y, the kernel also finishes the layer as the combine would: the
// group sums are added in ascending group order (the order in which the walk
// meets them), then the shared experts' row, and the result is cast once --
// the same additions in the same order, so y is the combine's bit for bit.
// The next row's loads are issued before the current row is added.  Every
// byte it moves is touched once, so its loads and stores are non-temporal:
// kept out of the L2 and the last-level cache, they no longer evict the
// weights and activations the next step's GEMMs read (measured on the
// OLMoE-shaped step: -8% here and -2.5% in the following up-projection;
// -13% in the decode step's up-projection).
template <int VPL, int Y, int SPLIT>  // Y: 0 none, 1 bf16, 2 fp32
__global__ __launch_bounds__(kRowWaves *kWave) void k_merge_slots(
    const f32x4 *__restrict__ y_epd, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ tok_epd, const int32_t *__restrict__ brim0, PlaceTab tab, int T,
    int k, int row_vec4, f32x4 *__restrict__ sfd_out, const f32x4 *__restrict__ y_sh,
    void *__restrict__ y) {
    const int lane = lane_id();
    const int gw = blockIdx.x * kRowWaves + threadIdx.x / kWave;
    const int t = gw / SPLIT;
    if (t >= T) return;
    const int c0 = (gw - t * SPLIT) * (VPL * kWave) + lane;  // this lane's first float4 column
    // Independent loads first, so that their latencies overlap: the token's
    // experts and EPD rows, its SFD row in every group (lane g: BRIM_0[g,
    // t]; only the groups it uses are read below) and the shared experts'
    // row.
    int e = 0, erow = 0, grow = 0;
    if (lane < k) {
        const size_t o = static_cast<size_t>(t) * k + lane;
        e = ids[o];
        erow = tok_epd[o];
    }
    if (lane < tab.Nd) grow = brim0[static_cast<size_t>(lane) * T + t];
    f32x4 ys[VPL];
    if constexpr (Y != 0) {
        if (y_sh) {
            const f32x4 *src = y_sh + static_cast<size_t>(t) * row_vec4;
#pragma unroll
            for (int i = 0; i < VPL; i++)
                ys[i] = __builtin_nontemporal_load(src + min(c0 + kWave * i, row_vec4 - 1));
        }
    }
    const int p = lane < k ? tab.grp[e] * tab.n + tab.slot[e] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < k; j++) rank += __shfl(p, j) < p;
    int sp = 0, se = 0;  // lane r: position and EPD row of the r-th expert
    for (int j = 0; j < k; j++) {
        const int rj = __shfl(rank, j), pj = __shfl(p, j), ej = __shfl(erow, j);
        if (rj == lane) {
            sp = pj;
            se = ej;
        }
    }
    // lane r: does it open its group, and the row its result is read from
    const int sg = sp / tab.n;
    const int prev_g = __shfl(sg, lane > 0 ? lane - 1 : 0);
    const int opens = lane == 0 || prev_g != sg;
    const int g_row = __shfl(grow, lane < k ? sg : 0);
    const int src_row = lane < k && opens ? g_row : se;
    f32x4 acc[VPL], ya[VPL], cur[VPL], nxt[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        ya[i] = acc[i];
    }
    auto load = [&](int r, f32x4 (&v)[VPL]) {
        const f32x4 *row = (__shfl(opens, r) ? sfd_out : y_epd) +
                           static_cast<size_t>(__shfl(src_row, r)) * row_vec4;
#pragma unroll
        for (int i = 0; i < VPL; i++)
            v[i] = __builtin_nontemporal_load(row + min(c0 + kWave * i, row_vec4 - 1));
    };
    int cur_srow = 0;
    load(0, cur);
    for (int r = 0; r < k; r++) {
        if (r + 1 < k) load(r + 1, nxt);
        const bool op = __shfl(opens, r) != 0;
        const bool closes = r + 1 == k || __shfl(opens, r + 1) != 0;
        if (op) cur_srow = __shfl(src_row, r);
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            acc[i] = op ? cur[i] : acc[i] + cur[i];
            cur[i] = nxt[i];
        }
        if (closes) {
            f32x4 *dst = sfd_out + static_cast<size_t>(cur_srow) * row_vec4;
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                const int c = c0 + kWave * i;
                if (!op && c < row_vec4) __builtin_nontemporal_store(acc[i], dst + c);
                if (Y) ya[i] += acc[i];
            }
        }
    }
    if constexpr (Y != 0) {
        if (y_sh) {
#pragma unroll
            for (int i = 0; i < VPL; i++) ya[i] += ys[i];
        }
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = c0 + kWave * i;
            if (c >= row_vec4) continue;
            const size_t o = static_cast<size_t>(t) * row_vec4 + c;
            if constexpr (Y == 1) {
                uint2 packed;
                packed.x = static_cast<uint32_t>(f32_to_bf16_bits(ya[i].x)) |
                           (static_cast<uint32_t>(f32_to_bf16_bits(ya[i].y)) << 16);
                packed.y = static_cast<uint32_t>(f32_to_bf16_bits(ya[i].z)) |
                           (static_cast<uint32_t>(f32_to_bf16_bits(ya[i].w)) << 16);
                typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
                __builtin_nontemporal_store(u32x2_t{packed.x, packed.y},
                                            reinterpret_cast<u32x2_t *>(y) + o);
            } else {
                reinterpret_cast<f32x4 *>(y)[o] = ya[i];
            }
        }
    }
}

}  // namespace

hipError_t launch_merge_slots(const float *y_epd, const int32_t *ids, const int32_t *tok_epd,
                              const int32_t *brim0, const PlaceTab &tab, int T, int k, int d,
                              float *sfd_out, const float *y_sh, void *y, int y_bf16,
                              hipStream_t s) {
    const int row_vec4 = d / 4;
    const int vpl = (row_vec4 + kWave - 1) / kWave;
    const dim3 block(kRowWaves * kWave);
    const f32x4 *ye = reinterpret_cast<const f32x4 *>(y_epd);
    f32x4 *so = reinterpret_cast<f32x4 *>(sfd_out);
    const f32x4 *ys = reinterpret_cast<const f32x4 *>(y_sh);
    const int ymode = y ? (y_bf16 ? 1 : 2) : 0;
#define OCC_MERGE_Y(V, YM, S)                                                             \
    k_merge_slots<V, YM, S><<<dim3(ceil_div(static_cast<size_t>(T) * S, kRowWaves)), block, 0, \
                              s>>>(ye, ids, tok_epd, brim0, tab, T, k, row_vec4, so, ys, y)
#define OCC_MERGE(V, S)                            \
    do {                                           \
        if (ymode == 1) OCC_MERGE_Y(V, 1, S);      \
        else if (ymode == 2) OCC_MERGE_Y(V, 2, S); \
        else OCC_MERGE_Y(V, 0, S);                 \
    } while (0)
    if (vpl <= 1) OCC_MERGE(1, 1);
    else if (vpl <= 2) OCC_MERGE(2, 1);
    else if (vpl <= 4) OCC_MERGE(4, 1);
    // d = 2048: eight waves per token, one 16-byte vector per lane and row
    // (against two waves of four: 4.7% faster at the Qwen shape, 2-4% on
    // the OLMoE- and DeepSeek-shaped batches; four waves of two were 1%
    // slower): more rows' loads in flight across the CU
    else if (vpl <= 8) OCC_MERGE(1, 8);
    else if (vpl <= 16) OCC_MERGE(4, 4);
    else OCC_MERGE(4, 8);
#undef OCC_MERGE
#undef OCC_MERGE_Y
    return hipGetLastError();
}

hipError_t launch_dispatch(const void *x, int T, int Nd, size_t row_bytes, const int32_t *brim0,
                           void *x_sfd, hipStream_t s, float *zero_out, int zero_cols) {
    const int row_vec = static_cast<int>(row_bytes / 16);
    const int vpl = (row_vec + kWave - 1) / kWave;
    const dim3 grid(ceil_div(T, kRowWaves)), block(kRowWaves * kWave);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    u32x4 *xd = static_cast<u32x4 *>(x_sfd);
    f32x4 *zo = reinterpret_cast<f32x4 *>(zero_out);
    const int zv = zero_cols / 4;
    if (vpl <= 1) k_dispatch<1><<<grid, block, 0, s>>>(xs, T, Nd, row_vec, brim0, xd, zo, zv);
    else if (vpl <= 2) k_dispatch<2><<<grid, block, 0, s>>>(xs, T, Nd, row_vec, brim0, xd, zo, zv);
    else if (vpl <= 4) k_dispatch<4><<<grid, block, 0, s>>>(xs, T, Nd, row_vec, brim0, xd, zo, zv);
    else if (vpl <= 8) k_dispatch<8><<<grid, block, 0, s>>>(xs, T, Nd, row_vec, brim0, xd, zo, zv);
    else k_dispatch<16><<<grid, block, 0, s>>>(xs, T, Nd, row_vec, brim0, xd, zo, zv);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, size_t n, int32_t v, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(std::min<size_t>(ceil_div(n, 256), 4096));
    k_fill_i32<<<grid > 0 ? grid : 1, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

hipError_t launch_combine(const float *sfd_out, const int32_t *brim0, const float *y_sh, int T,
                          int Nd, int d, int out_bf16, void *y, hipStream_t s) {
    const int row_vec4 = d / 4;
    const int vpl = (row_vec4 + kWave - 1) / kWave;
    const dim3 grid(ceil_div(T, kRowWaves)), block(kRowWaves * kWave);
    const f32x4 *so = reinterpret_cast<const f32x4 *>(sfd_out);
    const f32x4 *ys = reinterpret_cast<const f32x4 *>(y_sh);
#define OCC_COMBINE(V)                                                                        \
    do {                                                                                      \
        if (out_bf16) k_combine<V, true><<<grid, block, 0, s>>>(so, brim0, ys, T, Nd, row_vec4, y); \
        else k_combine<V, false><<<grid, block, 0, s>>>(so, brim0, ys, T, Nd, row_vec4, y);       \
    } while (0)
    if (vpl <= 1) OCC_COMBINE(1);
    else if (vpl <= 2) OCC_COMBINE(2);
    else if (vpl <= 4) OCC_COMBINE(4);
    else if (vpl <= 8) OCC_COMBINE(8);
    else if (vpl <= 16) OCC_COMBINE(16);
    else OCC_COMBINE(32);
#undef OCC_COMBINE
    return hipGetLastError();
}

}  // namespace occ
