// Internal helpers shared by the HIP sources of the Occult MoE-layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace occ {

constexpr int kWave = 64;

// Native 16-byte vectors for register-resident staging (HIP's uint4/float4
// wrap a union, which keeps per-thread arrays of them out of registers).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int kMaxNe = 256;
constexpr int kMaxNd = 64;
constexpr int kMaxK = 32;
constexpr int kMaxBins = kMaxNd + 2 * kMaxNe;  // BRIM bins: groups, experts, first contributors

// Row-tile capacity of the bf16 grouped GEMMs (at most this many tokens per
// workgroup tile); the BRIM scan gives each expert ceil(rows / capacity)
// tiles, whose rows the GEMMs share out evenly.
#ifndef OCC_GEMM_BM
#define OCC_GEMM_BM 320
#endif
constexpr int kGemmBmBf16 = OCC_GEMM_BM;
constexpr int kGemmBmF32 = 32;

// The expert placement, passed by value as a kernel argument (no device copy,
// validated on the host).  Position p = g*n + j holds expert `expert[p]`.
struct PlaceTab {
    uint8_t grp[kMaxNe];     // group of expert e
    uint8_t slot[kMaxNe];    // index of expert e inside its group
    uint8_t expert[kMaxNe];  // expert at placement position p
    int32_t Ne, Nd, n;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave scans and reductions on the DPP lane network (gfx9 row shifts and row
// broadcasts), with no LDS traffic: shifts by 1, 2, 4 and 8 inside each row
// of 16 lanes give row-local inclusive scans, then lane 15 of each row is
// added into the next row and lane 31 into the upper two rows.  A lane
// whose DPP source does not exist receives the identity.  The combination
// order is fixed, so results are deterministic.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int identity, int v) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float identity, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v),
                                                      CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_i<kDppRowShr1, 0xf>(0, v);
    v += dpp_i<kDppRowShr2, 0xf>(0, v);
    v += dpp_i<kDppRowShr4, 0xf>(0, v);
    v += dpp_i<kDppRowShr8, 0xf>(0, v);
    v += dpp_i<kDppRowBcast15, 0xa>(0, v);
    v += dpp_i<kDppRowBcast31, 0xc>(0, v);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
    return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppRowShr1, 0xf>(0.f, v);
    v += dpp_f<kDppRowShr2, 0xf>(0.f, v);
    v += dpp_f<kDppRowShr4, 0xf>(0.f, v);
    v += dpp_f<kDppRowShr8, 0xf>(0.f, v);
    v += dpp_f<kDppRowBcast15, 0xa>(0.f, v);
    v += dpp_f<kDppRowBcast31, 0xc>(0.f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppRowShr1, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppRowShr2, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppRowShr4, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppRowShr8, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppRowBcast15, 0xa>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppRowBcast31, 0xc>(-INFINITY, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Wave-wide arg-max of (value, index): larger value wins, ties to the lower
// index.  Every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        float ov = __shfl_xor(v, o);
        int oi = __shfl_xor(i, o);
        if (ov > v || (ov == v && oi < i)) {
            v = ov;
            i = oi;
        }
    }
}

inline unsigned ceil_div(size_t a, size_t b) { return static_cast<unsigned>((a + b - 1) / b); }

// Placement position owning row tile tm of a grouped GEMM: the last p < Ne
// with tile_off[p] <= tm (tile_off non-decreasing from 0, tm < tile_off[Ne]),
// i.e. the count of such p minus one.  The lanes read the schedule in one
// round trip (four entries each at most) and wave ballots count, instead of
// a binary search's log2(Ne) dependent loads at the start of every tile.
// Every lane of the wave must call it; all get the same result.
__device__ __forceinline__ int tile_owner(const int32_t *tile_off, int Ne, int tm) {
    const int lane = lane_id();
    int v[kMaxNe / kWave];
#pragma unroll
    for (int j = 0; j < kMaxNe / kWave; j++) {
        const int p = lane + kWave * j;
        v[j] = p < Ne ? tile_off[p] : 0x7fffffff;
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kMaxNe / kWave; j++) cnt += __popcll(__ballot(v[j] <= tm));
    return cnt - 1;
}

// Maximum of an unsigned 64-bit value over the wave (both halves moved by
// the same DPP steps as the scans above; 0 is the identity).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = static_cast<uint32_t>(dpp_i<CTRL, ROW_MASK>(0, static_cast<int>(v)));
    const uint32_t hi = static_cast<uint32_t>(dpp_i<CTRL, ROW_MASK>(0, static_cast<int>(v >> 32)));
    return static_cast<uint64_t>(hi) << 32 | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t o;
    o = dpp_u64<kDppRowShr1, 0xf>(v), v = o > v ? o : v;
    o = dpp_u64<kDppRowShr2, 0xf>(v), v = o > v ? o : v;
    o = dpp_u64<kDppRowShr4, 0xf>(v), v = o > v ? o : v;
    o = dpp_u64<kDppRowShr8, 0xf>(v), v = o > v ? o : v;
    o = dpp_u64<kDppRowBcast15, 0xa>(v), v = o > v ? o : v;
    o = dpp_u64<kDppRowBcast31, 0xc>(v), v = o > v ? o : v;
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), kWave - 1);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), kWave - 1);
    return static_cast<uint64_t>(hi) << 32 | lo;
}

// A grouped GEMM's row-tile schedule, filled to whole rounds of the CUs
// (run by one wave; vt[p] holds ceil(rows[p] / capacity) on entry, p < Ne
// <= 256).  With those tiles, a product of T0 row tiles x fill_cols column
// tiles ends in a partly empty round of the `slots` workgroups the GPU runs
// at once; the experts take extra row tiles, one at a time, until the count
// is the most that still fits the same number of rounds: each to the expert
// whose tiles hold the most rows (rows / tiles largest; ties to the lower
// placement position) among those whose tiles could still lose a 16-row
// block.  An expert's rows are shared out evenly over its tiles, so its
// tiles get shorter and the last round fills (at most max_fill extra tiles).
// Lane l keeps experts l + 64 j in registers; each step takes the wave's
// largest key floor(rows / tiles * 2^40) * 256 + (255 - p) (a 64-bit DPP max
// over the lanes), which orders the experts exactly as their rows / tiles
// while an expert has at most 4096 tiles.
__device__ inline uint64_t fill_key(int rows, int tiles, int p) {
    if (tiles == 0 || tiles >= (rows + 15) / 16) return 0;  // cannot split further
    // rows / tiles <= the tile capacity (< 512): the fp64 quotient is
    // correctly rounded and its 40 fractional bits keep distinct ratios of
    // experts with at most 4096 tiles apart (no integer division)
    const double r = static_cast<double>(rows) / static_cast<double>(tiles);
    return static_cast<uint64_t>(r * 1099511627776.0) << 8 | static_cast<uint64_t>(255 - p);
}
__device__ inline void fill_rounds(const int *rows, int *vt, int Ne, int fill_cols, int slots,
                                   int max_fill) {
    const int lane = lane_id();
    int v[4], t[4];
    uint64_t key[4];
    int t0 = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int p = lane + kWave * j;
        v[j] = p < Ne ? rows[p] : 0;
        t[j] = p < Ne ? vt[p] : 0;
        key[j] = p < Ne ? fill_key(v[j], t[j], p) : 0;
        t0 += t[j];
    }
    t0 = wave_sum_i(t0);
    const int64_t cols = fill_cols, rounds = (static_cast<int64_t>(t0) * cols + slots - 1) / slots;
    const int64_t room = rounds * slots / cols - t0;
    const int extra = static_cast<int>(room < max_fill ? room : max_fill);
    for (int it = 0; it < extra; it++) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < 4; j++) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
        if (best == 0) break;  // wave-uniform
        const int p = 255 - static_cast<int>(best & 255);
        if ((p & (kWave - 1)) == lane) {
            const int j = p / kWave;
#pragma unroll
            for (int q = 0; q < 4; q++)
                if (q == j) {
                    t[q] += 1;
                    key[q] = fill_key(v[q], t[q], p);
                }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int p = lane + kWave * j;
        if (p < Ne) vt[p] = t[j];
    }
}

}  // namespace occ
