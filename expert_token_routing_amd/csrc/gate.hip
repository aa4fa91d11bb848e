// Gate projection g(x) of the router (Occult paper, section 2.1: the router
// logits come from a single linear layer), logits = x W_r^T in fp32.
//
// bf16: one workgroup per 16 tokens x 16 experts, v_mfma_f32_16x16x32_bf16
// over K = d with the operands read straight from global memory (W_r is at
// most 256 x 8192 bf16 and stays in L2; a token row is read by the Ne/16
// workgroups of its row block).  The K range is split over the workgroup's
// 4 waves (a latency-bound product: each wave's chain is a quarter as long)
// and the 4 partial tiles are added in wave order through LDS.  Lane l holds
// the A fragment of token l & 15 and the B fragment of expert l & 15, both at
// K chunk l >> 4, and ends with the 4 logits of expert l & 15 for tokens
// 4 (l >> 4) .. 4 (l >> 4) + 3.  Inside a wave the K loop is unrolled by 4 so
// that 8 fragment loads are in flight per MFMA group.  The accumulation
// order is fixed, so the result does not depend on the launch.
// fp32: one thread per logit, a plain ascending dot product.
#include "launch.h"

namespace occ {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

constexpr int kGateUnroll = 4;
constexpr int kGateWaves = 4;

__global__ __launch_bounds__(kGateWaves *kWave) void k_gate_bf16(const uint16_t *__restrict__ x,
                                                                 const uint16_t *__restrict__ wr,
                                                                 int T, int d, int Ne,
                                                                 float *__restrict__ logits) {
    __shared__ f32x4 part[kGateWaves - 1][kWave];
    const int l = lane_id(), wv = threadIdx.x / kWave;
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
    const int ta = min(t0 + (l & 15), T - 1), eb = min(e0 + (l & 15), Ne - 1);
    const int kc = (l >> 4) * 8;
    const uint16_t *pa = x + static_cast<size_t>(ta) * d + kc;
    const uint16_t *pb = wr + static_cast<size_t>(eb) * d + kc;
    // this wave's 32-deep K steps
    const int steps = d / 32;
    const int kend = (wv + 1) * steps / kGateWaves * 32;
    int k0 = wv * steps / kGateWaves * 32;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (; k0 + 32 * kGateUnroll <= kend; k0 += 32 * kGateUnroll) {
        bf16x8_t a[kGateUnroll], b[kGateUnroll];
#pragma unroll
        for (int u = 0; u < kGateUnroll; u++) {
            a[u] = *reinterpret_cast<const bf16x8_t *>(pa + k0 + 32 * u);
            b[u] = *reinterpret_cast<const bf16x8_t *>(pb + k0 + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < kGateUnroll; u++)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
    }
    for (; k0 < kend; k0 += 32) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(pa + k0);
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t *>(pb + k0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    if (wv > 0) part[wv - 1][l] = acc;
    __syncthreads();
    if (wv > 0) return;
#pragma unroll
    for (int q = 0; q < kGateWaves - 1; q++) acc += part[q][l];
    const int e = e0 + (l & 15);
    if (e >= Ne) return;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int t = t0 + 4 * (l >> 4) + i;
        if (t < T) logits[static_cast<size_t>(t) * Ne + e] = acc[i];
    }
}

__global__ __launch_bounds__(256) void k_gate_f32(const float *__restrict__ x,
                                                  const float *__restrict__ wr, int T, int d,
                                                  int Ne, float *__restrict__ logits) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<size_t>(T) * Ne) return;
    const size_t t = i / Ne, e = i % Ne;
    const float *xr = x + t * d, *wrow = wr + e * d;
    float s = 0.f;
    for (int c = 0; c < d; c++) s = fmaf(xr[c], wrow[c], s);
    logits[i] = s;
}

}  // namespace

hipError_t launch_gate(const void *x, const void *w_router, int T, int d, int Ne, int bf16,
                       float *logits, hipStream_t s) {
    if (bf16) {
        const dim3 grid(ceil_div(T, 16), ceil_div(Ne, 16));
        k_gate_bf16<<<grid, kGateWaves * kWave, 0, s>>>(static_cast<const uint16_t *>(x),
                                           static_cast<const uint16_t *>(w_router), T, d, Ne,
                                           logits);
    } else {
        const size_t n = static_cast<size_t>(T) * Ne;
        k_gate_f32<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
            static_cast<const float *>(x), static_cast<const float *>(w_router), T, d, Ne, logits);
    }
    return hipGetLastError();
}

}  // namespace occ
