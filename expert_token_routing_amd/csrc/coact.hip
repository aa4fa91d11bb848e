// Co-activation statistics of a routed batch (Occult paper, section 2.1
// Eq. 3-4, section 2.2 and Table 1):
//   C[i][j]  tokens whose k experts include both i and j (ordered pairs, so
//            C[i][i] is expert i's load);
//   P        C / max_{i != j} C, one IEEE fp32 division per entry, zero
//            diagonal;
//   n_sfd    distinct groups summed over tokens (the replicas Dispatch
//            makes), CT = n_sfd / T, and the intra-group share of the
//            off-diagonal co-activations.
// k_coact builds a per-workgroup histogram of the k^2 pairs of each token in
// LDS (integer atomics, so the counts are exact in any order) and adds it to
// C with one global atomic per nonzero entry; k_coact_finish reduces and
// divides in one workgroup.
#include "launch.h"

namespace occ {
namespace {

constexpr int kCoactTokens = 1024;
constexpr int kLdsNe = 96;  // LDS histogram up to 96 x 96 counts (36 KB)

__global__ __launch_bounds__(256) void k_coact_zero(int32_t *C, int n, int64_t *n_sfd) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) C[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *n_sfd = 0;
}

// Caller ids outside 0..Ne-1 are counted as expert 0 (unspecified result,
// in-bounds accesses).
__device__ __forceinline__ int in_range(int e, int Ne) {
    return static_cast<unsigned>(e) < static_cast<unsigned>(Ne) ? e : 0;
}

__global__ __launch_bounds__(kCoactTokens) void k_coact(const int32_t *__restrict__ ids, int T,
                                                        int k, PlaceTab tab,
                                                        int32_t *__restrict__ C,
                                                        int64_t *__restrict__ n_sfd) {
    extern __shared__ int hist[];
    __shared__ int s_rep[kCoactTokens / kWave];
    const int Ne = tab.Ne;
    const bool in_lds = Ne <= kLdsNe;
    if (in_lds)
        for (int i = threadIdx.x; i < Ne * Ne; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const int t = blockIdx.x * kCoactTokens + threadIdx.x;
    int reps = 0;
    if (t < T) {
        const int32_t *it = ids + static_cast<size_t>(t) * k;
        uint64_t gmask = 0;
        for (int a = 0; a < k; a++) {
            const int ea = in_range(it[a], Ne);
            gmask |= 1ull << tab.grp[ea];
            for (int b = 0; b < k; b++) {
                const int idx = ea * Ne + in_range(it[b], Ne);
                if (in_lds) atomicAdd(&hist[idx], 1);
                else atomicAdd(&C[idx], 1);
            }
        }
        reps = __popcll(gmask);
    }
    reps = wave_sum_i(reps);
    if (lane_id() == 0) s_rep[threadIdx.x / kWave] = reps;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long s = 0;
        for (int w = 0; w < kCoactTokens / kWave; w++) s += s_rep[w];
        atomicAdd(reinterpret_cast<unsigned long long *>(n_sfd), static_cast<unsigned long long>(s));
    }
    if (in_lds)
        for (int i = threadIdx.x; i < Ne * Ne; i += blockDim.x)
            if (hist[i]) atomicAdd(&C[i], hist[i]);
}

__global__ __launch_bounds__(1024) void k_coact_finish(const int32_t *__restrict__ C, int T,
                                                       PlaceTab tab, float *__restrict__ P,
                                                       const int64_t *__restrict__ n_sfd,
                                                       double *__restrict__ ct,
                                                       double *__restrict__ intra) {
    __shared__ int s_max[1024 / kWave];
    __shared__ long long s_same[1024 / kWave], s_all[1024 / kWave];
    __shared__ int s_mx;
    const int Ne = tab.Ne;
    int mx = 0;
    long long same = 0, all = 0;
    for (int i = threadIdx.x; i < Ne * Ne; i += blockDim.x) {
        const int r = i / Ne, c = i % Ne;
        if (r == c) continue;
        const int v = C[i];
        mx = max(mx, v);
        all += v;
        if (tab.grp[r] == tab.grp[c]) same += v;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        mx = max(mx, __shfl_xor(mx, o));
        same += __shfl_xor(same, o);
        all += __shfl_xor(all, o);
    }
    const int wv = threadIdx.x / kWave;
    if (lane_id() == 0) {
        s_max[wv] = mx;
        s_same[wv] = same;
        s_all[wv] = all;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int m = 0;
        long long sa = 0, al = 0;
        for (int w = 0; w < static_cast<int>(blockDim.x / kWave); w++) {
            m = max(m, s_max[w]);
            sa += s_same[w];
            al += s_all[w];
        }
        s_mx = m;
        *ct = T > 0 ? static_cast<double>(*n_sfd) / static_cast<double>(T) : 0.0;
        *intra = al > 0 ? static_cast<double>(sa) / static_cast<double>(al) : 0.0;
    }
    __syncthreads();
    const int m = s_mx;
    for (int i = threadIdx.x; i < Ne * Ne; i += blockDim.x) {
        const int r = i / Ne, c = i % Ne;
        P[i] = (r == c || m == 0) ? 0.f : static_cast<float>(C[i]) / static_cast<float>(m);
    }
}

}  // namespace

hipError_t launch_coact(const int32_t *ids, int T, int k, const PlaceTab &tab, int32_t *C,
                        float *P, int64_t *n_sfd, double *ct, double *intra, hipStream_t s) {
    const int nn = tab.Ne * tab.Ne;
    k_coact_zero<<<ceil_div(nn, 256), 256, 0, s>>>(C, nn, n_sfd);
    const size_t lds = tab.Ne <= kLdsNe ? sizeof(int) * nn : 0;
    k_coact<<<ceil_div(T, kCoactTokens), kCoactTokens, lds, s>>>(ids, T, k, tab, C, n_sfd);
    k_coact_finish<<<1, 1024, 0, s>>>(C, T, tab, P, n_sfd, ct, intra);
    return hipGetLastError();
}

}  // namespace occ
