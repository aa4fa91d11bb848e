// Router: top-k softmax gating (Occult paper, section 2.1, Eq. 2) with
// routing-score-based collaboration pruning (section 3.3).
//
// One 64-lane wave per token; lane l holds the logits of experts l, l+64, ...
// Softmax max and denominator are wave reductions; the top k come from k
// rounds of a wave arg-max on (logit, -index), so the order is (logit
// descending, index ascending).  Softmax is monotone, so selecting on the
// logits selects the top k probabilities.
#include "launch.h"

namespace occ {
namespace {

constexpr int kRouteWaves = 4;  // tokens per workgroup

template <int NI>
struct TokenLogits {
    float v[NI];
};

// k rounds of arg-max over the experts whose group bit is set in `allowed`.
// Winners go to sel/sel_l (per-wave LDS, k entries).
template <int NI>
__device__ void select_topk(const TokenLogits<NI> &l, int Ne, int k, uint64_t allowed,
                            const uint8_t *s_grp, int *sel, float *sel_l) {
    const int lane = lane_id();
    uint32_t taken = 0;
    bool ok[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const int e = lane + kWave * i;
        ok[i] = e < Ne && ((allowed >> s_grp[e]) & 1ull);
    }
    for (int j = 0; j < k; j++) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const int e = lane + kWave * i;
            if (ok[i] && !((taken >> i) & 1u) && (l.v[i] > bv || (l.v[i] == bv && e < bi))) {
                bv = l.v[i];
                bi = e;
            }
        }
        wave_argmax(bv, bi);
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        if (lane == 0) {
            sel[j] = bi;
            sel_l[j] = bv;
        }
    }
    __builtin_amdgcn_wave_barrier();
}

template <int NI>
__global__ __launch_bounds__(kRouteWaves *kWave) void k_route(const float *__restrict__ logits,
                                                              int T, int Ne, int k,
                                                              int prune_rule, int G,
                                                              PlaceTab tab,
                                                              int32_t *__restrict__ ids,
                                                              float *__restrict__ w) {
    __shared__ uint8_t s_grp[kMaxNe];
    __shared__ int s_sel[kRouteWaves][kMaxK];
    __shared__ float s_sell[kRouteWaves][kMaxK];
    for (int e = threadIdx.x; e < Ne; e += blockDim.x) s_grp[e] = tab.grp[e];
    __syncthreads();

    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int t = blockIdx.x * kRouteWaves + wv;
    if (t >= T) return;

    TokenLogits<NI> l;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const int e = lane + kWave * i;
        l.v[i] = e < Ne ? logits[static_cast<size_t>(t) * Ne + e] : -INFINITY;
        m = fmaxf(m, l.v[i]);
    }
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NI; i++)
        if (lane + kWave * i < Ne) s += expf(l.v[i] - m);
    s = wave_sum(s);

    int *sel = s_sel[wv];
    float *sel_l = s_sell[wv];
    const int Nd = tab.Nd;
    const uint64_t all_groups = Nd >= 64 ? ~0ull : ((1ull << Nd) - 1);
    select_topk<NI>(l, Ne, k, all_groups, s_grp, sel, sel_l);

    if (prune_rule != 0 && G < Nd) {
        uint64_t span = 0;
        for (int j = 0; j < k; j++) span |= 1ull << s_grp[sel[j]];
        if (__popcll(span) > G) {
            uint64_t chosen = 0;
            if (prune_rule == 1) {
                // TRAVERSE: groups of the top-k list in score order, first G.
                int have = 0;
                for (int j = 0; j < k && have < G; j++) {
                    const uint64_t bit = 1ull << s_grp[sel[j]];
                    if (!(chosen & bit)) {
                        chosen |= bit;
                        have++;
                    }
                }
            } else {
                // GROUPSUM: lane g sums, in top-k order, the fp32 logits of the
                // group's top-k members; G rounds of arg-max pick the groups.
                float score = 0.f;
                bool elig = false;
                for (int j = 0; j < k; j++) {
                    if (s_grp[sel[j]] == lane) {
                        score = score + sel_l[j];
                        elig = true;
                    }
                }
                for (int r = 0; r < G; r++) {
                    const bool cand = lane < Nd && elig && !((chosen >> lane) & 1ull);
                    float bv = cand ? score : -INFINITY;
                    int bi = cand ? lane : 0x7fffffff;
                    wave_argmax(bv, bi);
                    if (bi == 0x7fffffff) break;
                    chosen |= 1ull << bi;
                }
            }
            __builtin_amdgcn_wave_barrier();
            select_topk<NI>(l, Ne, k, chosen, s_grp, sel, sel_l);
        }
    }

    if (lane < k) {
        const size_t o = static_cast<size_t>(t) * k + lane;
        ids[o] = sel[lane];
        w[o] = expf(sel_l[lane] - m) / s;
    }
}

}  // namespace

hipError_t launch_route(const float *logits, int T, int Ne, int k, int prune_rule, int G,
                        const PlaceTab &tab, int32_t *ids, float *w, hipStream_t s) {
    const dim3 grid(ceil_div(T, kRouteWaves)), block(kRouteWaves * kWave);
    const int ni = (Ne + kWave - 1) / kWave;
    switch (ni) {
        case 1: k_route<1><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, ids, w); break;
        case 2: k_route<2><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, ids, w); break;
        case 3: k_route<3><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, ids, w); break;
        default: k_route<4><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, ids, w); break;
    }
    return hipGetLastError();
}

}  // namespace occ
