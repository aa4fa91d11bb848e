// Router: top-k softmax gating (Occult paper, section 2.1, Eq. 2) with
// collaboration pruning (section 3.3), routing-score-based or
// expert-similarity-based.
//
// Without pruning and with at most 64 experts, k_route_rows takes one
// 16-lane row per token (below).  Otherwise one 64-lane wave per token;
// lane l holds the logits of experts l, l+64, ...
// Softmax max and denominator are wave reductions.  The top k are selected
// without cross-lane shuffles: each logit maps to an unsigned key that keeps
// its order, the k-th largest key is found bit by bit from wave ballots
// (a radix select), ties at that key go to the lower expert index, and a
// selected expert's place in the list is the number of selected experts
// that precede it in (logit descending, index ascending) order.  Softmax is
// monotone, so selecting on the logits selects the top k probabilities.  A
// NaN logit ranks as -inf, so the k results are always distinct experts.
#include "launch.h"

namespace occ {
namespace {

constexpr int kRouteWaves = 4;  // tokens per workgroup

template <int NI>
struct TokenLogits {
    float v[NI];
};

// Key of a logit for selection: a larger logit has a larger key, -0 and +0
// share one key (they compare equal), and -inf maps to 0x007fffff, so every
// logit's key is above 0, the key of experts that may not be chosen.
__device__ __forceinline__ uint32_t logit_key(float v) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The k experts of largest logit among those whose group bit is set in
// `allowed`, in (logit descending, index ascending) order, go to sel / sel_l
// (per-wave LDS, k entries; sel_l holds the logit, NaN read as -inf).
template <int NI>
__device__ void select_topk(const TokenLogits<NI> &l, int Ne, int k, uint64_t allowed,
                            const uint8_t *s_grp, int *sel, float *sel_l) {
    const int lane = lane_id();
    float v[NI];
    uint32_t key[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const int e = lane + kWave * i;
        v[i] = l.v[i] == l.v[i] ? l.v[i] : -INFINITY;
        const bool ok = e < Ne && ((allowed >> s_grp[e]) & 1ull);
        key[i] = ok ? logit_key(v[i]) : 0u;
    }
    // k-th largest key: the largest t with at least k keys >= t
    uint32_t thr = 0;
    for (int b = 31; b >= 0; b--) {
        const uint32_t cand = thr | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NI; i++) cnt += __popcll(__ballot(key[i] >= cand));
        if (cnt >= k) thr = cand;
    }
    // every key above thr, then keys equal to thr in expert order up to k
    int need = k;
#pragma unroll
    for (int i = 0; i < NI; i++) need -= __popcll(__ballot(key[i] > thr));
    const uint64_t below = (1ull << lane) - 1ull;
    bool take[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const uint64_t eq = __ballot(key[i] == thr);
        take[i] = key[i] > thr || (key[i] == thr && static_cast<int>(__popcll(eq & below)) < need);
        need -= min(need, static_cast<int>(__popcll(eq)));
    }
    // place in the list: selected experts with a larger key, or an equal key
    // and a lower index
    int rank[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) rank[i] = 0;
#pragma unroll
    for (int i2 = 0; i2 < NI; i2++) {
        for (uint64_t m = __ballot(take[i2]); m; m &= m - 1) {
            const int j = __builtin_ctzll(m);
            const uint32_t kj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key[i2]), j));
            const int ej = j + kWave * i2;
#pragma unroll
            for (int i = 0; i < NI; i++)
                rank[i] += kj > key[i] || (kj == key[i] && ej < lane + kWave * i);
        }
    }
#pragma unroll
    for (int i = 0; i < NI; i++)
        if (take[i]) {
            sel[rank[i]] = lane + kWave * i;
            sel_l[rank[i]] = v[i];
        }
    __builtin_amdgcn_wave_barrier();
}

// Bit e of a 256-bit expert set held as four words.
__device__ __forceinline__ bool in_set(const uint64_t (&m)[4], int e) {
    const uint64_t w = e < 64 ? m[0] : e < 128 ? m[1] : e < 192 ? m[2] : m[3];
    return (w >> (e & 63)) & 1ull;
}
__device__ __forceinline__ void add_to_set(uint64_t (&m)[4], int e) {
    const uint64_t bit = 1ull << (e & 63);
    if (e < 64) m[0] |= bit;
    else if (e < 128) m[1] |= bit;
    else if (e < 192) m[2] |= bit;
    else m[3] |= bit;
}

// Expert-similarity-based pruning (section 3.3): walking the top-k list
// sel[0..k) in score order, an expert outside the allowed groups is replaced
// by the first expert of its ranked similarity row that is allowed and not
// yet selected (the list's allowed experts plus earlier replacements).  The
// replacement keeps the replaced expert's place, and its logit in sel_l, so
// it inherits the routing weight.  The lanes test 64 row entries at a time
// and a ballot finds the first hit.  A row that is not a permutation of the
// experts may find none; the expert then stays (in bounds, unspecified).
__device__ void replace_similar(const int32_t *__restrict__ sim_rank, int Ne, int k,
                                uint64_t chosen, const uint8_t *s_grp, int *sel) {
    const int lane = lane_id();
    uint64_t picked[4] = {0, 0, 0, 0};
    for (int j = 0; j < k; j++)
        if ((chosen >> s_grp[sel[j]]) & 1ull) add_to_set(picked, sel[j]);
    for (int j = 0; j < k; j++) {
        const int e = sel[j];
        if ((chosen >> s_grp[e]) & 1ull) continue;
        const int32_t *row = sim_rank + static_cast<size_t>(e) * Ne;
        int rep = e;
        for (int q0 = 0; q0 < Ne; q0 += kWave) {
            const int q = q0 + lane;
            const int c = q < Ne ? row[q] : -1;
            const bool ok = c >= 0 && c < Ne && ((chosen >> s_grp[c]) & 1ull) && !in_set(picked, c);
            const uint64_t hit = __ballot(ok);
            if (hit) {
                rep = __shfl(c, __builtin_ctzll(hit));
                break;
            }
        }
        add_to_set(picked, rep);
        if (lane == 0) sel[j] = rep;
        __builtin_amdgcn_wave_barrier();
    }
}

// The plain top k (no pruning) for Ne <= 64 experts: one DPP
// row of 16 lanes per token, four tokens per wave; lane r holds the logits
// of experts r, r + 16, r + 32, r + 48.  Row maxima and sums are four
// row-shift steps, after which lane 15 of the row holds the result, and a
// row broadcast spreads it over the row.  The top k are k rounds of a row
// maximum of the logits' order-keeping keys followed by a row minimum of
// the expert indices that hold it, so ties go to the lower index as in the
// wave kernel; round i's winner is recorded by lane i (lane i - 16 for
// i >= 16) and cleared by its owner.  The softmax denominator
// takes 6 addition levels, as in the wave kernel (two inside the lane,
// four across the row): the same error bound, possibly another rounding.
constexpr int kRouteRowThreads = 256;  // 16 tokens per workgroup

// Lane 15 of each row of 16 lanes, copied to the whole row (the
// row_newbcast DPP control of gfx90a and later).
constexpr int kDppRowNewBcast15 = 0x15F;
__device__ __forceinline__ int row_bcast15(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kDppRowNewBcast15, 0xf, 0xf, false);
}
__device__ __forceinline__ float row_bcast15(float v) { return __int_as_float(row_bcast15(__float_as_int(v))); }

template <int N>  // N = ceil(k / 16) rounds per recording lane (1)
__global__ __launch_bounds__(kRouteRowThreads) void k_route_rows(const float *__restrict__ logits,
                                                                 int T, int Ne, int k,
                                                                 int32_t *__restrict__ ids,
                                                                 float *__restrict__ w) {
    const int lane = lane_id(), r = lane & 15;
    const int t = (blockIdx.x * kRouteRowThreads + static_cast<int>(threadIdx.x)) >> 4;
    const bool live = t < T;  // a row past T computes on -inf and stores nothing
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int e = r + 16 * j;
        v[j] = live && e < Ne ? logits[static_cast<size_t>(t) * Ne + e] : -INFINITY;
    }
    // row maximum
    float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    m = fmaxf(m, dpp_f<kDppRowShr1, 0xf>(-INFINITY, m));
    m = fmaxf(m, dpp_f<kDppRowShr2, 0xf>(-INFINITY, m));
    m = fmaxf(m, dpp_f<kDppRowShr4, 0xf>(-INFINITY, m));
    m = fmaxf(m, dpp_f<kDppRowShr8, 0xf>(-INFINITY, m));
    m = row_bcast15(m);
    // denominator: two levels in the lane, four across the row
    float ex[4];
#pragma unroll
    for (int j = 0; j < 4; j++) ex[j] = r + 16 * j < Ne ? expf(v[j] - m) : 0.f;
    float s = (ex[0] + ex[1]) + (ex[2] + ex[3]);
    s += dpp_f<kDppRowShr1, 0xf>(0.f, s);
    s += dpp_f<kDppRowShr2, 0xf>(0.f, s);
    s += dpp_f<kDppRowShr4, 0xf>(0.f, s);
    s += dpp_f<kDppRowShr8, 0xf>(0.f, s);
    s = row_bcast15(s);
    uint32_t key[4];  // 0: not an expert, or already chosen
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float x = v[j] == v[j] ? v[j] : -INFINITY;  // NaN ranks as -inf
        key[j] = r + 16 * j < Ne ? logit_key(x) : 0u;
    }
    uint32_t mine_key[N];
    int mine_e[N];
#pragma unroll
    for (int q = 0; q < N; q++) {
        mine_key[q] = 0;
        mine_e[q] = 0;
    }
    for (int i = 0; i < k; i++) {
        // the row's largest key ...
        uint32_t b = max(max(key[0], key[1]), max(key[2], key[3]));
        b = max(b, static_cast<uint32_t>(dpp_i<kDppRowShr1, 0xf>(0, static_cast<int>(b))));
        b = max(b, static_cast<uint32_t>(dpp_i<kDppRowShr2, 0xf>(0, static_cast<int>(b))));
        b = max(b, static_cast<uint32_t>(dpp_i<kDppRowShr4, 0xf>(0, static_cast<int>(b))));
        b = max(b, static_cast<uint32_t>(dpp_i<kDppRowShr8, 0xf>(0, static_cast<int>(b))));
        b = static_cast<uint32_t>(row_bcast15(static_cast<int>(b)));
        // ... and the lowest expert that holds it, as the largest 255 - e
        // (e < 64, so 0 marks a lane without one)
        uint32_t c = 0;
#pragma unroll
        for (int j = 3; j >= 0; j--) c = key[j] == b ? 255u - (r + 16 * j) : c;
        c = max(c, static_cast<uint32_t>(dpp_i<kDppRowShr1, 0xf>(0, static_cast<int>(c))));
        c = max(c, static_cast<uint32_t>(dpp_i<kDppRowShr2, 0xf>(0, static_cast<int>(c))));
        c = max(c, static_cast<uint32_t>(dpp_i<kDppRowShr4, 0xf>(0, static_cast<int>(c))));
        c = max(c, static_cast<uint32_t>(dpp_i<kDppRowShr8, 0xf>(0, static_cast<int>(c))));
        const int e = 255 - row_bcast15(static_cast<int>(c));
#pragma unroll
        for (int j = 0; j < 4; j++) key[j] = r + 16 * j == e ? 0u : key[j];
#pragma unroll
        for (int q = 0; q < N; q++)
            if (i == r + 16 * q) {
                mine_key[q] = b;
                mine_e[q] = e;
            }
    }
#pragma unroll
    for (int q = 0; q < N; q++) {
        const int slot = r + 16 * q;
        if (live && slot < k) {
            // the logit back from its key (exact; -0 reads as +0, NaN as -inf)
            const uint32_t kb = mine_key[q];
            const float l = __uint_as_float((kb & 0x80000000u) ? (kb & 0x7fffffffu) : ~kb);
            const size_t o = static_cast<size_t>(t) * k + slot;
            ids[o] = mine_e[q];
            w[o] = expf(l - m) / s;
        }
    }
}

// Caller-supplied routing made safe for the BRIM kernels: a token's id that
// is out of range or repeats an earlier one is replaced by the lowest expert
// not yet in the token's list, with weight 0.  Valid tokens are copied
// unchanged.  One thread per token.
__global__ __launch_bounds__(256) void k_sanitize_ids(const int32_t *__restrict__ ids_in,
                                                      const float *__restrict__ w_in, int T,
                                                      int k, int Ne, int32_t *__restrict__ ids,
                                                      float *__restrict__ w) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const size_t o = static_cast<size_t>(t) * k;
    for (int j = 0; j < k; j++) {
        int e = ids_in[o + j];
        float wj = w_in[o + j];
        bool ok = e >= 0 && e < Ne;
        for (int q = 0; q < j && ok; q++) ok = ids[o + q] != e;
        if (!ok) {
            wj = 0.f;
            for (e = 0; e < Ne; e++) {
                bool used = false;
                for (int q = 0; q < j && !used; q++) used = ids[o + q] == e;
                if (!used) break;
            }
        }
        ids[o + j] = e;
        w[o + j] = wj;
    }
}

template <int NI>
__global__ __launch_bounds__(kRouteWaves *kWave) void k_route(const float *__restrict__ logits,
                                                              int T, int Ne, int k,
                                                              int prune_rule, int G,
                                                              PlaceTab tab,
                                                              const int32_t *__restrict__ sim_rank,
                                                              int32_t *__restrict__ ids,
                                                              float *__restrict__ w) {
    __shared__ uint8_t s_grp[kMaxNe];
    __shared__ int s_sel[kRouteWaves][kMaxK];
    __shared__ float s_sell[kRouteWaves][kMaxK];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int t = blockIdx.x * kRouteWaves + wv;
    // the logits load is issued before the table fill and its barrier
    TokenLogits<NI> l;
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const int e = lane + kWave * i;
        l.v[i] = e < Ne && t < T ? logits[static_cast<size_t>(t) * Ne + e] : -INFINITY;
    }
    for (int e = threadIdx.x; e < Ne; e += blockDim.x) s_grp[e] = tab.grp[e];
    __syncthreads();
    if (t >= T) return;

    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; i++) m = fmaxf(m, l.v[i]);
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
        if (static_cast<int>(__popcll(span)) > G) {
            uint64_t chosen = 0;
            if (prune_rule == 1 || prune_rule == 3) {
                // TRAVERSE (and similarity-based pruning): groups of the top-k
                // list in score order, first G.
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
            if (prune_rule == 3)
                replace_similar(sim_rank, Ne, k, chosen, s_grp, sel);
            else
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
                        const PlaceTab &tab, const int32_t *sim_rank, int32_t *ids, float *w,
                        hipStream_t s) {
    if (prune_rule == 0 && Ne <= kWave) {
        const dim3 g(ceil_div(static_cast<size_t>(T) * 16, kRouteRowThreads)), b(kRouteRowThreads);
        if (k <= 16) k_route_rows<1><<<g, b, 0, s>>>(logits, T, Ne, k, ids, w);
        else k_route_rows<2><<<g, b, 0, s>>>(logits, T, Ne, k, ids, w);
        return hipGetLastError();
    }
    const dim3 grid(ceil_div(T, kRouteWaves)), block(kRouteWaves * kWave);
    const int ni = (Ne + kWave - 1) / kWave;
    switch (ni) {
        case 1: k_route<1><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, sim_rank, ids, w); break;
        case 2: k_route<2><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, sim_rank, ids, w); break;
        case 3: k_route<3><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, sim_rank, ids, w); break;
        default: k_route<4><<<grid, block, 0, s>>>(logits, T, Ne, k, prune_rule, G, tab, sim_rank, ids, w); break;
    }
    return hipGetLastError();
}

hipError_t launch_sanitize_ids(const int32_t *ids_in, const float *w_in, int T, int k, int Ne,
                               int32_t *ids, float *w, hipStream_t s) {
    k_sanitize_ids<<<ceil_div(T, 256), 256, 0, s>>>(ids_in, w_in, T, k, Ne, ids, w);
    return hipGetLastError();
}

}  // namespace occ
