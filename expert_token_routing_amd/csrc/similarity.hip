// Expert similarity table (Occult paper, appendix A.3, Eq. 6-8), used by the
// expert-similarity-based collaboration pruning of section 3.3.
//
//   k_sim_gram  gram[i][j] += sum over the batch's tokens of H[t][i] H[t][j],
//               fp64, tokens in ascending order for every entry.  The product
//               of two fp32 logits is exact in fp64, so an FMA rounds exactly
//               like a separate add and each entry is bit-identical to the
//               plain sequential sum.  A 256-thread workgroup owns a 16 x 16
//               block of entries and stages 256-token slabs of its 32 logit
//               columns in LDS.
//   k_sim_rank  one workgroup per row i: the squared cosine similarity
//               T2[i][j] = gram[i][j]^2 / (gram[i][i] gram[j][j]) (Eq. 7; Eq. 8
//               has the same value, its 1/N factors cancel), 0 when a column
//               is all zero, and the row's ranking: rank[i][q] is the q-th
//               most similar expert, ties to the lower index.  Entry j's place
//               is the number of entries that precede it, so the ranking is a
//               permutation without any sort.
#include "launch.h"

namespace occ {
namespace {

constexpr int kSimTile = 16;    // gram entries per side of a workgroup's block
constexpr int kSimSlab = 256;   // tokens staged per LDS slab

__global__ __launch_bounds__(kSimTile *kSimTile) void k_sim_gram(const float *__restrict__ H,
                                                                 int T, int Ne,
                                                                 double *__restrict__ gram) {
    __shared__ float si[kSimSlab][kSimTile];
    __shared__ float sj[kSimSlab][kSimTile];
    const int i0 = blockIdx.y * kSimTile, j0 = blockIdx.x * kSimTile;
    const int a = threadIdx.x / kSimTile, b = threadIdx.x % kSimTile;
    const int i = i0 + a, j = j0 + b;
    const bool own = i < Ne && j < Ne;
    double acc = own ? gram[static_cast<size_t>(i) * Ne + j] : 0.0;
    for (int t0 = 0; t0 < T; t0 += kSimSlab) {
        const int nt = min(kSimSlab, T - t0);
        __syncthreads();
        for (int q = threadIdx.x; q < nt * kSimTile; q += blockDim.x) {
            const int t = q / kSimTile, c = q % kSimTile;
            const float *row = H + static_cast<size_t>(t0 + t) * Ne;
            si[t][c] = i0 + c < Ne ? row[i0 + c] : 0.f;
            sj[t][c] = j0 + c < Ne ? row[j0 + c] : 0.f;
        }
        __syncthreads();
        for (int t = 0; t < nt; t++)
            acc = fma(static_cast<double>(si[t][a]), static_cast<double>(sj[t][b]), acc);
    }
    if (own) gram[static_cast<size_t>(i) * Ne + j] = acc;
}

__global__ __launch_bounds__(kMaxNe) void k_sim_rank(const double *__restrict__ gram, int Ne,
                                                     double *__restrict__ t2,
                                                     int32_t *__restrict__ rank) {
    __shared__ double s[kMaxNe];
    const int i = blockIdx.x, j = threadIdx.x;
    double v = 0.0;
    if (j < Ne) {
        const double gii = gram[static_cast<size_t>(i) * Ne + i];
        const double gjj = gram[static_cast<size_t>(j) * Ne + j];
        const double gij = gram[static_cast<size_t>(i) * Ne + j];
        const double den = gii * gjj;
        v = den > 0.0 ? (gij * gij) / den : 0.0;
        if (t2) t2[static_cast<size_t>(i) * Ne + j] = v;
        s[j] = v;
    }
    __syncthreads();
    if (j < Ne) {
        int pos = 0;
        for (int q = 0; q < Ne; q++) pos += (s[q] > v || (s[q] == v && q < j)) ? 1 : 0;
        rank[static_cast<size_t>(i) * Ne + pos] = j;
    }
}

}  // namespace

hipError_t launch_sim_gram(const float *H, int T, int Ne, double *gram, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int nb = ceil_div(Ne, kSimTile);
    k_sim_gram<<<dim3(nb, nb), kSimTile * kSimTile, 0, s>>>(H, T, Ne, gram);
    return hipGetLastError();
}

hipError_t launch_sim_rank(const double *gram, int Ne, double *t2, int32_t *rank, hipStream_t s) {
    k_sim_rank<<<Ne, kMaxNe, 0, s>>>(gram, Ne, t2, rank);
    return hipGetLastError();
}

}  // namespace occ
