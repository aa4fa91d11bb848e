// Grouped GEMMs of the backward pass on the bf16 matrix cores of gfx950
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation): the transposed sparse
// matrix multiplications that the Occult paper builds "for both forward and
// backward passes" (section 1; its appendix A.2 gives the forward ones).
//
// Every backward product has an operand whose contraction index is the
// strided one: the weights in the input gradients (dh = dy W_d contracts over
// W_d's rows) and both token-row operands in the weight gradients (dW = sum
// over an expert's rows).  Such "K-major" operands are loaded as they lie in
// memory -- each global row is one k, 256 contiguous columns of it are a
// 512-byte LDS row -- and gfx950's LDS transpose read (ds_read_b64_tr_b16)
// turns them into MFMA fragments: in each 16-lane group, lane 4a+b names the
// 8 bytes at row k0+a, columns c0+4b..c0+4b+3, and lane i receives the four
// values of column c0+i from rows k0..k0+3.  Two such reads give a lane its
// 8 consecutive k.  The 16-byte chunks of a K-major LDS row are XOR-swizzled
// by key(k) = 2 ((k mod 8) xor (4 * bit 3 of k)), which keeps each read's 16
// rows x 32 bytes on distinct bank windows (two 256-byte cycles, the
// minimum); "K-contiguous" operands use the forward kernels' layout.
//
// Tiles are up to 320 rows (dgrad; its experts' row blocks shared out evenly
// over ceil(rows / 320) tiles, as in the forward GEMMs) or 256 rows (wgrad)
// x 256 outputs per 512-thread workgroup (8 waves, each 128 columns of its
// wave row's 16-row blocks), K in 64-deep slices through two LDS buffers
// filled by direct global->LDS loads, as in the forward GEMMs.
//   k_bwd_dgrad  A = gathered K-contiguous rows, B = an expert's weights read
//                K-major (or, for the shared experts' dh, their W_d copied
//                transposed beforehand and read like A, which measured 2%
//                faster on that product family; for the routed experts the
//                copy of all their W_d would cost what it saves); routed row
//                tiles over expert segments.  Epilogues:
//                SwiGLU backward (dh -> dg, du and the routing-weight
//                gradient's per-tile partial sums) or the fp32 merge of EPD
//                rows into their SFD rows (first contributors store, the rest
//                add).
//   k_bwd_wgrad  A and B both K-major token rows of one expert; K = that
//                expert's rows (tail rows read a zero row); the fp32 tile is
//                stored into the expert's weight gradient.
#include <type_traits>

#include "launch.h"

namespace occ {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int NT = 512;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_M = NT / kWave / 2;            // 4
constexpr int WM = BM / WAVES_M, WN = BN / 2;      // wgrad: 64 x 128 per wave
constexpr int MI = WM / 16, NI = WN / 16;          // 4 x 8 MFMA blocks
constexpr int CHUNKS = BK / 8;                     // 16-byte chunks per K-contiguous row
constexpr int OP = BM * BK;                        // bf16 elements per operand tile
constexpr int STAGE = 2 * OP;
constexpr int NSTAGE = 2;
static_assert(BM == BN, "both operand tiles share one size");
static_assert(NSTAGE * STAGE * 2 <= 160 * 1024, "LDS");
// dgrad: up to kBwdRowTile gathered rows (K-contiguous) against a K-major
// weight tile of BN columns
constexpr int BMD = kBwdRowTile;
constexpr int MID = BMD / 16 / WAVES_M;            // 16-row blocks per wave row
constexpr int A_LDD = BMD / 64;                    // A loads per thread per slice
constexpr int OPA = BMD * BK;                      // bf16 elements of the A tile
constexpr int STAGED = OPA + OP;
static_assert(NSTAGE * STAGED * 2 + BMD * 4 <= 160 * 1024, "LDS");

constexpr int kBand = 8;  // row tiles per band of the dgrad tile order

// Block mi of wave row wm starts at this row: blocks are dealt to the wave
// rows in turn, so the two wave rows sharing a SIMD hold ceil(blocks / 2).
__device__ __forceinline__ int block_row(int wm, int mi) { return (wm + WAVES_M * mi) * 16; }

// A segment of len rows in n row tiles: ceil(len / 16) blocks dealt out as
// evenly as possible; tile j's first row and row count.
__device__ __forceinline__ void split_rows(int len, int n, int j, int &m0, int &rows) {
    const int B = (len + 15) >> 4, base = B / n, rem = B - base * n;
    m0 = 16 * (j * base + min(j, rem));
    rows = min(16 * (base + (j < rem ? 1 : 0)), len - m0);
}

// ---- K-contiguous operand tiles: rows of 64 k, chunk c at c ^ ((r >> 1) & 7)
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * BK + ((chunk ^ ((row >> 1) & (CHUNKS - 1))) << 3);
}

// ---- K-major operand tiles: rows of 256 columns for one k each
__device__ __forceinline__ int kkey(int k) { return ((k & 7) ^ ((k >> 1) & 4)) << 1; }
[[maybe_unused]] __device__ __forceinline__ int kmaj(int k, int col) {
    return k * BM + ((((col >> 3) ^ kkey(k))) << 3) + (col & 7);
}

// Direct global->LDS load (see the forward GEMMs): the LDS address goes to
// M0 through an input operand bound to that register, so the compiler writes
// M0 itself and knows it is live.
__device__ __forceinline__ void dma16(const void *g, uint32_t m0) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "{m0}"(m0)
                 : "memory");
}

__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// Addresses of K-major fragments with few live registers.  For a wave whose
// columns start at cw (a multiple of 16 whose chunk bits do not meet those of
// 16 f) and fragment f at cw + 16 f, kmaj(k, cw + 16 f + 4 b) equals
// P(k) + (X(k) ^ 16 f) with P(k) = k BM + 8 (b >> 1) + (4 b mod 8) and
// X(k) = 8 ((cw / 8) xor key(k)): the swizzle only touches chunk bits 1-3, the
// fragment index only chunk bits 1-3 above the wave's base, and b >> 1 is
// chunk bit 0.  A lane keeps P and X for its four rows (two per 32-deep step).
struct KmajAddr {
    int P[2][2], X[2][2];  // [step ks][row k1 or k1 + 4]
};
__device__ __forceinline__ void kmaj_addr(int cw, KmajAddr &o) {
    const int l = lane_id(), G = l >> 4, a = (l >> 2) & 3, b = l & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int k = 32 * ks + 8 * G + a + 4 * h;
            o.P[ks][h] = k * BM + 8 * (b >> 1) + ((4 * b) & 7);
            o.X[ks][h] = 8 * ((cw >> 3) ^ kkey(k));
        }
}
// MFMA fragment f (8 consecutive k of column cw + 16 f + (lane & 15), k chunk
// lane >> 4 of 32-deep step ks) from a K-major tile, by two transpose reads.
__device__ __forceinline__ bf16x8_t kmaj_frag(const uint16_t *tile, const KmajAddr &ad, int ks,
                                              int f) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(tile + ad.P[ks][0] + (ad.X[ks][0] ^ (16 * f))));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(tile + ad.P[ks][1] + (ad.X[ks][1] ^ (16 * f))));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}
// Marks X as changed each iteration, so that the compiler keeps four values
// per operand instead of hoisting one precomputed address per fragment out
// of the K loop (which spilled the weight-gradient kernel at 256 VGPRs).
__device__ __forceinline__ void launder(KmajAddr &ad) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int h = 0; h < 2; h++) asm volatile("" : "+v"(ad.X[ks][h]));
}

// MFMA fragment from a K-contiguous tile: row r, chunk (ks * 4 + lane >> 4).
__device__ __forceinline__ bf16x8_t rows_frag(const uint16_t *tile, int r, int ks) {
    return *reinterpret_cast<const bf16x8_t *>(tile + swz(r, ks * 4 + (lane_id() >> 4)));
}

// Workgroup -> (row tile, column tile), each XCD taking a contiguous range
// (workgroup b runs on XCD b % 8), column tiles fastest.
__device__ __forceinline__ bool map_tile(int m_tiles, int n_tiles, int &tm, int &tn) {
    const int total = m_tiles * n_tiles;
    const int per = (total + 7) >> 3;
    const int b = blockIdx.x, idx = b >> 3;
    if (idx >= per) return false;
    const int logical = (b & 7) * per + idx;
    if (logical >= total) return false;
    tm = logical / n_tiles;
    tn = logical - tm * n_tiles;
    return true;
}

// Issues the direct loads of one K-major operand slice: 64 k-rows of 256
// columns.  Wave w, load i moves slice rows 2 (8 i + w) and +1, lane l the
// physical chunk l & 31 of row l >> 5; row[i] points at column 0 of the
// slice's columns in the global row of slice row 2 (8 i + w) + (l >> 5).
__device__ __forceinline__ int kmajor_row(int i, int w) { return 2 * (8 * i + w) + (lane_id() >> 5); }

__device__ __forceinline__ void issue_kmajor(uint32_t lds, const uint16_t *const (&row)[4], int w) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int c = (l & 31) ^ kkey(kmajor_row(i, w));
        dma16(row[i] + 8 * c, __builtin_amdgcn_readfirstlane(lds + (8 * i + w) * 1024));
    }
}

// The MFMA is issued with the operands' roles swapped (it computes the
// transposed 16 x 16 block), so that lane l holds output row (l & 15) of
// the mi block and the 4 consecutive columns 4 (l >> 4) .. +3 of the ni
// block: the epilogues then move 8- and 16-byte row pieces.
// SWAP = false keeps the plain layout: lane l holds rows 4 (l >> 4) .. +3 of
// column (l & 15), so 16 lanes cover 64 contiguous bytes of a row -- the
// better shape for the fp32 atomic adds of the merge.
template <bool SWAP, int NV = MI, int M = MI>
__device__ __forceinline__ void mfma_tile(const bf16x8_t (&a)[M], const bf16x8_t (&b)[NI],
                                          f32x4 (&acc)[M][NI]) {
#pragma unroll
    for (int mi = 0; mi < NV; mi++)
#pragma unroll
        for (int ni = 0; ni < NI; ni++)
            acc[mi][ni] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[ni], a[mi], acc[mi][ni], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
}

typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- dgrad ----

// BKC: B1 holds the weights transposed (expert e's N x K block, row n
// K-contiguous), loaded and read like A instead of through transpose reads.
template <int EPI, bool BKC>
__global__ __launch_bounds__(NT, 2) void k_bwd_dgrad(BwdDgradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGED];
    __shared__ int s_dst[EPI == BWD_EPI_MERGE ? BMD : 1];
    int tm, tn;
    const int m_tiles = a.tile_off[a.Ne], n_tiles = (a.N + BN - 1) / BN;
    if (!map_tile(m_tiles, n_tiles, tm, tn)) return;
    const int p = tile_owner(a.tile_off, a.Ne, tm);
    if (a.phase != 2) {
        // bands of kBand row tiles, column tiles outermost inside a band, as
        // in the forward GEMMs
        const int r = a.tile_off[p + 1] - a.tile_off[p];
        const int local = (tm - a.tile_off[p]) * n_tiles + tn;
        const int band = local / (kBand * n_tiles), rb0 = band * kBand;
        const int rb = min(kBand, r - rb0), idx = local - band * kBand * n_tiles;
        tn = idx / rb;
        tm = a.tile_off[p] + rb0 + idx - tn * rb;
    }
    const int seg0 = a.seg_off[p], len = a.seg_off[p + 1] - seg0;
    const int nf = a.phase ? a.first_cnt[p] : 0;
    const int seg = a.phase == 2 ? seg0 + nf : seg0;
    int m0, rows;
    split_rows(a.phase == 1 ? nf : len - nf, a.tile_off[p + 1] - a.tile_off[p], tm - a.tile_off[p],
               m0, rows);
    const int e = a.tab.expert[p];
    const int n0 = tn * BN;

    const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
    if constexpr (EPI == BWD_EPI_MERGE) {
        // each row's destination, looked up once per row (not in series by
        // every lane in the epilogue); the K loop's barriers publish it.
        // With split, rows after the segment's first contributors go to
        // their own EPD rows of epd_out, marked by a negative entry ~erow.
        if (tid < rows) {
            const int pos = seg + m0 + tid;
            const int erow = a.a_rows ? a.a_rows[pos] : pos;
            s_dst[tid] = a.split && m0 + tid >= a.first_cnt[p] ? ~erow
                                                               : (a.dst_rows ? a.dst_rows[erow] : erow);
        }
    }
    const uint16_t *A = static_cast<const uint16_t *>(a.A);
    // A: K-contiguous gathered rows, thread rows r0 + 64 i, chunk slot tid & 7
    const uint16_t *a_src[A_LDD];
    {
        const int r0 = tid / CHUNKS;
#pragma unroll
        for (int i = 0; i < A_LDD; i++) {
            const int r = min(r0 + 64 * i, rows - 1);
            const int pos = seg + m0 + r;
            const int src = a.a_rows ? a.a_rows[pos] : pos;
            const int ch = (tid % CHUNKS) ^ (((r0 + 64 * i) >> 1) & (CHUNKS - 1));
            a_src[i] = A + static_cast<size_t>(src) * a.lda + a.a_col + 8 * ch;
        }
    }
    // B: rows k of expert e's weights, from B1 for k < ksplit, else B2
    const uint16_t *B1 = static_cast<const uint16_t *>(a.B1) + static_cast<size_t>(e) * a.ksplit * a.N;
    const uint16_t *B2 = a.B2 ? static_cast<const uint16_t *>(a.B2) +
                                    static_cast<size_t>(e) * (a.K - a.ksplit) * a.N
                              : nullptr;
    const int ncol = min(n0, a.N - BN);  // N >= BN; the last tile may overlap the previous one
    // BKC: rows ncol + r0 + 64 i of the transposed block, as the A loads
    const uint16_t *bt_src[BKC ? BN / 64 : 1];
    if constexpr (BKC) {
        const int r0 = tid / CHUNKS;
#pragma unroll
        for (int i = 0; i < BN / 64; i++) {
            const int ch = (tid % CHUNKS) ^ (((r0 + 64 * i) >> 1) & (CHUNKS - 1));
            bt_src[i] = static_cast<const uint16_t *>(a.B1) +
                        (static_cast<size_t>(e) * a.N + ncol + r0 + 64 * i) * a.K + 8 * ch;
        }
    }
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>(smem));
    const int nk = a.K / BK;

    const int wm = w >> 1, wn = w & 1;
    KmajAddr adB;
    kmaj_addr(wn * WN, adB);
    f32x4 acc[MID][NI];
#pragma unroll
    for (int mi = 0; mi < MID; mi++)
#pragma unroll
        for (int ni = 0; ni < NI; ni++) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the wave's blocks that hold rows, and its A loads (8-row groups 64 i +
    // 8 w) that do: the others are neither loaded nor multiplied (their LDS
    // rows keep stale values, which reach only rows that are never stored)
    const int nv = __builtin_amdgcn_readfirstlane(
        min(MID, max(0, (((rows + 15) >> 4) - wm + WAVES_M - 1) / WAVES_M)));
    const int na = __builtin_amdgcn_readfirstlane(min(A_LDD, max(0, (rows - 8 * w + 63) / 64)));
    auto k_loop = [&](auto nv_const) {
        constexpr int NV = decltype(nv_const)::value;
        for (int kt = 0; kt <= nk; kt++) {
            // slice kt is issued in iteration kt, consumed in iteration kt + 1
            if (kt > 0) {
                wait_all_loads();
                __syncthreads();
            }
            if constexpr (!BKC) launder(adB);
            if (kt < nk) {
                const uint32_t st = lds0 + static_cast<uint32_t>((kt % NSTAGE) * STAGED * 2);
                const int k0 = kt * BK;
#pragma unroll
                for (int i = 0; i < A_LDD; i++)
                    if (i < na)
                        dma16(a_src[i] + k0, __builtin_amdgcn_readfirstlane(st + (8 * i + w) * 1024));
                if constexpr (BKC) {
#pragma unroll
                    for (int i = 0; i < BN / 64; i++)
                        dma16(bt_src[i] + k0,
                              __builtin_amdgcn_readfirstlane(st + OPA * 2 + (8 * i + w) * 1024));
                } else {
                    const uint16_t *brow[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int kk = k0 + kmajor_row(i, w);
                        brow[i] = (kk < a.ksplit ? B1 + static_cast<size_t>(kk) * a.N
                                                 : B2 + static_cast<size_t>(kk - a.ksplit) * a.N) +
                                  ncol;
                    }
                    issue_kmajor(st + OPA * 2, brow, w);
                }
            }
            if (kt == 0 || NV == 0) continue;
            const uint16_t *sA = smem + ((kt - 1) % NSTAGE) * STAGED, *sB = sA + OPA;
#pragma unroll
            for (int ks = 0; ks < BK / 32; ks++) {
                bf16x8_t fa[MID], fb[NI];
#pragma unroll
                for (int mi = 0; mi < NV; mi++) fa[mi] = rows_frag(sA, block_row(wm, mi) + (l & 15), ks);
#pragma unroll
                for (int ni = 0; ni < NI; ni++)
                    fb[ni] = BKC ? rows_frag(sB, wn * WN + ni * 16 + (l & 15), ks)
                                 : kmaj_frag(sB, adB, ks, ni);
                mfma_tile<EPI == BWD_EPI_SWIGLU, NV, MID>(fa, fb, acc);
            }
        }
    };
    switch (nv) {
        case MID: k_loop(std::integral_constant<int, MID>{}); break;
        case MID - 1: k_loop(std::integral_constant<int, MID - 1>{}); break;
        case MID - 2: k_loop(std::integral_constant<int, MID - 2>{}); break;
        case MID - 3: k_loop(std::integral_constant<int, MID - 3>{}); break;
        case MID - 4: k_loop(std::integral_constant<int, MID - 4>{}); break;
        default: k_loop(std::integral_constant<int, 0>{}); break;
    }
    static_assert(MID == 5, "the switch above covers 0 .. MID blocks");

    // SWIGLU: acc[mi][ni][v] is row block_row(wm, mi) + (l & 15), column
    // (relative to the loaded columns) wn*WN + ni*16 + 4*(l >> 4) + v.
    // MERGE: row block_row(wm, mi) + 4*(l >> 4) + v, column wn*WN + ni*16 + (l & 15).
    const int cloc = wn * WN + 4 * (l >> 4);
    if constexpr (EPI == BWD_EPI_SWIGLU) {
        // dh -> dg, du (bf16) and this tile half's share of dw = <dh, a>
        const uint16_t *gu = static_cast<const uint16_t *>(a.gu);
        uint16_t *out = static_cast<uint16_t *>(a.out);
        // The pre-activations of block mi + 1 are loaded before block mi's
        // results are stored: a load placed after those stores would wait
        // for them (the compiler cannot tell the buffers apart), leaving one
        // load latency per block in series.  The routing weight comes with them.
        auto row_pos = [&](int mi) { return seg + m0 + min(block_row(wm, mi) + (l & 15), rows - 1); };
        auto load_gu = [&](int mi, u16x4(&g4)[NI], u16x4(&u4)[NI], float &wr) {
            wr = a.row_w ? a.row_w[row_pos(mi)] : 1.f;
            const uint16_t *gr = gu + static_cast<size_t>(row_pos(mi)) * a.gu_ld + a.gu_col;
#pragma unroll
            for (int ni = 0; ni < NI; ni++) {
                const int f = ncol + cloc + ni * 16;
                g4[ni] = *reinterpret_cast<const u16x4 *>(gr + f);
                u4[ni] = *reinterpret_cast<const u16x4 *>(gr + a.gu_uoff + f);
            }
        };
        u16x4 g4s[NI], u4s[NI];
        float wr;
        load_gu(0, g4s, u4s, wr);
#pragma unroll
        for (int mi = 0; mi < MID; mi++) {
            const int r = block_row(wm, mi) + (l & 15);
            const bool ok = r < rows;
            const int pos = row_pos(mi);
            uint16_t *orow = out + static_cast<size_t>(pos) * a.out_ld + a.out_col;
            u16x4 g4n[NI], u4n[NI];
            float wrn = 1.f;
            if (mi + 1 < MID) load_gu(mi + 1, g4n, u4n, wrn);
            float part = 0.f;
#pragma unroll
            for (int ni = 0; ni < NI; ni++) {
                const int f = ncol + cloc + ni * 16;  // 4 consecutive features f..f+3
                if (f < n0) continue;  // overlapped columns belong to the previous tile
                const u16x4 g4 = g4s[ni], u4 = u4s[ni];
                u16x4 dg4, du4;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const float g = bf16_bits_to_f32(g4[v]), u = bf16_bits_to_f32(u4[v]);
                    // hardware reciprocal: dg and du are rounded to bf16
                    const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-g));
                    const float dh = acc[mi][ni][v];
                    part += dh * (g * sg * u);
                    const float da = wr * dh;
                    dg4[v] = f32_to_bf16_bits(da * u * sg * (1.f + g * (1.f - sg)));
                    du4[v] = f32_to_bf16_bits(da * g * sg);
                }
                if (ok) {
                    *reinterpret_cast<u16x4 *>(orow + f) = dg4;
                    *reinterpret_cast<u16x4 *>(orow + a.out_uoff + f) = du4;
                }
            }
            // the 4 lanes holding this row (l >> 4 = 0..3) sum, one write per wave half
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            if (a.dw_part && ok && l < 16)
                a.dw_part[static_cast<size_t>(pos) * a.dw_stride + 2 * tn + wn] = part;
            if (mi + 1 < MID) {
#pragma unroll
                for (int ni = 0; ni < NI; ni++) {
                    g4s[ni] = g4n[ni];
                    u4s[ni] = u4n[ni];
                }
                wr = wrn;
            }
        }
    } else {
        // merge into SFD rows (or dense rows): store, or add
        float *out = a.merge_out;
#pragma unroll
        for (int mi = 0; mi < MID; mi++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int r = block_row(wm, mi) + 4 * (l >> 4) + v;
                if (r >= rows) continue;
                const int d = s_dst[r];
                float *drow = d < 0 ? a.epd_out + static_cast<size_t>(~d) * a.N
                                    : out + static_cast<size_t>(d) * a.N;
#pragma unroll
                for (int ni = 0; ni < NI; ni++) {
                    const int c = ncol + wn * WN + ni * 16 + (l & 15);
                    if (c < n0) continue;
                    if (a.merge_store) drow[c] = acc[mi][ni][v];
                    else unsafeAtomicAdd(drow + c, acc[mi][ni][v]);
                }
            }
    }
}

// ---------------------------------------------------------------- wgrad ----

// Window of gathered row indices kept in LDS (with the two K slices, all
// 160 KB of it).
constexpr int kRowsLds = 8192;
static_assert(NSTAGE * STAGE * 2 + kRowsLds * 4 <= 160 * 1024, "LDS");

__global__ __launch_bounds__(NT, 2) void k_bwd_wgrad(BwdWgradArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGE];
    __shared__ int s_rows[kRowsLds];
    const int m_tiles = (a.M + BM - 1) / BM, n_tiles = (a.N + BN - 1) / BN;
    const int parts = a.k_parts > 1 ? a.k_parts : 1;
    int tq, tn;
    if (!map_tile(parts * a.n_groups * m_tiles, n_tiles, tq, tn)) return;
    // chunk of K (rows) this tile sums: the chunks are outermost, so the
    // tiles an XCD runs together share their rows' operand strips
    const int part = tq / (a.n_groups * m_tiles);
    tq -= part * a.n_groups * m_tiles;
    const int grp = tq / m_tiles, tm = tq - grp * m_tiles;
    const int seg0 = a.seg_off ? a.seg_off[grp] : 0;
    const int len_all = a.seg_off ? a.seg_off[grp + 1] - seg0 : a.rows;
    const int k_begin = parts > 1 ? part * a.k_chunk : 0;
    const int seg = seg0 + k_begin;
    const int len = parts > 1 ? max(0, min(len_all - k_begin, a.k_chunk)) : len_all;
    const int e = a.seg_off ? a.tab.expert[grp] : grp;
    // M, N >= 256: the last tile of a dimension may overlap the previous one
    const int m0 = tm * BM, n0 = tn * BN;
    const int mload = min(m0, a.M - BM), nload = min(n0, a.N - BN);

    const int w = threadIdx.x / kWave, l = lane_id();
    const uint16_t *A = static_cast<const uint16_t *>(a.A);
    const uint16_t *B = static_cast<const uint16_t *>(a.B);
    const uint16_t *Z = static_cast<const uint16_t *>(a.zero_row);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>(smem));
    const int nk = (len + BK - 1) / BK;
    // The K dimension is the expert's rows; at most one operand is gathered
    // (gidx).  Its index list comes into LDS in windows of kRowsLds rows: one
    // window holds a segment of up to that length, and a longer one's next
    // window is loaded at the top of the iteration that first needs it,
    // after the barrier, when no direct load is in flight.  An index read
    // from global memory inside the loop would instead sit behind the slice
    // in flight (its wait is a wait for every earlier load): on the
    // Qwen-shaped batch, whose experts hold ~4400 rows each, the weight
    // gradients took 13-16% longer with the indices of segments over 4096
    // rows read that way.  K-rows past the segment read the zero row.
    const int32_t *gidx = a.a_rows ? a.a_rows : a.b_rows;
    auto stage = [&](int base) {  // segment rows [base, base + kRowsLds)
        const int n = min(len - base, kRowsLds);
        for (int i = threadIdx.x; i < n; i += NT) s_rows[i] = gidx[seg + base + i];
        __syncthreads();
    };
    static_assert(kRowsLds % BK == 0, "a slice never straddles two index windows");
    const int acol = a.a_col0 + grp * a.a_col_grp + mload;
    const int bcol = a.b_col0 + grp * a.b_col_grp + nload;
    const bool ga = a.a_rows != nullptr;

    const int wm = w >> 1, wn = w & 1;
    KmajAddr adA, adB;
    kmaj_addr(wm * WM, adA);
    kmaj_addr(wn * WN, adB);
    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; mi++)
#pragma unroll
        for (int ni = 0; ni < NI; ni++) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    // One loop with gathered rows and one without, so that the pointer
    // arithmetic of each is straight-line code.
    auto k_loop = [&](auto gather_const) {
        constexpr bool GATHER = decltype(gather_const)::value;
        int src[4];  // gathered source rows of this thread's four k-rows
        auto slice_rows = [&](int kt) {
            if constexpr (GATHER) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    // clamped into the window; len >= 1 whenever a slice is issued
                    const int kc = min(kt * BK + kmajor_row(i, w), len - 1);
                    src[i] = s_rows[kc % kRowsLds];
                }
            }
        };
        if (GATHER && nk > 0) stage(0);
        for (int kt = 0; kt <= nk; kt++) {
            // slice kt is issued in iteration kt, consumed in iteration kt + 1
            if (kt > 0) {
                wait_all_loads();
                __syncthreads();
            }
            if (GATHER && kt > 0 && kt < nk && (kt * BK) % kRowsLds == 0) stage(kt * BK);
            launder(adA);
            launder(adB);
            if (kt < nk) {
                slice_rows(kt);
                const uint32_t st = lds0 + static_cast<uint32_t>((kt % NSTAGE) * STAGE * 2);
                const uint16_t *arow[4], *brow[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int kk = kt * BK + kmajor_row(i, w);
                    const int ra = GATHER && ga ? src[i] : seg + kk;
                    const int rb = GATHER && !ga ? src[i] : seg + kk;
                    arow[i] = kk < len ? A + static_cast<size_t>(ra) * a.lda + acol : Z;
                    brow[i] = kk < len ? B + static_cast<size_t>(rb) * a.ldb + bcol : Z;
                }
                issue_kmajor(st, arow, w);
                issue_kmajor(st + OP * 2, brow, w);
            }
            if (kt == 0) continue;
            const uint16_t *sA = smem + ((kt - 1) % NSTAGE) * STAGE, *sB = sA + OP;
#pragma unroll
            for (int ks = 0; ks < BK / 32; ks++) {
                bf16x8_t fa[MI], fb[NI];
#pragma unroll
                for (int mi = 0; mi < MI; mi++) fa[mi] = kmaj_frag(sA, adA, ks, mi);
#pragma unroll
                for (int ni = 0; ni < NI; ni++) fb[ni] = kmaj_frag(sB, adB, ks, ni);
                mfma_tile<true>(fa, fb, acc);
            }
        }
    };
    if (gidx) k_loop(std::true_type{});
    else k_loop(std::false_type{});

    // C[e] rows m < msplit -> C1, the rest -> C2 (gate and up halves), or
    // with a split K this chunk's partial tile; each lane stores 4
    // consecutive columns of a row
    float *P = parts > 1 ? a.part + static_cast<size_t>(part) * a.n_groups * a.M * a.N : nullptr;
#pragma unroll
    for (int mi = 0; mi < MI; mi++) {
        const int m = mload + wm * WM + mi * 16 + (l & 15);
        if (m < m0) continue;
        float *row = P ? P + (static_cast<size_t>(grp) * a.M + m) * a.N
                       : (m < a.msplit ? a.C1 + (static_cast<size_t>(e) * a.msplit + m) * a.N
                                       : a.C2 + (static_cast<size_t>(e) * (a.M - a.msplit) +
                                                 (m - a.msplit)) * a.N);
#pragma unroll
        for (int ni = 0; ni < NI; ni++) {
            const int n = nload + wn * WN + ni * 16 + 4 * (l >> 4);
            if (n >= n0) *reinterpret_cast<f32x4 *>(row + n) = acc[mi][ni];
        }
    }
}

// The split weight gradients' partial tiles, added in chunk order: 4
// consecutive columns per thread, written to C1 / C2 as the tiles would be.
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float *__restrict__ part, int parts,
                                                      int n_groups, int M, int N, int msplit,
                                                      float *__restrict__ C1,
                                                      float *__restrict__ C2) {
    const size_t total = static_cast<size_t>(n_groups) * M * N / 4;
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const size_t plane = static_cast<size_t>(n_groups) * M * N;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(part) + i;
    f32x4 acc = __builtin_nontemporal_load(src);
    for (int p = 1; p < parts; p++) acc += __builtin_nontemporal_load(src + p * plane / 4);
    const size_t o = 4 * i, n = o % N, gm = o / N;
    const int grp = static_cast<int>(gm / M), m = static_cast<int>(gm % M);
    float *row = m < msplit ? C1 + (static_cast<size_t>(grp) * msplit + m) * N
                            : C2 + (static_cast<size_t>(grp) * (M - msplit) + (m - msplit)) * N;
    *reinterpret_cast<f32x4 *>(row + n) = acc;
}

unsigned grid_for(size_t tiles) { return static_cast<unsigned>(8 * ((tiles + 7) / 8)); }

}  // namespace

// The split is chosen by an estimate in units of one 64-row K slice of one
// tile: rounds of 256 CUs x slices per chunk, plus the ordered reduction's
// traffic (each chunk's partials read once, the result written once, about
// 14 MB per slice time at HBM speed), over 1..16 chunks of at least 1024
// rows.  A fixed count of CUs keeps the choice (and so the summation order
// and the workspace size) a function of the shape alone.  On the Qwen-shaped
// layer's shared expert it picks 13 chunks for dW_down (176 tiles: 69% of
// the CUs for the whole launch otherwise) and 8 for [dW_g; dW_u] (352
// tiles, 1.4 rounds).
int wgrad_k_parts(int n_groups, int M, int N, int rows) {
    const long tiles = static_cast<long>(n_groups) * ceil_div(M, BM) * ceil_div(N, BN);
    const long slices = (rows + BK - 1) / BK;
    const double out_mb = static_cast<double>(n_groups) * M * N * 4 / 1e6;
    if (tiles <= 0 || slices <= 0) return 1;
    double best = 0;
    int best_s = 1;
    for (int s = 1; s <= 16; s++) {
        const long chunk = (slices + s - 1) / s;
        if (s > 1 && chunk < 16) break;
        const long rounds = (tiles * s + 255) / 256;
        const double t = static_cast<double>(rounds) * chunk + (s > 1 ? (s + 1) * out_mb / 14.0 : 0);
        if (s == 1 || t < best) {
            best = t;
            best_s = s;
        }
    }
    return best_s;
}

int wgrad_k_chunk(int rows, int parts) {
    const int slices = (rows + BK - 1) / BK;
    return ((slices + parts - 1) / parts) * BK;
}

hipError_t launch_bwd_dgrad(const BwdDgradArgs &a, size_t max_m_tiles, hipStream_t s) {
    const unsigned grid = grid_for(max_m_tiles * ((a.N + BN - 1) / BN));
    if (grid == 0) return hipSuccess;
    if (a.b_kcontig && (a.epilogue != BWD_EPI_SWIGLU || a.B2 || a.ksplit != a.K))
        return hipErrorInvalidValue;
    if (a.epilogue == BWD_EPI_SWIGLU) {
        if (a.b_kcontig) k_bwd_dgrad<BWD_EPI_SWIGLU, true><<<grid, NT, 0, s>>>(a);
        else k_bwd_dgrad<BWD_EPI_SWIGLU, false><<<grid, NT, 0, s>>>(a);
    } else {
        k_bwd_dgrad<BWD_EPI_MERGE, false><<<grid, NT, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const BwdWgradArgs &a, hipStream_t s) {
    if (a.a_rows && a.b_rows) return hipErrorInvalidValue;
    const int parts = a.k_parts > 1 && !a.seg_off && a.part ? a.k_parts : 1;
    BwdWgradArgs b = a;
    b.k_parts = parts;
    const unsigned grid = grid_for(static_cast<size_t>(parts) * a.n_groups *
                                   ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
    if (grid == 0) return hipSuccess;
    k_bwd_wgrad<<<grid, NT, 0, s>>>(b);
    if (parts > 1) {
        const size_t total = static_cast<size_t>(a.n_groups) * a.M * a.N / 4;
        k_wgrad_reduce<<<ceil_div(total, 256), 256, 0, s>>>(a.part, parts, a.n_groups, a.M, a.N,
                                                           a.msplit, a.C1, a.C2);
    }
    return hipGetLastError();
}

}  // namespace occ
