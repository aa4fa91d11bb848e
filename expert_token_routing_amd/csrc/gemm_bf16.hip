// Grouped expert GEMMs on the bf16 matrix cores of gfx950 (MFMA
// v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// These are the paper's sparse matrix multiplications (appendix A.2):
//   up    SMM scattering SFD -> EPD (Algorithm 6) fused with the SwiGLU
//         activation and the weight modulation (Algorithm 7): for each
//         expert, its EPD rows gather their SFD rows (the condensed BRIM_1,
//         section 3.1 footnote 2) and produce
//           epd[r, f] = bf16( w_r * silu(a_r . Wg[f]) * (a_r . Wu[f]) );
//         the weight scales the hidden state after the activation, which is
//         exact because the down-projection is linear;
//   down  SMM merging EPD -> SFD (Algorithm 8): each EPD row's product with
//         W_down is added in fp32 to its SFD row (several experts of one group
//         share that row -- the intra-group pre-aggregation of section 3.1).
//
// Tiling (the grouped build; the dense build's four-wave pipelined loop is
// described where it is defined): a 512-thread workgroup (8 waves, one
// workgroup per CU, two waves per SIMD) computes a tile of up to 320 rows x
// 256 MFMA output columns.  The
// rows come in 16-row blocks dealt to the four wave rows in turn, and each
// wave holds 128 columns of its blocks.  In the up GEMM the 256 columns
// are 128 gate and 128 up rows of the same output features, so the SwiGLU
// epilogue has both operands in registers.  K is consumed in 64-deep slices
// (each row's slice is one 128-byte line) through two 72 KB LDS buffers
// filled by direct global->LDS loads: slice kt+1 is issued right after the
// barrier that opens slice kt and lands during its MFMA work.  Measured on
// the OLMoE-shaped layer, this beats 32-deep slices in a 3- to 5-deep ring
// by 9% in the up-projection (a deeper ring of 64-byte slices did not help:
// the load path, not its depth, is the limit).  The 16-byte chunks of an LDS
// row are XOR-swizzled by row so that fragment reads of 16 consecutive rows
// hit distinct banks.  The up GEMM's bf16 output tile is staged through LDS
// and written as whole 16-byte row chunks.
//
// Scheduling: the BRIM scan gives each expert ceil(rows / BM) row tiles
// (tile_off), so every tile reads one expert's weights, and the expert's
// row blocks are shared out evenly among them.  With 320-row capacity an
// expert of 1025-1067 rows is four tiles of 256-272 rows instead of four
// full 256-row tiles and a fifth of at most 43 rows that costs as much as a
// full one (the tile's time is set by its weight loads).  Measured on the
// OLMoE-shaped layer (287 -> 255 row tiles): -3% in both projections; the
// balance is imperfect because a 17-block tile gives one SIMD pair 9 blocks.
// A wave skips the MFMAs and the direct loads of blocks that hold no rows.
// Workgroup b runs on
// XCD b % 8; tiles are renumbered so that each XCD takes a contiguous range
// of an expert-major tile order (inside an expert, bands of 8 row tiles
// walked column by column, except in the atomic merge phase; a dense product
// the same way): the workgroups sharing an expert's weights and a row tile's
// activations share one L2.
// 256-row tiles halve the weight bytes fetched per flop against 128-row
// tiles (measured: 1.6 vs 2.5 GB beyond L2 per up-projection launch on the
// OLMoE-shaped layer).  The 128-row build (the decode regime) shares all of
// this with four two-block wave rows.
#include <algorithm>

#include "launch.h"

namespace occ {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef f32x4 f32x4_t;
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

#ifndef OCC_GEMM_BK
#define OCC_GEMM_BK 64
#endif
#ifndef OCC_GEMM_WG_PER_CU
#define OCC_GEMM_WG_PER_CU 1
#endif
#ifndef OCC_XCD_MAP
#define OCC_XCD_MAP 1
#endif
// One source, three builds: this file builds the kGemmBmBf16-row kernels;
// gemm_bf16_m128.hip includes it with 128-row tiles, and gemm_bf16_dense.hip
// with 256-row tiles, four waves and the pipelined K loop (OCC_GEMM_PIPE),
// each with suffixed kernel and launcher names.
#ifndef OCC_GEMM_TILE_M
#define OCC_GEMM_TILE_M kGemmBmBf16
#endif
#ifndef OCC_GEMM_SUFFIX
#define OCC_GEMM_SUFFIX
#endif
#define OCC_CAT2(a, b) a##b
#define OCC_CAT(a, b) OCC_CAT2(a, b)
#define OCC_NAMED(name) OCC_CAT(name, OCC_GEMM_SUFFIX)
constexpr int BM = OCC_GEMM_TILE_M;  // rows (tokens) per tile
constexpr int BN = 256;           // MFMA columns per tile
constexpr int BK = OCC_GEMM_BK;   // K slice
#ifndef OCC_GEMM_NT
#define OCC_GEMM_NT 512
#endif
constexpr int NT = OCC_GEMM_NT;          // threads: (NT/128) x 2 waves
constexpr int WAVES_M = NT / kWave / 2;
constexpr int WM = BM / WAVES_M, WN = BN / 2;  // wave sub-tile
constexpr int MI = WM / 16, NI = WN / 16;
constexpr int CHUNKS = BK / 8;           // 16-byte chunks per LDS row
constexpr int ROWS_PER_PASS = NT / CHUNKS;  // rows one pass of the workgroup moves
constexpr int A_LD = BM / ROWS_PER_PASS;
constexpr int B_LD = BN / ROWS_PER_PASS;
constexpr int STAGE = (BM + BN) * BK;    // bf16 elements per LDS buffer
#ifndef OCC_GEMM_NSTAGE
#define OCC_GEMM_NSTAGE 2
#endif
constexpr int NSTAGE = OCC_GEMM_NSTAGE;  // LDS ring filled by direct global->LDS loads
static_assert(NSTAGE >= 2 && NSTAGE <= 5, "ring depth");
static_assert(BK == 32 || BK == 64, "a wave load moves 1 KB: 16 rows of 64 bytes or 8 of 128");
constexpr int OUT_PITCH = 128 + 8;       // up epilogue staging row (elements)
static_assert(NSTAGE * STAGE * 2 * OCC_GEMM_WG_PER_CU <= 160 * 1024, "LDS");
static_assert(BM * OUT_PITCH <= NSTAGE * STAGE, "epilogue staging fits in the K buffers");

// Chunk c of row r sits at chunk slot c ^ ((r >> 1) mod chunks-per-row).  A
// 16-byte fragment read covers 16 consecutive rows at one logical chunk;
// measured on gfx950 (one workgroup timing ds_read_b128 patterns), this key
// reads such a fragment without bank conflicts for both 64- and 128-byte
// rows, while r mod 4 or (r >> 2) mod 4 on 64-byte rows cost 35-45% more
// LDS time.
__device__ __forceinline__ int swz_key(int row) { return row >> 1; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (swz_key(row) & (BK / 8 - 1))) << 3); }

// The K chunk of tile row `row` that this thread fetches.  Thread t moves
// rows (t / CHUNKS) + i * ROWS_PER_PASS, i.e. wave w owns 16-row groups; the
// direct loads write LDS slot t % CHUNKS of the row, so the thread fetches
// the logical chunk that the swizzle puts in that slot.
__device__ __forceinline__ int fetch_chunk(int row) {
    const int c = threadIdx.x % CHUNKS;
    return c ^ (swz_key(row) & (CHUNKS - 1));
}

// Workgroup -> (row tile, column tile).  Returns false when there is no tile.
__device__ __forceinline__ bool map_tile(int m_tiles, int n_tiles, int &tm, int &tn) {
    const int total = m_tiles * n_tiles;
    const int per = (total + 7) >> 3;
    const int b = blockIdx.x, idx = b >> 3;
    if (idx >= per) return false;
#if OCC_XCD_MAP
    const int logical = (b & 7) * per + idx;
#else
    const int logical = b;
#endif
    if (logical >= total) return false;
    tm = logical / n_tiles;
    tn = logical - tm * n_tiles;
    return true;
}

// Order of the tiles of one expert (or of a dense product): an r x c grid of
// row x column tiles is walked in bands of OCC_GEMM_BAND row tiles, and
// inside a band column by column, so the 32 workgroups an XCD runs at a time
// hold 8 row tiles x 4 column tiles of one band (448 KB of distinct operand
// bytes per 64-deep K slice at 320 x 256 tiles) rather than one row tile x 32
// column tiles (the row-major order of a dense product: 1.06 MB) or, for an
// expert of 14 row tiles walked column by column, 14 x 2-3 (650 KB).
// Measured (bands of 1, 2, 4, 8 and unbounded): 8 is best for the
// up-projection, though by little -- the Qwen-shaped layer's step -1.5%, the
// OLMoE- and DeepSeek-shaped ones -0.5% against unbounded bands -- so L2
// reuse is not what bounds these GEMMs.  The routed down-projection (8
// column tiles of d = 2048) takes bands of 16, which for these batches'
// experts of at most 14 row tiles is column by column over the whole expert:
// against 8, 2% faster on the Qwen-shaped and pruned OLMoE batches, even on
// the others (bands of 2 and 4 slower); dense launches keep 8 (the
// Qwen-shaped shared down-projection measured 8% slower with 16).  Local
// index `local` -> (row tile lm, column tn).
#ifndef OCC_GEMM_BAND
#define OCC_GEMM_BAND 8
#endif
constexpr int kBandDown = 16;
__device__ __forceinline__ void band_order(int local, int r, int c, int &lm, int &tn, int B = OCC_GEMM_BAND) {
    const int band = local / (B * c);
    const int rb0 = band * B;
    const int rb = min(B, r - rb0);
    const int idx = local - band * B * c;
    tn = idx / rb;
    lm = rb0 + idx - tn * rb;
}

struct Tile {
    int e;     // expert
    int seg;   // first row of the expert's segment
    int m0;    // first row of the tile inside the segment
    int rows;  // valid rows in the tile (at most BM)
    int n0;    // first column (output feature) of the tile
    int first; // phase 3: the tile's first `first` rows are first contributors
};

// A segment of len rows in n = ceil(len / BM) row tiles: its ceil(len / 16)
// MFMA row blocks are dealt out as evenly as possible (the first B mod n
// tiles take one more), so an expert of 1030 rows is four tiles of 272, 256,
// 256 and 246 rows rather than four full tiles and one of 6 rows.  Tile j's
// first row and row count.
__device__ __forceinline__ void split_rows(int len, int n, int j, int &m0, int &rows) {
    const int B = (len + 15) >> 4, base = B / n, rem = B - base * n;
    m0 = 16 * (j * base + min(j, rem));
    rows = min(16 * (base + (j < rem ? 1 : 0)), len - m0);
}

// Routed tiles walk expert segments [seg_off[p], seg_off[p+1]) -- all rows
// (phases 0 and 3), the first first_cnt[p] rows (phase 1) or the rest (phase 2) --
// with the phase's row-tile schedule tile_off; shared tiles (seg_off NULL)
// walk M rows.
__device__ __forceinline__ bool tile_of(const int32_t *seg_off, const int32_t *tile_off, int M,
                                        int m_tiles_dense, int Ne, const PlaceTab &tab,
                                        int n_tiles, int n_step, Tile &t,
                                        const int32_t *first_cnt = nullptr, int phase = 0,
                                        int band = OCC_GEMM_BAND) {  // routed launches
    int tm, tn;
    if (seg_off) {
        const int m_tiles = tile_off[Ne];
        if (!map_tile(m_tiles, n_tiles, tm, tn)) return false;
        const int p = tile_owner(tile_off, Ne, tm);
        if (phase != 2) {
            // Bands of row tiles, column tiles outermost inside a band: the
            // workgroups that run together on an XCD then share fewer weight
            // column tiles (the larger share of the L2 misses).  Column tiles
            // outermost was measured on the OLMoE-shaped layer at -4% in the
            // up-projection and in the first merge phase against row order;
            // the atomic phase is faster in row order.
            int lm;
            band_order((tm - tile_off[p]) * n_tiles + tn, tile_off[p + 1] - tile_off[p], n_tiles,
                       lm, tn, band);
            tm = tile_off[p] + lm;
        }
        const int seg0 = seg_off[p], len = seg_off[p + 1] - seg0;
        const int nf = phase == 1 || phase == 2 ? first_cnt[p] : 0;
        t.e = tab.expert[p];
        t.seg = phase == 2 ? seg0 + nf : seg0;
        split_rows(phase == 1 ? nf : len - nf, tile_off[p + 1] - tile_off[p], tm - tile_off[p],
                   t.m0, t.rows);
        t.first = phase == 3 ? first_cnt[p] - t.m0 : 0;
    } else {
        const int m_tiles = m_tiles_dense;
        if (!map_tile(m_tiles, n_tiles, tm, tn)) return false;
        band_order(tm * n_tiles + tn, m_tiles, n_tiles, tm, tn);
        t.e = 0;
        t.seg = 0;
        split_rows(M, m_tiles, tm, t.m0, t.rows);
        t.first = 0;
    }
    t.n0 = tn * n_step;
    return true;
}

// The tile's 16-row blocks are dealt to the wave rows in turn: wave row wm
// owns blocks wm, wm + WAVES_M, ...; its mi-th block starts at this row.
// The two wave rows that share a SIMD (wm and wm + 2) then hold
// ceil(blocks / 2) blocks between them whatever the tile's height.
__device__ __forceinline__ int block_row(int wm, int mi) { return (wm + WAVES_M * mi) * 16; }

// NV: the wave's blocks that hold rows (the others are not multiplied).
// SWAP issues the MFMA with the operands' roles exchanged, which yields the
// transposed 16 x 16 block: lane l then holds row (l & 15) and the four
// consecutive columns 4 (l >> 4) .. + 3 (the plain layout gives a lane four
// rows of one column).
template <int NV, bool SWAP>
__device__ __forceinline__ void mma_slice(const uint16_t *sA, const uint16_t *sB, int wm,
                                          const int (&brow)[NI], f32x4_t (&acc)[MI][NI]) {
    if constexpr (NV > 0) {
        const int l = lane_id();
#pragma unroll
        for (int ks = 0; ks < BK / 32; ks++) {
            const int chunk = ks * 4 + (l >> 4);
            bf16x8_t a[NV], b[NI];
#pragma unroll
            for (int mi = 0; mi < NV; mi++)
                a[mi] = *reinterpret_cast<const bf16x8_t *>(sA + swz(block_row(wm, mi) + (l & 15), chunk));
#pragma unroll
            for (int ni = 0; ni < NI; ni++)
                b[ni] = *reinterpret_cast<const bf16x8_t *>(sB + swz(brow[ni], chunk));
            // The matrix-core burst runs at raised wave priority: of the two
            // waves sharing a SIMD, the one whose MFMAs are ready issues
            // first and the other's fragment reads fall in between
            // (up-projection -2% on the OLMoE-shaped batch).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int mi = 0; mi < NV; mi++)
#pragma unroll
                for (int ni = 0; ni < NI; ni++)
                    acc[mi][ni] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[ni], a[mi], acc[mi][ni], 0, 0, 0)
                                       : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        }
    }
}

// Direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l writes LDS bytes [m0 + 16 l, m0 + 16 l + 16).  m0 must be
// wave-uniform.  Issued as inline assembly because the compiler's builtin
// does not model the LDS write; completion is tracked with vmcnt below.  The
// LDS address is an input operand bound to M0 ("{m0}"), so the compiler
// itself writes M0 before the instruction and knows the register is live
// (M0 is reserved and may not be named as a clobber); the s_nop is the wait
// state between that write and the load.
__device__ __forceinline__ void dma16(const void *g, uint32_t m0) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "{m0}"(m0)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait until at most n (wave-uniform, 0 <= n <= N) loads are in flight; the
// count is an immediate of the instruction, hence the chain.
template <int N>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
    if constexpr (N == 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= N) wait_vmcnt<N>();
        else wait_vmcnt_le<N - 1>(n);
    }
}

#ifndef OCC_GEMM_PIPE
#define OCC_GEMM_PIPE 0
#endif

// Where a thread's direct loads read: its A rows (the tile's rows, gathered)
// and its B rows (weight rows), at the thread's fetch chunk.  a_at(i, k0) is
// load slot i's A address at K offset k0, b_at(i, bo) slot i's B address at
// B offset bo.
struct PtrSrc {  // one 64-bit address per slot
    const uint16_t *a[A_LD], *b[B_LD];
    __device__ const uint16_t *a_at(int i, int k0) const { return a[i] + k0; }
    __device__ const uint16_t *b_at(int i, size_t bo) const { return b[i] + bo; }
};
// K loop shared by both GEMMs; src gives the direct loads' addresses.  A ring of NSTAGE LDS buffers is filled
// by direct loads: slice kt+NSTAGE-1 is issued right after the barrier that
// opens slice kt, so each load has NSTAGE-1 slices of MFMA work to land,
// and the barrier also certifies that every wave has finished reading the
// buffer it overwrites (slice kt-1's).  B is laid out as blocks of ksp-wide
// K ranges, blk elements apart (the shared experts' down weights); one block
// (ksp = K) is the plain case.
// The wave issues only its first na A loads per slice (the 8-row groups
// that hold rows; the LDS rows it skips keep stale values, which reach only
// output rows that are never stored) and multiplies its first NV blocks.
// pre() runs once the first slices are issued: per-row tables the epilogue
// needs are loaded there, their latency hidden under those slices' (the
// loop's first barrier publishes what it writes to LDS).
#if !OCC_GEMM_PIPE
template <int NV, bool SWAP, class Src, class Pre>
__device__ __forceinline__ void k_loop(const Src &src, int K, int ksp, size_t blk, uint16_t *smem,
                                       int wm, const int (&brow)[NI], f32x4_t (&acc)[MI][NI], int na,
                                       Pre &pre) {
    constexpr int LOADS = A_LD + B_LD;
    const int per_slice = na + B_LD;  // loads the wave issues per slice
    const int nk = K / BK;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>(smem));
    auto issue = [&](int kt) {
        const int k0 = kt * BK;
        const size_t bo = ksp == K ? static_cast<size_t>(k0)
                                   : static_cast<size_t>(k0 / ksp) * blk + static_cast<size_t>(k0 % ksp);
        const uint32_t st = lds0 + static_cast<uint32_t>((kt % NSTAGE) * STAGE * 2);
#pragma unroll
        for (int i = 0; i < A_LD; i++)
            if (i < na)
                dma16(src.a_at(i, k0), __builtin_amdgcn_readfirstlane(st + (i * (NT / kWave) + w) * kWave * 16));
#pragma unroll
        for (int i = 0; i < B_LD; i++)
            dma16(src.b_at(i, bo), __builtin_amdgcn_readfirstlane(st + BM * BK * 2 + (i * (NT / kWave) + w) * kWave * 16));
    };
    constexpr int D = NSTAGE - 1;  // slices in flight ahead of the one consumed
    for (int kt = 0; kt < D && kt < nk; kt++) issue(kt);
    pre();
    for (int kt = 0; kt < nk; kt++) {
        // Slices kt+1 .. min(kt+D, nk)-1 may stay in flight.
        const int ahead = min(kt + D, nk) - 1 - kt;
        wait_vmcnt_le<(D - 1) * LOADS>(ahead * per_slice);
        __syncthreads();
        if (kt + D < nk) issue(kt + D);
        uint16_t *buf = smem + (kt % NSTAGE) * STAGE;
        mma_slice<NV, SWAP>(buf, buf + BM * BK, wm, brow, acc);
    }
    __syncthreads();
}
#endif

#if OCC_GEMM_PIPE
// The pipelined K loop of the four-wave build (gemm_bf16_dense.hip: one
// wave per SIMD, 128 x 128 per wave, 256 accumulators per lane).  With no
// second wave on the SIMD to fill the gaps, the loop is software-pipelined
// inside the wave: the fragments of a 32-deep step are double-buffered in
// registers, so the next step's LDS reads, and the next slice's direct
// loads, are issued between the current step's MFMAs.  One barrier per
// 64-deep slice, after the slice's first step, once the next slice has
// landed; it also certifies that every wave has read the slice whose buffer
// the following loads overwrite.  Per 256 x 256 x 32 step a wave reads 16
// fragments for 64 MFMAs (0.25 per MFMA against 0.33 in the eight-wave
// build), and every wave issues all of its load slots (rows past the
// tile's repeat its last row), since a load skipped under a branch would
// split the MFMA stream into blocks.
static_assert(NT == 256 && NSTAGE == 2 && BK == 64, "pipelined loop: 4 waves, two 64-deep slots");

// Fragment registers of one 32-deep step: the wave's NV A blocks and NI B
// blocks; the loop keeps two sets, one multiplied while the other is read.
template <int NV>
struct Frags {
    bf16x8_t a[NV > 0 ? NV : 1];
    bf16x8_t b[NI];
};

// Fragment reads with constant offsets: every block's 16 rows start at a
// multiple of 16, so the swizzle key of a lane's row is (l & 15) >> 1 for
// all of them and a lane's offset inside any block is the same.  `ab` / `bb`
// point at that lane offset in the wave's first A / B block of one buffer
// and one 32-deep half; block i then sits a constant number of rows further
// (A: WAVES_M * 16 i; B: the up-projection pairs gate and up blocks 128
// rows apart, the down-projection's are consecutive), so the compiler folds
// it into the read's immediate offset.  Read r of a step: B blocks first,
// since the MFMAs take every B block with A block 0 first.
template <bool UP>
__device__ constexpr int b_block_off(int ni) {
    return UP ? (ni < NI / 2 ? 0 : 128) + (ni % (NI / 2)) * 16 : ni * 16;
}
template <int NV, bool UP>
__device__ __forceinline__ void frag_read(Frags<NV> &f, int r, const uint16_t *ab, const uint16_t *bb) {
    if (r < NI)
        f.b[r] = *reinterpret_cast<const bf16x8_t *>(bb + b_block_off<UP>(r) * BK);
    else
        f.a[r - NI] = *reinterpret_cast<const bf16x8_t *>(ab + WAVES_M * 16 * (r - NI) * BK);
}

// One 32-deep step: the NV x NI MFMAs on `cur`, with the reads of the next
// step's fragments (into `nxt`, when READ) spread over its first three
// quarters and the `nd` direct loads dma(d) over all of it, at most one of
// each after an MFMA (those that find no MFMA follow the last).  A
// scheduling barrier after each MFMA keeps that order.  (The loads issued
// in the step's first quarter or half instead were measured 2-5% slower in
// both products.)
template <int NV, bool SWAP, bool READ, class Dma>
__device__ __forceinline__ void pipe_step(const Frags<NV> &cur, Frags<NV> &nxt, const uint16_t *ab,
                                          const uint16_t *bb, f32x4_t (&acc)[MI][NI], int nd,
                                          Dma &dma) {
    constexpr int NM = NV * NI, NR = NV + NI, ND = A_LD + B_LD;
    constexpr int RSPAN = NM * 3 / 4 > NR ? NM * 3 / 4 : NR;  // read r after MFMA r * RSPAN / NR
    constexpr int DSPAN = NM > ND ? NM : ND;                  // load d after MFMA d * DSPAN / ND
#pragma unroll
    for (int m = 0; m < NM; m++) {
        const int mi = m / NI, ni = m % NI;
        acc[mi][ni] = SWAP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.b[ni], cur.a[mi], acc[mi][ni], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[mi], cur.b[ni], acc[mi][ni], 0, 0, 0);
        const int r = (m * NR + RSPAN - 1) / RSPAN;
        if (READ && r < NR && r * RSPAN / NR == m) frag_read<NV, SWAP>(nxt, r, ab, bb);
        const int d = (m * ND + DSPAN - 1) / DSPAN;
        if (d < ND && d * DSPAN / ND == m && d < nd) dma(d);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (READ) {
#pragma unroll
        for (int r = 0; r < NR; r++)
            if (r * RSPAN / NR >= NM) frag_read<NV, SWAP>(nxt, r, ab, bb);
    }
#pragma unroll
    for (int d = 0; d < ND; d++)
        if (d * DSPAN / ND >= NM && d < nd) dma(d);
}

template <int NV, bool SWAP, class Src, class Pre>
__device__ __forceinline__ void k_loop(const Src &src, int K, int ksp, size_t blk, uint16_t *smem,
                                       int wm, const int (&brow)[NI], f32x4_t (&acc)[MI][NI], int,
                                       Pre &pre) {
    constexpr int LOADS = A_LD + B_LD;
    const int nk = K / BK;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int c0 = lane_id() >> 4;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<size_t>(smem));
    // Direct load d of slice kt: A rows (d < A_LD) or B rows.  The B offset
    // of the slice (blocks of ksp along K) is computed once per slice.
    auto b_off = [&](int kt) {
        const int k0 = kt * BK;
        return ksp == K ? static_cast<size_t>(k0)
                        : static_cast<size_t>(k0 / ksp) * blk + static_cast<size_t>(k0 % ksp);
    };
    auto load = [&](int kt, size_t bo, int d) {
        const uint32_t st = lds0 + static_cast<uint32_t>((kt & 1) * STAGE * 2);
        if (d < A_LD) {
            dma16(src.a_at(d, kt * BK), __builtin_amdgcn_readfirstlane(st + (d * (NT / kWave) + w) * kWave * 16));
        } else {
            const int i = d - A_LD;
            dma16(src.b_at(i, bo), __builtin_amdgcn_readfirstlane(st + BM * BK * 2 + (i * (NT / kWave) + w) * kWave * 16));
        }
    };
    for (int d = 0; d < LOADS; d++) load(0, b_off(0), d);
    pre();
    if (nk > 1)
        for (int d = 0; d < LOADS; d++) load(1, b_off(1), d);
    wait_vmcnt_le<LOADS>(nk > 1 ? LOADS : 0);
    __syncthreads();
    // Lane offsets of the two 32-deep halves of a slice (see frag_read).
    const int key = (lane_id() & 15) >> 1;
    const int h0 = (c0 ^ key) << 3, h1 = ((4 + c0) ^ key) << 3;
    const int ao = (wm * 16 + (lane_id() & 15)) * BK, bo0 = (BM + brow[0]) * BK;
    auto ab = [&](int slot, int h) { return smem + slot * STAGE + ao + h; };
    auto bb = [&](int slot, int h) { return smem + slot * STAGE + bo0 + h; };
    Frags<NV> f0, f1;
#pragma unroll
    for (int r = 0; r < NV + NI; r++) frag_read<NV, SWAP>(f0, r, ab(0, h0), bb(0, h0));
    auto none = [](int) {};
    int kt = 0;
    for (; kt + 2 < nk; kt++) {  // slice kt; slice kt+2's loads go out during its second step
        const int slot = kt & 1;
        pipe_step<NV, SWAP, true>(f0, f1, ab(slot, h1), bb(slot, h1), acc, 0, none);
        wait_vmcnt<0>();
        __syncthreads();
        const size_t bo = b_off(kt + 2);
        auto dma = [&](int d) { load(kt + 2, bo, d); };
        pipe_step<NV, SWAP, true>(f1, f0, ab(slot ^ 1, h0), bb(slot ^ 1, h0), acc, LOADS, dma);
    }
    if (kt + 1 < nk) {  // the last but one slice: nothing left to load
        const int slot = kt & 1;
        pipe_step<NV, SWAP, true>(f0, f1, ab(slot, h1), bb(slot, h1), acc, 0, none);
        wait_vmcnt<0>();
        __syncthreads();
        pipe_step<NV, SWAP, true>(f1, f0, ab(slot ^ 1, h0), bb(slot ^ 1, h0), acc, 0, none);
        kt++;
    }
    {  // the last slice
        const int slot = kt & 1;
        pipe_step<NV, SWAP, true>(f0, f1, ab(slot, h1), bb(slot, h1), acc, 0, none);
        pipe_step<NV, SWAP, false>(f1, f0, ab(slot, h0), bb(slot, h0), acc, 0, none);
    }
    __syncthreads();
}
#endif

// Runs the K loop with the wave's block count as a constant.
template <bool SWAP, int NV = MI, class Src, class Pre>
__device__ __forceinline__ void run_k_loop(int nv, const Src &src, int K, int ksp, size_t blk,
                                           uint16_t *smem, int wm, const int (&brow)[NI],
                                           f32x4_t (&acc)[MI][NI], int na, Pre &pre) {
    if constexpr (NV == 0) {
        k_loop<0, SWAP>(src, K, ksp, blk, smem, wm, brow, acc, na, pre);
    } else if constexpr (OCC_GEMM_PIPE) {
        // a wave with rows multiplies all of its blocks (those past the
        // tile's rows hold repeated rows whose results are not stored)
        if (nv > 0) k_loop<MI, SWAP>(src, K, ksp, blk, smem, wm, brow, acc, na, pre);
        else k_loop<0, SWAP>(src, K, ksp, blk, smem, wm, brow, acc, na, pre);
    } else {
        if (nv >= NV) k_loop<NV, SWAP>(src, K, ksp, blk, smem, wm, brow, acc, na, pre);
        else run_k_loop<SWAP, NV - 1>(nv, src, K, ksp, blk, smem, wm, brow, acc, na, pre);
    }
}

// The wave's share of a tile of `rows` rows: its blocks that hold rows, and
// its A loads (wave w's load i moves rows i * ROWS_PER_PASS + w * 8 .. + 7)
// that do.
__device__ __forceinline__ void wave_share(int rows, int wm, int &nv, int &na) {
    const int blocks = (rows + 15) >> 4;
    nv = __builtin_amdgcn_readfirstlane(min(MI, max(0, (blocks - wm + WAVES_M - 1) / WAVES_M)));
    const int first = static_cast<int>(threadIdx.x) / kWave * (kWave / CHUNKS);
    na = __builtin_amdgcn_readfirstlane(
        min(A_LD, max(0, (rows - first + ROWS_PER_PASS - 1) / ROWS_PER_PASS)));
}

// Second bound: waves per SIMD = workgroups per CU x NT / 256.
__global__ __launch_bounds__(NT, OCC_GEMM_WG_PER_CU * NT / 256) void OCC_NAMED(k_gemm_up)(UpArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGE];
    __shared__ float s_w[BM];
    Tile t;
    if (!tile_of(a.seg_off, a.tile_off, a.M, a.m_tiles, a.Ne, a.tab, (a.N + 127) / 128, 128, t))
        return;

    const int tid = threadIdx.x, r0 = tid / CHUNKS;
    const int K = a.K, N = a.N;
    const uint16_t *A = static_cast<const uint16_t *>(a.A);
    const uint16_t *Wg = static_cast<const uint16_t *>(a.Wg) + static_cast<size_t>(t.e) * N * K;
    const uint16_t *Wu = static_cast<const uint16_t *>(a.Wu) + static_cast<size_t>(t.e) * N * K;
    PtrSrc src;
#pragma unroll
    for (int i = 0; i < A_LD; i++) {
        const int r = min(r0 + i * ROWS_PER_PASS, t.rows - 1);
        const int row = t.seg + t.m0 + r;
        const int arow = a.a_rows ? a.a_rows[row] : row;
        src.a[i] = A + static_cast<size_t>(arow) * K + fetch_chunk(r0 + i * ROWS_PER_PASS) * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; i++) {
        const int rb = r0 + i * ROWS_PER_PASS;
        const int f = min(t.n0 + (rb & 127), N - 1);
        src.b[i] = (rb < 128 ? Wg : Wu) + static_cast<size_t>(f) * K + fetch_chunk(rb) * 8;
    }

    const int l = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;  // wm < WAVES_M
    int brow[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ni++)
        brow[ni] = (ni < NI / 2 ? 0 : 128) + wn * 64 + (ni % (NI / 2)) * 16 + (l & 15);
    f32x4_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; mi++)
#pragma unroll
        for (int ni = 0; ni < NI; ni++) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    int nv, na;
    wave_share(t.rows, wm, nv, na);
    // The rows' routing weights, loaded once by one thread per row (loaded by
    // every lane in the epilogue, they were waited for one by one).
    auto pre = [&] {
        if (tid < t.rows) s_w[tid] = a.row_w ? a.row_w[t.seg + t.m0 + tid] : 1.f;
    };
    run_k_loop<true>(nv, src, K, K, 0, smem, wm, brow, acc, na, pre);

    // SwiGLU + modulation in registers (the sigmoid's division by the
    // hardware reciprocal: the result is rounded to bf16, and the IEEE
    // division sequence made the epilogue -- during which the matrix cores
    // idle -- several times longer); bf16 tiles staged in LDS (the K
    // buffers are free after the loop's last barrier) and written as whole
    // 16-byte row chunks: the hidden state, then in training the gate and up
    // pre-activations the backward pass reads (two more passes through the
    // same staging rows; written lane by lane they were 2-byte stores).
    // All three are non-temporal: the hidden states are read back only by
    // the next launch and the pre-activations by the backward pass, and kept
    // out of the L2 they leave the weight and activation slices that the
    // running tiles share (measured on the OLMoE-shaped layer: -1.5% here,
    // -4% in the decode step; the same hint on the down-projection's fp32
    // stores cost 6-10%).
    constexpr int CH = 128 / 8;  // 16-byte chunks per staged row
    auto stage = [&](int which) {  // 0: h, 1: g, 2: u
        // lane l holds row (l & 15) of each block and features 4 (l >> 4) .. + 3
        // of each 16-feature group (the MFMAs ran with their operands
        // exchanged): one 8-byte LDS write per group
#pragma unroll
        for (int mi = 0; mi < MI; mi++) {
            const int r = block_row(wm, mi) + (l & 15);
            const float wr = s_w[min(r, t.rows - 1)];
#pragma unroll
            for (int ni = 0; ni < NI / 2; ni++) {
                u16x4 o;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const float g = acc[mi][ni][v], u = acc[mi][ni + NI / 2][v];
                    const float x = which == 0 ? g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u * wr
                                               : (which == 1 ? g : u);
                    o[v] = f32_to_bf16_bits(x);
                }
                *reinterpret_cast<u16x4 *>(smem + r * OUT_PITCH + wn * 64 + ni * 16 + 4 * (l >> 4)) = o;
            }
        }
        __syncthreads();
    };
    auto flush = [&](uint16_t *base, size_t ld) {  // staged rows -> base[row * ld + n0 ..]
#pragma unroll 4
        for (int i = tid; i < BM * CH; i += NT) {
            const int r = i / CH, c = (i % CH) * 8;
            if (r >= t.rows || t.n0 + c >= N) continue;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * OUT_PITCH + c);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(
                                               base + (static_cast<size_t>(t.seg) + t.m0 + r) * ld + t.n0 + c));
        }
    };
    stage(0);
    flush(static_cast<uint16_t *>(a.out), N);
    if (a.gu_out) {
        // training: keep the pre-activations for the backward pass, row r
        // holding g in columns [0, N) and u in [N, 2N)
        uint16_t *gu = static_cast<uint16_t *>(a.gu_out);
        __syncthreads();
        stage(1);
        flush(gu, 2 * static_cast<size_t>(N));
        __syncthreads();
        stage(2);
        flush(gu + N, 2 * static_cast<size_t>(N));
    }
}

__global__ __launch_bounds__(NT, OCC_GEMM_WG_PER_CU * NT / 256) void OCC_NAMED(k_gemm_down)(DownArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGE];
    __shared__ int s_dst[BM];
    Tile t;
    if (!tile_of(a.seg_off, a.tile_off, a.M, a.m_tiles, a.Ne, a.tab, (a.N + BN - 1) / BN, BN, t,
                 a.first_cnt, a.phase, kBandDown))
        return;

    const int tid = threadIdx.x, r0 = tid / CHUNKS;
    const int K = a.K, N = a.N, ksp = a.k_split;
    const uint16_t *A = static_cast<const uint16_t *>(a.A);
    // W is (blocks of N x ksp) along K; routed experts have one block (ksp = K).
    const uint16_t *W = static_cast<const uint16_t *>(a.W) + static_cast<size_t>(t.e) * N * K;
    PtrSrc src;
#pragma unroll
    for (int i = 0; i < A_LD; i++) {
        const int r = min(r0 + i * ROWS_PER_PASS, t.rows - 1);
        const int row = t.seg + t.m0 + r;
        const int arow = a.rows ? a.rows[row] : row;
        src.a[i] = A + static_cast<size_t>(arow) * K + fetch_chunk(r0 + i * ROWS_PER_PASS) * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; i++) {
        const int n = min(t.n0 + r0 + i * ROWS_PER_PASS, N - 1);
        src.b[i] = W + static_cast<size_t>(n) * ksp + fetch_chunk(r0 + i * ROWS_PER_PASS) * 8;
    }
    const size_t blk = static_cast<size_t>(N) * ksp;

    const int l = lane_id(), wv = tid / kWave, wm = wv >> 1, wn = wv & 1;  // wm < WAVES_M
    int brow[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ni++) brow[ni] = wn * WN + ni * 16 + (l & 15);
    f32x4_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; mi++)
#pragma unroll
        for (int ni = 0; ni < NI; ni++) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    int nv, na;
    wave_share(t.rows, wm, nv, na);
    // The SFD row of each of the tile's rows, looked up once by one thread
    // per row (two dependent loads): looked up by every lane in the
    // epilogue, the lookups ran in series, one L2 round trip pair per row
    // (measured on the OLMoE-shaped layer: -10% in the first merge phase,
    // -5% in the atomic phase).  Phase 3 sends the rows after the first
    // contributors to their own EPD rows instead, marked by a negative entry
    // ~erow.
    auto pre = [&] {
        if (a.dst_rows && tid < t.rows) {
            const size_t row = static_cast<size_t>(t.seg) + t.m0 + tid;
            const int erow = a.rows ? a.rows[row] : static_cast<int>(row);
            s_dst[tid] = a.phase == 3 && tid >= t.first ? ~erow : a.dst_rows[erow];
        }
    };
    run_k_loop<false>(nv, src, K, ksp, blk, smem, wm, brow, acc, na, pre);

    float *out = a.out;
#pragma unroll
    for (int mi = 0; mi < MI; mi++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int r = block_row(wm, mi) + 4 * (l >> 4) + v;
            if (r >= t.rows) continue;
            const size_t row = static_cast<size_t>(t.seg) + t.m0 + r;
            if (a.dst_rows) {
                const int d = s_dst[r];
                float *dst = d < 0 ? a.epd_out + static_cast<size_t>(~d) * N
                                   : out + static_cast<size_t>(d) * N;
                if (a.phase == 1 || a.phase == 3) {
#pragma unroll
                    for (int ni = 0; ni < NI; ni++) {
                        const int c = t.n0 + wn * WN + ni * 16 + (l & 15);
                        if (c < N) dst[c] = acc[mi][ni][v];
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < NI; ni++) {
                        const int c = t.n0 + wn * WN + ni * 16 + (l & 15);
                        if (c < N) unsafeAtomicAdd(dst + c, acc[mi][ni][v]);
                    }
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < NI; ni++) {
                    const int c = t.n0 + wn * WN + ni * 16 + (l & 15);
                    if (c < N) out[row * N + c] = acc[mi][ni][v];
                }
            }
        }
}

unsigned grid_for(size_t m_tiles, size_t n_tiles) {
    const size_t total = m_tiles * n_tiles;
    return static_cast<unsigned>(8 * ((total + 7) / 8));
}

// Row tiles of a dense product of M rows against n_tiles column tiles: the
// fewest that hold every row (ceil(M / BM)), raised as far as the launch
// still takes the same number of rounds of the GPU's workgroup slots, so the
// last round is filled with shorter tiles instead of running partly empty
// (the Qwen-shaped layer's shared down-projection: 205 x 8 tiles are 6.4
// rounds of 256 CUs, run as 7; 224 x 8 tiles of 293 rows fill the 7 rounds).
// At most one 16-row block per tile.
int dense_row_tiles(int M, int n_tiles) {
    const int m0 = static_cast<int>(ceil_div(M, BM));
    const long slots = static_cast<long>(compute_units()) * OCC_GEMM_WG_PER_CU;
    if (m0 == 0 || n_tiles == 0 || slots <= 0) return m0;
    const long rounds = (static_cast<long>(m0) * n_tiles + slots - 1) / slots;
    const long m = std::min<long>(rounds * slots / n_tiles, (M + 15) / 16);
    return static_cast<int>(std::max<long>(m0, m));
}

}  // namespace

hipError_t OCC_NAMED(launch_gemm_up_bf16)(const UpArgs &a, size_t max_m_tiles, hipStream_t s) {
    UpArgs b = a;
#ifdef OCC_GEMM_DENSE_ONLY
    // routed row-tile schedules are cut for the grouped builds' tile height
    if (a.seg_off) return hipErrorInvalidValue;
#endif
    const int n_tiles = static_cast<int>(ceil_div(a.N, 128));
    if (!a.seg_off) {
        b.m_tiles = dense_row_tiles(a.M, n_tiles);
        max_m_tiles = static_cast<size_t>(b.m_tiles);
    }
    const unsigned grid = grid_for(max_m_tiles, n_tiles);
    if (grid == 0) return hipSuccess;
    OCC_NAMED(k_gemm_up)<<<grid, NT, 0, s>>>(b);
    return hipGetLastError();
}

hipError_t OCC_NAMED(launch_gemm_down_bf16)(const DownArgs &a, size_t max_m_tiles, hipStream_t s) {
    DownArgs b = a;
#ifdef OCC_GEMM_DENSE_ONLY
    // routed row-tile schedules are cut for the grouped builds' tile height
    if (a.seg_off) return hipErrorInvalidValue;
#endif
    const int n_tiles = static_cast<int>(ceil_div(a.N, BN));
    if (!a.seg_off) {
        b.m_tiles = dense_row_tiles(a.M, n_tiles);
        max_m_tiles = static_cast<size_t>(b.m_tiles);
    }
    const unsigned grid = grid_for(max_m_tiles, n_tiles);
    if (grid == 0) return hipSuccess;
    OCC_NAMED(k_gemm_down)<<<grid, NT, 0, s>>>(b);
    return hipGetLastError();
}

}  // namespace occ
