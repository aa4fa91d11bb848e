// The bf16 GEMMs for large dense products (the shared experts over a long
// batch): 256 x 256 tiles computed by four waves, one per SIMD, each holding
// 128 x 128 outputs (256 accumulators per lane), with the K loop
// software-pipelined inside the wave (fragment reads and the next slice's
// direct loads issued between the MFMAs).  The larger wave tile reads a
// quarter fewer LDS fragment bytes per flop than the eight-wave build's
// 80 x 128.  Measured on the Qwen-shaped shared expert (T = 65,536, d =
// 2048, F = 5632): up-projection 2.44 -> 2.28 ms, down-projection 1.31 ->
// 1.22 ms, with identical results (the per-element accumulation order is
// the same).  The grouped expert GEMMs stay on the 320-row build: there the
// 256-row tiles' extra weight traffic and the per-tile start of this loop
// outweigh it (routed down-projection 14% slower), and so do dense products
// of few rounds of tiles (a 16,384-token down-projection 7% slower), hence
// the size rule in the library's dispatch.  Dense launches only.
#define OCC_GEMM_TILE_M 256
#define OCC_GEMM_NT 256
#define OCC_GEMM_PIPE 1
#define OCC_GEMM_DENSE_ONLY 1
#define OCC_GEMM_SUFFIX _dense
#include "gemm_bf16.hip"
