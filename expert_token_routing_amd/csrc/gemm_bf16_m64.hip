// The bf16 grouped GEMMs with 64-row tiles, for batches in which each expert
// sees few rows (the decode regime).  Such launches stream the weights from
// HBM with little reuse; the smaller slices (40 KB instead of 72 KB) leave
// room for a third ring slot, which keeps one more slice in flight (measured on the 512-token decode step:
// up-projection 138 -> 126 us; a fourth slot gives nothing more).
#define OCC_GEMM_TILE_M 64
#define OCC_GEMM_NSTAGE 3
#define OCC_GEMM_SUFFIX _m64
#include "gemm_bf16.hip"
