// The bf16 grouped GEMMs with 64-row tiles, for batches in which each expert
// sees few rows (the decode regime): a 256-row tile would spend most of its
// MFMA work on padding while the weights it streams are the same.  Such
// launches stream weights from HBM with little reuse, so a third ring slot
// keeps one more slice in flight (measured on the 512-token decode step:
// up-projection 138 -> 126 us; a fourth slot gives nothing more).
#define OCC_GEMM_TILE_M 64
#define OCC_GEMM_NSTAGE 3
#define OCC_GEMM_SUFFIX _m64
#include "gemm_bf16.hip"
