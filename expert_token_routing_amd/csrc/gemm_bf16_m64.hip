// The bf16 grouped GEMMs with 64-row tiles, for batches in which each expert
// sees few rows (the decode regime): a 256-row tile would spend most of its
// MFMA work on padding while the weights it streams are the same.
#define OCC_GEMM_TILE_M 64
#define OCC_GEMM_SUFFIX _m64
#include "gemm_bf16.hip"
