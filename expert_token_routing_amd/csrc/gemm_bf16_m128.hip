// The bf16 grouped GEMMs with 128-row tiles, for batches in which each expert
// sees few rows (the decode regime).  Such launches stream the weights from
// HBM with little reuse, so what counts is that each weight column tile is
// streamed by as few workgroups as possible: at 512 tokens (experts of 47 to
// 80 rows) 64-row tiles made 760 tiles, nearly three rounds of the 256 CUs,
// and 128-row tiles make 512, two rounds, every expert in one row tile
// (measured on the decode step: up-projection 119 -> 107 us, down-projection
// 70 -> 65 us).  Blocks without rows are neither loaded nor multiplied, so
// the taller tile costs little.  The smaller slices (48 KB instead of 72 KB)
// leave room for a third ring slot, which keeps one more slice in flight (a
// fourth gave nothing more).
#define OCC_GEMM_TILE_M 128
#define OCC_GEMM_NSTAGE 3
#define OCC_GEMM_SUFFIX _m128
#include "gemm_bf16.hip"
