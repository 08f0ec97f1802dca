// route_plan.cpp -- the router's launch plan (host code only), shared by the
// router's launcher and the workspace layout of the C ABI.
#include "moe_internal.h"

namespace moe {

// bf16 with E a multiple of 128 (E <= 512): the DMA-fed gate GEMM on
// 64- or 128-token blocks, its K split in powers of two (each part a multiple of
// 32 and at least 256) until the grid has one block per CU (256); every
// block writes fp32 partial logits and the top-k kernel sums them in split
// order and routes.
//
// Otherwise (fp32, other E): BM tokens per block; K split in powers of two
// (each part >= 128 and a multiple of 32) until the grid has >= 1024 blocks.
// Large batches: 64-token blocks, each block's gate-weight slice read once
// per 64 tokens instead of 32 (the slices come from L2 and that traffic
// bounded the kernel), with at most 4 K-splits (more splits write and re-read
// more partial logits).  One split: the block routes its tokens itself.
RoutePlan route_plan(int T, int h, int E, int precision) {
  constexpr int kBK = 32;
  RoutePlan p;
  if (precision != MOE_PREC_F32 && E % 128 == 0 && E <= 512 && h % 256 == 0) {
    p.dma = 1;
    // 128-token blocks where there are at least 32 of them: each block's
    // gate-weight slice serves twice the tokens (half the L2 reads and LDS
    // operand bytes per FLOP of 64-token blocks)
    p.bm = T >= 4096 ? 128 : 64;
    const int mtiles = (T + p.bm - 1) / p.bm;
    p.splits = 1;
    while (mtiles * p.splits < 256 && h / (p.splits * 2) >= 256 && (h / (p.splits * 2)) % kBK == 0)
      p.splits *= 2;
    return p;
  }
  p.dma = 0;
  p.bm = (T >= 8192 && E <= 384) ? 64 : (T >= 4096 && E <= 384) ? 32 : 16;
  const int mtiles = (T + p.bm - 1) / p.bm;
  const int max_splits = p.bm == 64 ? 4 : 1 << 20;
  p.splits = 1;
  while (mtiles * p.splits < 1024 && p.splits < max_splits && h / (p.splits * 2) >= 128 &&
         (h / (p.splits * 2)) % kBK == 0)
    p.splits *= 2;
  return p;
}

size_t route_partial_bytes(int T, int h, int E, int precision) {
  const RoutePlan p = route_plan(T, h, E, precision);
  return (p.dma || p.splits > 1) ? static_cast<size_t>(p.splits) * T * E * 4 : 0;
}

}  // namespace moe
