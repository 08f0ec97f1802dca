// route_plan.cpp -- the router's launch plan (host code only), shared by the
// router's launcher and the workspace layout of the C ABI.
#include "moe_internal.h"

namespace moe {

// BM tokens per block; K split in powers of two (each part >= 128 and a
// multiple of 32, the K-tile of the gate kernel) until the grid has >= 1024
// blocks.  Large batches: 64-token blocks, each block's gate-weight slice
// read once per 64 tokens instead of 32 (the slices come from L2 and that
// traffic bounded the kernel), with at most 4 K-splits (more splits write and
// re-read more partial logits).
RoutePlan route_plan(int T, int h, int E) {
  constexpr int kBK = 32;
  RoutePlan p;
  p.bm = (T >= 8192 && E <= 384) ? 64 : (T >= 4096 && E <= 384) ? 32 : 16;
  const int mtiles = (T + p.bm - 1) / p.bm;
  const int max_splits = p.bm == 64 ? 4 : 1 << 20;
  p.splits = 1;
  while (mtiles * p.splits < 1024 && p.splits < max_splits && h / (p.splits * 2) >= 128 &&
         (h / (p.splits * 2)) % kBK == 0)
    p.splits *= 2;
  return p;
}

size_t route_partial_bytes(int T, int h, int E) {
  const RoutePlan p = route_plan(T, h, E);
  return p.splits > 1 ? static_cast<size_t>(p.splits) * T * E * 4 : 0;
}

}  // namespace moe
