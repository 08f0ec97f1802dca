// ffn_plan.cpp -- which expert-FFN launches may gather their Linear1 rows
// from the layer input (host code only), shared by the forward's launcher
// and the expert FFN's argument check.
#include "moe_internal.h"

namespace moe {

// Mirrors the grouped GEMM dispatch for bf16: Linear1 runs on the DMA kernel
// (whose token-row DMAs take per-row offsets) unless the batch is
// decode-sized without 512-wide n-tiles or the widths allow only 128-wide
// ones; every byte offset into the input must stay below 2^32.
bool ffn_gathers(int precision, int T, int h, int E, int k, int f) {
  if (precision != MOE_PREC_BF16) return false;
  const long rows = static_cast<long>(T) * k;
  const bool w512 = (h % 512 == 0) && ((2 * f) % 512 == 0);
  const bool wide = (h % 256 == 0) && ((2 * f) % 256 == 0);
  const bool small = rows < 16L * E && !w512;
  return wide && !small && static_cast<unsigned long long>(T) * h * 2 <= 0xffffffffull;
}

}  // namespace moe
