// combine.hip -- Token Combine of the routed MoE layer (CANN "mega_moe" page,
// §计算过程 Token Combine; DeepSeek-V4 blog post, §模型与入口 for the shared
// expert added at weight 1):
//   y[t] = sum_{j = 0..k-1} G[t, j] * Yp[dst_row[t*k + j]] + Ys[t]
// fp32 accumulation in the fixed order j ascending, then the shared row, one
// rounding to the output type.  A gather-reduce: one block per token, each
// thread owns 16-byte column chunks, so every load and the store are
// 16-byte and row-contiguous.
#include "moe_internal.h"

namespace moe {
namespace {

template <int PREC>
__global__ __launch_bounds__(256) void combine_kernel(int h, int k,
                                                      const void* __restrict__ Yp,
                                                      const int32_t* __restrict__ dst_row,
                                                      const float* __restrict__ G,
                                                      const void* __restrict__ Ys,
                                                      void* __restrict__ Y) {
  __shared__ int32_t s_row[kMaxTopk];
  __shared__ float s_g[kMaxTopk];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = dst_row[static_cast<size_t>(t) * k + threadIdx.x];
    s_g[threadIdx.x] = G[static_cast<size_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  if (PREC == MOE_PREC_F32) {
    const int nv = h / 4;
    for (int v = threadIdx.x; v < nv; v += 256) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j = 0; j < k; ++j) {
        const int r = s_row[j];
        if (r < 0) continue;
        const float g = s_g[j];
        float4 y = reinterpret_cast<const float4*>(static_cast<const float*>(Yp) +
                                                   static_cast<size_t>(r) * h)[v];
        acc.x = fmaf(g, y.x, acc.x);
        acc.y = fmaf(g, y.y, acc.y);
        acc.z = fmaf(g, y.z, acc.z);
        acc.w = fmaf(g, y.w, acc.w);
      }
      if (Ys) {
        float4 s = reinterpret_cast<const float4*>(static_cast<const float*>(Ys) +
                                                   static_cast<size_t>(t) * h)[v];
        acc.x += s.x;
        acc.y += s.y;
        acc.z += s.z;
        acc.w += s.w;
      }
      reinterpret_cast<float4*>(static_cast<float*>(Y) + static_cast<size_t>(t) * h)[v] = acc;
    }
  } else {
    const int nv = h / 8;
    for (int v = threadIdx.x; v < nv; v += 256) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      // groups of 8 rows: all loads of a group are issued before any is used
      for (int j0 = 0; j0 < k; j0 += 8) {
        uint4 yr[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          const int r = (j < k) ? s_row[j] : -1;
          yr[q] = make_uint4(0u, 0u, 0u, 0u);
          if (r >= 0)
            yr[q] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Yp) +
                                                   static_cast<size_t>(r) * h)[v];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          if (j >= k || s_row[j] < 0) continue;
          const float g = s_g[j];
          uint32_t w[4] = {yr[q].x, yr[q].y, yr[q].z, yr[q].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[2 * c] = fmaf(g, __uint_as_float(w[c] << 16), acc[2 * c]);
            acc[2 * c + 1] = fmaf(g, __uint_as_float(w[c] & 0xffff0000u), acc[2 * c + 1]);
          }
        }
      }
      if (Ys) {
        uint4 s = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Ys) +
                                                 static_cast<size_t>(t) * h)[v];
        uint32_t w[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += __uint_as_float(w[q] << 16);
          acc[2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
        }
      }
      uint4 o;
      o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
      o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
      o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
      o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(Y) + static_cast<size_t>(t) * h)[v] = o;
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.precision == MOE_PREC_F32)
    hipLaunchKernelGGL(combine_kernel<MOE_PREC_F32>, dim3(a.T), dim3(256), 0, stream, a.h, a.k,
                       a.Yp, a.dst_row, a.G, a.Ys, a.Y);
  else
    hipLaunchKernelGGL(combine_kernel<MOE_PREC_BF16>, dim3(a.T), dim3(256), 0, stream, a.h, a.k,
                       a.Yp, a.dst_row, a.G, a.Ys, a.Y);
  return hipGetLastError();
}

}  // namespace moe
