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

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// 16-byte loads and stores marked non-temporal: the expert rows are read
// once and the output written once, so neither should displace lines that
// other work re-reads (measured: the V4-Pro combine 0.184 -> 0.147 ms).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

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
    // two 16-byte column chunks per thread and trip; a trip issues the loads
    // of up to 8 expert rows and the shared row for both chunks before it
    // uses any of them
    const int nv = h / 8;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int v0 = threadIdx.x; v0 < nv; v0 += 512) {
      const int v1 = v0 + 256;
      const bool has1 = v1 < nv;
      float acc[2][8];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[c][q] = 0.0f;
      uint4 s0 = zero, s1 = zero;
      for (int j0 = 0; j0 < k; j0 += 8) {
        uint4 y0[8], y1[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          const int r = (j < k) ? s_row[j] : -1;
          y0[q] = zero;
          y1[q] = zero;
          if (r >= 0) {
            const uint4* row = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Yp) +
                                                              static_cast<size_t>(r) * h);
            y0[q] = load_nt(row + v0);
            if (has1) y1[q] = load_nt(row + v1);
          }
        }
        if (j0 == 0 && Ys) {
          const uint4* srow = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Ys) +
                                                             static_cast<size_t>(t) * h);
          s0 = load_nt(srow + v0);
          if (has1) s1 = load_nt(srow + v1);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          if (j >= k || s_row[j] < 0) continue;
          const float g = s_g[j];
          const uint32_t w0[4] = {y0[q].x, y0[q].y, y0[q].z, y0[q].w};
          const uint32_t w1[4] = {y1[q].x, y1[q].y, y1[q].z, y1[q].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[0][2 * c] = fmaf(g, __uint_as_float(w0[c] << 16), acc[0][2 * c]);
            acc[0][2 * c + 1] = fmaf(g, __uint_as_float(w0[c] & 0xffff0000u), acc[0][2 * c + 1]);
            acc[1][2 * c] = fmaf(g, __uint_as_float(w1[c] << 16), acc[1][2 * c]);
            acc[1][2 * c + 1] = fmaf(g, __uint_as_float(w1[c] & 0xffff0000u), acc[1][2 * c + 1]);
          }
        }
      }
      const uint4 sv[2] = {s0, s1};
      uint4* yrow = reinterpret_cast<uint4*>(static_cast<uint16_t*>(Y) + static_cast<size_t>(t) * h);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c == 1 && !has1) break;
        if (Ys) {
          const uint32_t w[4] = {sv[c].x, sv[c].y, sv[c].z, sv[c].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[c][2 * q] += __uint_as_float(w[q] << 16);
            acc[c][2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
          }
        }
        uint4 o;
        o.x = f32_to_bf16(acc[c][0]) | (static_cast<uint32_t>(f32_to_bf16(acc[c][1])) << 16);
        o.y = f32_to_bf16(acc[c][2]) | (static_cast<uint32_t>(f32_to_bf16(acc[c][3])) << 16);
        o.z = f32_to_bf16(acc[c][4]) | (static_cast<uint32_t>(f32_to_bf16(acc[c][5])) << 16);
        o.w = f32_to_bf16(acc[c][6]) | (static_cast<uint32_t>(f32_to_bf16(acc[c][7])) << 16);
        store_nt(yrow + (c == 0 ? v0 : v1), o);
      }
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
