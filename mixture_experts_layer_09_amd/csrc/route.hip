// route.hip -- the router of the routed MoE layer: gating linear, affinity,
// selection by bias-adjusted score, and the mixing weights (DeepSeek-V4 blog
// post, §路由张量 and §Hash 路由; "Megatron 分布式训练全维度并行技术文档"
// §4.2 for the softmax router).
//
// One kernel.  A block owns BM tokens and every expert column:
//   - gate GEMM: l = X Wg over K-tiles of 64, bf16 MFMA 16x16x32 with fp32
//     accumulation (fp32 inputs use FMA), X tiles and transposed Wg tiles
//     staged in LDS, the next tile prefetched into registers;
//   - the logits tile goes to LDS; each wave then takes whole token rows:
//     lane l holds experts l, l+64, ...; affinity (sigmoid / softmax /
//     sqrt-softplus), key = a + beta, k rounds of a wave-wide argmax by
//     shuffles (ties to the lower expert id), weights alpha * a / sum a.
//   - hash routing reads the selection from tid2eid and keeps the weights.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;          // K per LDS tile
constexpr int kPadH = 8;         // bf16 padding per LDS row (16 B)
constexpr int kLdsRow = kBK + kPadH;

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Load a 4(k) x 8(n) bf16 block of Wg rows k0..k0+3, columns n0..n0+7 and
// store it transposed into Bs[n][k] (8 x 8-byte LDS writes).
__device__ __forceinline__ void load_b_block(const uint16_t* __restrict__ Wg, int h, int E, int k0,
                                             int n0, uint32_t (&r)[4][4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint16_t* p = Wg + static_cast<size_t>(k0 + q) * E + n0;
    if (n0 + 8 <= E) {
      // n0 is a multiple of 8 and E a multiple of 8 in this branch's aligned case
      if ((E & 7) == 0) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        r[q][0] = v.x;
        r[q][1] = v.y;
        r[q][2] = v.z;
        r[q][3] = v.w;
        continue;
      }
    }
    uint16_t e[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] = (n0 + c < E) ? p[c] : static_cast<uint16_t>(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) r[q][c] = e[2 * c] | (static_cast<uint32_t>(e[2 * c + 1]) << 16);
  }
  (void)h;
}

__device__ __forceinline__ void store_b_block(uint16_t* Bs, int kl, int nl, const uint32_t (&r)[4][4]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t d0 = __builtin_amdgcn_perm(r[1][c >> 1], r[0][c >> 1], sel);
    uint32_t d1 = __builtin_amdgcn_perm(r[3][c >> 1], r[2][c >> 1], sel);
    *reinterpret_cast<uint2*>(Bs + (nl + c) * kLdsRow + kl) = make_uint2(d0, d1);
  }
}

template <int BM, int EP, int PREC>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  // LDS: during the GEMM, As[BM][kLdsRow] + Bs[EP][kLdsRow] (bf16); afterwards
  // the same memory holds the fp32 logits tile [BM][EP + 1].
  constexpr size_t kGemmBytes = (BM + EP) * kLdsRow * 2;
  constexpr size_t kLogitBytes = BM * (EP + 1) * 4;
  constexpr size_t kLds = kGemmBytes > kLogitBytes ? kGemmBytes : kLogitBytes;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  float* logit = reinterpret_cast<float*>(lds);
  constexpr int LR = EP + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m0 = blockIdx.x * BM;
  const int T = a.T, h = a.h, E = a.E, k = a.k;

  if (PREC == MOE_PREC_F32) {
    // fp32: plain FMA, one (row, expert) pair per thread per step
    const float* X = static_cast<const float*>(a.X);
    const float* Wg = static_cast<const float*>(a.Wg);
    for (int p = tid; p < BM * EP; p += kThreads) {
      int r = p / EP, e = p % EP;
      int t = min(m0 + r, T - 1);
      float s = 0.0f;
      if (e < E)
        for (int c = 0; c < h; ++c) s = fmaf(X[static_cast<size_t>(t) * h + c], Wg[static_cast<size_t>(c) * E + e], s);
      logit[r * LR + e] = s;
    }
    __syncthreads();
  } else {
    uint16_t* As = reinterpret_cast<uint16_t*>(lds);
    uint16_t* Bs = As + BM * kLdsRow;
    const uint16_t* X = static_cast<const uint16_t*>(a.X);
    const uint16_t* Wg = static_cast<const uint16_t*>(a.Wg);
    constexpr int kNT = EP / 64;  // 16-wide n-tiles per wave (wave owns EP/4 columns)
    constexpr int kMT = BM / 16;
    constexpr int kAChunks = BM * kBK / 8;                     // 16-byte chunks of the A tile
    constexpr int kAPer = (kAChunks + kThreads - 1) / kThreads;
    constexpr int kBBlocks = (kBK / 4) * (EP / 8);              // 4x8 blocks of the B tile
    constexpr int kBPer = (kBBlocks + kThreads - 1) / kThreads;
    f32x4_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[kAPer];
    uint32_t rb[kBPer][4][4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int q = 0; q < kAPer; ++q) {
        int c = tid + q * kThreads;
        if (c < kAChunks) {
          int r = c / (kBK / 8), c8 = c % (kBK / 8);
          int t = min(m0 + r, T - 1);
          ra[q] = *reinterpret_cast<const uint4*>(X + static_cast<size_t>(t) * h + k0 + c8 * 8);
        }
      }
#pragma unroll
      for (int q = 0; q < kBPer; ++q) {
        int b = tid + q * kThreads;
        if (b < kBBlocks) {
          int nb = b % (EP / 8), kb = b / (EP / 8);
          load_b_block(Wg, h, E, k0 + kb * 4, nb * 8, rb[q]);
        }
      }
    };
    auto sstore = [&]() {
#pragma unroll
      for (int q = 0; q < kAPer; ++q) {
        int c = tid + q * kThreads;
        if (c < kAChunks) {
          int r = c / (kBK / 8), c8 = c % (kBK / 8);
          *reinterpret_cast<uint4*>(As + r * kLdsRow + c8 * 8) = ra[q];
        }
      }
#pragma unroll
      for (int q = 0; q < kBPer; ++q) {
        int b = tid + q * kThreads;
        if (b < kBBlocks) {
          int nb = b % (EP / 8), kb = b / (EP / 8);
          store_b_block(Bs, kb * 4, nb * 8, rb[q]);
        }
      }
    };
    gload(0);
    for (int k0 = 0; k0 < h; k0 += kBK) {
      __syncthreads();  // previous tile fully consumed
      sstore();
      __syncthreads();
      if (k0 + kBK < h) gload(k0 + kBK);
#pragma unroll
      for (int kk = 0; kk < kBK; kk += 32) {
        bf16x8_t af[kMT];
#pragma unroll
        for (int i = 0; i < kMT; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(As + (i * 16 + (lane & 15)) * kLdsRow + kk +
                                                     (lane >> 4) * 8);
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          bf16x8_t bfr = *reinterpret_cast<const bf16x8_t*>(
              Bs + (wave * (EP / 4) + j * 16 + (lane & 15)) * kLdsRow + kk + (lane >> 4) * 8);
#pragma unroll
          for (int i = 0; i < kMT; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // LDS now becomes the logits tile
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          logit[(i * 16 + (lane >> 4) * 4 + v) * LR + wave * (EP / 4) + j * 16 + (lane & 15)] =
              acc[i][j][v];
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  constexpr int kQ = EP / 64;  // expert values per lane
  const bool hash = (a.token_ids != nullptr && a.tid2eid != nullptr);
  for (int r = wave; r < BM; r += kThreads / 64) {
    const int t = m0 + r;
    if (t >= T) break;  // uniform across the wave
    float av[kQ], key[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      int e = lane + 64 * q;
      float l = (e < E) ? logit[r * LR + e] + (a.gate_bias ? a.gate_bias[e] : 0.0f) : -INFINITY;
      av[q] = l;
    }
    if (a.score_fn == MOE_SCORE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < kQ; ++q) m = fmaxf(m, av[q]);
      m = wave_max(m);
      float z = 0.0f;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        av[q] = (lane + 64 * q < E) ? expf(av[q] - m) : 0.0f;
        z += av[q];
      }
      z = wave_sum(z);
#pragma unroll
      for (int q = 0; q < kQ; ++q) av[q] = av[q] / z;
    } else if (a.score_fn == MOE_SCORE_SQRT_SOFTPLUS) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        float l = av[q];
        float sp = l > 0.0f ? l + log1pf(expf(-l)) : log1pf(expf(l));
        av[q] = (lane + 64 * q < E) ? sqrtf(sp) : 0.0f;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kQ; ++q)
        av[q] = (lane + 64 * q < E) ? 1.0f / (1.0f + expf(-av[q])) : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      int e = lane + 64 * q;
      key[q] = (e < E) ? av[q] + ((a.beta && !hash) ? a.beta[e] : 0.0f) : -INFINITY;
      if (a.keys && e < E) a.keys[static_cast<size_t>(t) * E + e] = key[q];
    }
    // lane j (< k) keeps choice j: its expert id and unbiased affinity
    int my_id = -1;
    float my_a = 0.0f;
    if (!hash) {
      unsigned taken = 0u;
      for (int j = 0; j < k; ++j) {
        float bk = -INFINITY, ba = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          int e = lane + 64 * q;
          if (!(taken & (1u << q)) && e < E && better(key[q], e, bk, bi)) {
            bk = key[q];
            bi = e;
            ba = av[q];
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          float ok = __shfl_xor(bk, o, 64);
          int oi = __shfl_xor(bi, o, 64);
          float oa = __shfl_xor(ba, o, 64);
          if (better(ok, oi, bk, bi)) {
            bk = ok;
            bi = oi;
            ba = oa;
          }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
          my_id = bi;
          my_a = ba;
        }
      }
    } else {
      const int tok = a.token_ids[t];
      const bool ok_tok = tok >= 0 && tok < a.vocab;
      for (int j = 0; j < k; ++j) {
        int e = ok_tok ? a.tid2eid[static_cast<size_t>(tok) * k + j] : -1;
        if (e < 0 || e >= E) e = -1;
        float v = 0.0f;
        if (e >= 0) {
          int qs = e >> 6;
          float mine = 0.0f;
#pragma unroll
          for (int q = 0; q < kQ; ++q)
            if (q == qs) mine = av[q];
          v = __shfl(mine, e & 63, 64);
        }
        if (lane == j) {
          my_id = e;
          my_a = v;
        }
      }
      if (lane < k && my_id < 0) a.flag[0] = 1;
    }
    const float den = wave_sum(lane < k ? my_a : 0.0f);
    if (lane < k) {
      a.ids[static_cast<size_t>(t) * k + lane] = my_id;
      float g = a.renorm ? a.alpha * my_a / den : a.alpha * my_a;
      a.G[static_cast<size_t>(t) * k + lane] = (my_id >= 0) ? g : 0.0f;
    }
  }
}

template <int BM, int EP>
hipError_t launch_ep(const RouteArgs& a, hipStream_t stream) {
  dim3 grid((a.T + BM - 1) / BM);
  if (a.precision == MOE_PREC_F32)
    hipLaunchKernelGGL((route_kernel<BM, EP, MOE_PREC_F32>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((route_kernel<BM, EP, MOE_PREC_BF16>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int BM>
hipError_t launch_bm(const RouteArgs& a, hipStream_t stream) {
  if (a.E <= 64) return launch_ep<BM, 64>(a, stream);
  if (a.E <= 128) return launch_ep<BM, 128>(a, stream);
  if (a.E <= 256) return launch_ep<BM, 256>(a, stream);
  if (a.E <= 384) return launch_ep<BM, 384>(a, stream);
  return launch_ep<BM, 512>(a, stream);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  // Large T: 32 tokens per block halves the re-reads of Wg; small T: 16 keeps
  // more blocks in flight.
  if (a.T >= 4096 && a.E <= 384) return launch_bm<32>(a, stream);
  return launch_bm<16>(a, stream);
}

}  // namespace moe
