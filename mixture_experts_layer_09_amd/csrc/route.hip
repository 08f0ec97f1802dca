// route.hip -- the router of the routed MoE layer: gating linear, affinity,
// selection by bias-adjusted score, and the mixing weights (DeepSeek-V4 blog
// post, §路由张量 and §Hash 路由; "Megatron 分布式训练全维度并行技术文档"
// §4.2 for the softmax router).
//
// gate_kernel: a block owns BM tokens and every expert column (E padded to a
// multiple of 64; each of the 4 waves owns a quarter) over a range of K.
// K-slices of 32 go through a double-buffered LDS tile, the next slice
// prefetched into registers: token rows are K-contiguous, gate-weight rows
// ([h, E] row-major) are copied as they are and the MFMA B fragments are
// read with the transposing LDS load ds_read_b64_tr_b16 (see grouped_gemm.hip
// for its lane mapping).  Rows are padded by 16 bytes, which puts the 16 rows
// of an operand read, and the 4 rows of each transposing read, on distinct
// bank groups.  bf16 MFMA 16x16x32, fp32 accumulation (fp32 inputs use FMA).
//
// K is split (powers of two) until the grid has about 1024 blocks.  With one
// K range the logits tile goes to LDS and the block finishes the routing
// itself; otherwise each block writes partial logits for its K range and
// route_epilogue_kernel sums them in a fixed order and routes.
//
// The routing epilogue takes one token row per wave: lane l holds experts l,
// l+64, ...; affinity (sigmoid / softmax / sqrt-softplus), key = a + beta, k
// rounds of a wave-wide argmax by shuffles (ties to the lower expert id),
// weights alpha * a / sum a (or alpha * a).  Hash routing reads the selection
// from tid2eid and keeps the weights.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;                  // K elements per LDS tile
constexpr int kARow = kBK * 2 + 16;      // bytes per padded token row

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ i16x4_t ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

// The routing of one token from its logits (lane l holds logits of experts
// l + 64 q in lg[q]); writes ids, G and optionally keys.
template <int EP>
__device__ __forceinline__ void route_token(const RouteArgs& a, int t, int lane, float (&lg)[EP / 64]) {
  constexpr int kQ = EP / 64;
  const int E = a.E, k = a.k;
  const bool hash = (a.token_ids != nullptr && a.tid2eid != nullptr);
  float av[kQ], key[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int e = lane + 64 * q;
    av[q] = (e < E) ? lg[q] + (a.gate_bias ? a.gate_bias[e] : 0.0f) : -INFINITY;
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
      const float l = av[q];
      const float sp = l > 0.0f ? l + log1pf(expf(-l)) : log1pf(expf(l));
      av[q] = (lane + 64 * q < E) ? sqrtf(sp) : 0.0f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kQ; ++q) av[q] = (lane + 64 * q < E) ? 1.0f / (1.0f + expf(-av[q])) : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int e = lane + 64 * q;
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
        const int e = lane + 64 * q;
        if (!(taken & (1u << q)) && e < E && better(key[q], e, bk, bi)) {
          bk = key[q];
          bi = e;
          ba = av[q];
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ok = __shfl_xor(bk, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const float oa = __shfl_xor(ba, o, 64);
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
        const int qs = e >> 6;
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
    const float g = a.renorm ? a.alpha * my_a / den : a.alpha * my_a;
    a.G[static_cast<size_t>(t) * k + lane] = (my_id >= 0) ? g : 0.0f;
  }
}

// Logits of BM tokens x EP experts over K range [kb, ke) (multiples of 32).
// FUSED: finish the routing in the block; else write partial logits
// part[split][t][e] (fp32, E columns).
template <int BM, int EP, int PREC, bool FUSED>
__global__ __launch_bounds__(kThreads) void gate_kernel(RouteArgs a, int kchunk, float* part) {
  constexpr int BRow = EP * 2 + 16;  // bytes per padded gate-weight row in LDS
  constexpr int kAStage = BM * kARow;
  constexpr int kBStage = kBK * BRow;
  constexpr int kStage = kAStage + kBStage;
  constexpr int LR = EP + 1;  // fp32 logits tile row
  constexpr size_t kGemmBytes = 2 * kStage;
  constexpr size_t kLogitBytes = FUSED ? static_cast<size_t>(BM) * LR * 4 : 0;
  constexpr size_t kLds = kGemmBytes > kLogitBytes ? kGemmBytes : kLogitBytes;
  __shared__ __attribute__((aligned(16))) char lds[kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m0 = blockIdx.x * BM;
  const int split = blockIdx.y;
  const int T = a.T, h = a.h, E = a.E;
  const int kb = split * kchunk, ke = min(h, kb + kchunk);
  float* logit = reinterpret_cast<float*>(lds);

  if (PREC == MOE_PREC_F32) {
    // fp32: plain FMA, one (row, expert) pair per thread per step
    const float* X = static_cast<const float*>(a.X);
    const float* Wg = static_cast<const float*>(a.Wg);
    for (int p = tid; p < BM * EP; p += kThreads) {
      const int r = p / EP, e = p % EP;
      const int t = min(m0 + r, T - 1);
      float s = 0.0f;
      if (e < E)
        for (int c = kb; c < ke; ++c)
          s = fmaf(X[static_cast<size_t>(t) * h + c], Wg[static_cast<size_t>(c) * E + e], s);
      if (FUSED)
        logit[r * LR + e] = s;
      else if (m0 + r < T && e < E)
        part[(static_cast<size_t>(split) * T + m0 + r) * E + e] = s;
    }
  } else {
    const char* X = static_cast<const char*>(a.X);
    const char* Wg = static_cast<const char*>(a.Wg);
    constexpr int kNT = EP / 64;  // 16-column n-tiles per wave
    constexpr int kMT = BM / 16;
    constexpr int kAChunks = BM * 4;            // 16-byte chunks of the A tile
    constexpr int kBChunks = kBK * EP / 8;      // 16-byte chunks of the B tile
    constexpr int kAPer = (kAChunks + kThreads - 1) / kThreads;
    constexpr int kBPer = (kBChunks + kThreads - 1) / kThreads;
    const bool e_aligned = (E % 8) == 0;
    f32x4_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    i32x4_t ra[kAPer];
    i32x4_t rb[kBPer];
    auto gload = [&](int k0) {
#pragma unroll
      for (int q = 0; q < kAPer; ++q) {
        const int c = (tid + q * kThreads) % kAChunks;
        const int r = c >> 2, c16 = c & 3;
        const int t = min(m0 + r, T - 1);
        ra[q] = *reinterpret_cast<const i32x4_t*>(X + (static_cast<size_t>(t) * h + k0) * 2 + c16 * 16);
      }
#pragma unroll
      for (int q = 0; q < kBPer; ++q) {
        const int c = (tid + q * kThreads) % kBChunks;
        const int r = c / (EP / 8), n8 = c % (EP / 8);
        const size_t row = static_cast<size_t>(k0 + r) * E;
        if (e_aligned && n8 * 8 + 8 <= E) {
          rb[q] = *reinterpret_cast<const i32x4_t*>(Wg + (row + n8 * 8) * 2);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int e0 = n8 * 8 + 2 * p;
            const uint32_t lo = e0 < E ? reinterpret_cast<const uint16_t*>(Wg)[row + e0] : 0u;
            const uint32_t hi = e0 + 1 < E ? reinterpret_cast<const uint16_t*>(Wg)[row + e0 + 1] : 0u;
            w[p] = lo | (hi << 16);
          }
          rb[q] = i32x4_t{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                          static_cast<int>(w[3])};
        }
      }
    };
    auto sstore = [&](int buf) {
      char* st = lds + buf * kStage;
#pragma unroll
      for (int q = 0; q < kAPer; ++q) {
        const int c = (tid + q * kThreads) % kAChunks;
        *reinterpret_cast<i32x4_t*>(st + (c >> 2) * kARow + (c & 3) * 16) = ra[q];
      }
#pragma unroll
      for (int q = 0; q < kBPer; ++q) {
        const int c = (tid + q * kThreads) % kBChunks;
        const int r = c / (EP / 8), n8 = c % (EP / 8);
        *reinterpret_cast<i32x4_t*>(st + kAStage + r * BRow + n8 * 16) = rb[q];
      }
    };
    // per-lane LDS offsets of the operand reads
    const int grp = lane >> 4, p = lane & 15;
    int a_off[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) a_off[i] = (i * 16 + (lane & 15)) * kARow + grp * 16;
    int b_off[kNT][2];
#pragma unroll
    for (int j = 0; j < kNT; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = 8 * grp + 4 * hh + (p >> 2);
        const int col = wave * (EP / 4) + j * 16 + (p & 3) * 4;
        b_off[j][hh] = kAStage + r * BRow + col * 2;
      }
    const int KT = (ke - kb) / kBK;
    gload(kb);
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      sstore(buf);
      __syncthreads();
      if (kt + 1 < KT) gload(kb + (kt + 1) * kBK);
      const char* st = lds + buf * kStage;
      bf16x8_t bfr[kNT];
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const i16x4_t lo4 = ds_read_tr16(st + b_off[j][0]);
        const i16x4_t hi4 = ds_read_tr16(st + b_off[j][1]);
        const i16x8_t v = i16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        bfr[j] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(st + a_off[i]);
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();  // LDS is reused for the logits tile below
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = i * 16 + (lane >> 4) * 4 + v;
          const int e = wave * (EP / 4) + j * 16 + (lane & 15);
          if (FUSED)
            logit[r * LR + e] = acc[i][j][v];
          else if (m0 + r < T && e < E)
            part[(static_cast<size_t>(split) * T + m0 + r) * E + e] = acc[i][j][v];
        }
  }
  if (!FUSED) return;
  __syncthreads();
  for (int r = wave; r < BM; r += kThreads / 64) {
    const int t = m0 + r;
    if (t >= T) break;  // uniform across the wave
    float lg[EP / 64];
#pragma unroll
    for (int q = 0; q < EP / 64; ++q) lg[q] = logit[r * LR + lane + 64 * q];
    route_token<EP>(a, t, lane, lg);
  }
}

// Sums split partial logits and routes: one wave per token.
template <int EP>
__global__ __launch_bounds__(kThreads) void route_epilogue_kernel(RouteArgs a, int splits,
                                                                  const float* part) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= a.T) return;
  float lg[EP / 64];
#pragma unroll
  for (int q = 0; q < EP / 64; ++q) {
    const int e = lane + 64 * q;
    float s = 0.0f;
    if (e < a.E)
      for (int sp = 0; sp < splits; ++sp) s += part[(static_cast<size_t>(sp) * a.T + t) * a.E + e];
    lg[q] = s;
  }
  route_token<EP>(a, t, lane, lg);
}

template <int BM, int EP>
hipError_t launch_ep(const RouteArgs& a, int splits, hipStream_t stream) {
  const int mtiles = (a.T + BM - 1) / BM;
  const int kchunk = a.h / splits;
  float* part = a.part;
  dim3 grid(mtiles, splits);
  if (splits == 1) {
    if (a.precision == MOE_PREC_F32)
      hipLaunchKernelGGL((gate_kernel<BM, EP, MOE_PREC_F32, true>), grid, dim3(kThreads), 0,
                         stream, a, kchunk, part);
    else
      hipLaunchKernelGGL((gate_kernel<BM, EP, MOE_PREC_BF16, true>), grid, dim3(kThreads), 0,
                         stream, a, kchunk, part);
    return hipGetLastError();
  }
  if (a.precision == MOE_PREC_F32)
    hipLaunchKernelGGL((gate_kernel<BM, EP, MOE_PREC_F32, false>), grid, dim3(kThreads), 0, stream,
                       a, kchunk, part);
  else
    hipLaunchKernelGGL((gate_kernel<BM, EP, MOE_PREC_BF16, false>), grid, dim3(kThreads), 0,
                       stream, a, kchunk, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((route_epilogue_kernel<EP>), dim3((a.T + 3) / 4), dim3(kThreads), 0, stream,
                     a, splits, static_cast<const float*>(part));
  return hipGetLastError();
}

template <int BM>
hipError_t launch_bm(const RouteArgs& a, int splits, hipStream_t stream) {
  if (a.E <= 64) return launch_ep<BM, 64>(a, splits, stream);
  if (a.E <= 128) return launch_ep<BM, 128>(a, splits, stream);
  if (a.E <= 256) return launch_ep<BM, 256>(a, splits, stream);
  if (a.E <= 384) return launch_ep<BM, 384>(a, splits, stream);
  return launch_ep<BM, 512>(a, splits, stream);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const RoutePlan p = route_plan(a.T, a.h, a.E);
  if (p.bm == 64) return launch_bm<64>(a, p.splits, stream);
  return p.bm == 32 ? launch_bm<32>(a, p.splits, stream) : launch_bm<16>(a, p.splits, stream);
}

}  // namespace moe
