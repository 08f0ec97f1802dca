// permute.hip -- dispatch of the routed MoE layer: per-expert counts, the
// destination row of every (token, choice) assignment, and the duplicating
// row copy X -> Xp (CANN "mega_moe" page, §计算过程 EP Dispatch; DeepSeek-V4
// blog post, §计数与重排).
//
// Three kernels, no global atomics, deterministic:
//   1. count_rank: block b takes assignments [b*2048, (b+1)*2048) of the flat
//      array ids[T*k] as 32 groups of 64 (one per wave and round).  Inside a
//      group a lane finds its rank among the group's earlier lanes with the
//      same expert by reading the 64 lanes' experts in turn; the group's per-expert counts go to LDS,
//      a scan over the 32 groups per expert turns them into group bases, and
//      the block writes its per-expert counts blk_cnt[b][e] and each
//      assignment's rank among the block's earlier assignments to the same
//      expert.  Large blocks keep the per-block count table short, so the
//      single-block scan that follows reads few rows of it.
//   2. scan: one block turns blk_cnt into counts[e], offsets[e] (exclusive
//      prefix over experts) and, in place, blk_cnt[b][e] = offsets[e] + sum
//      of blk_cnt[b'][e] over b' < b (the block's base row for expert e).
//   3. scatter: one block per token; dst_row[t*k+j] = base + rank, src_tok of
//      that row = t, and the token row is copied to each of its k rows with
//      16-byte loads and stores.  For A8W8 the row is quantised once, to
//      e4m3 (scale = max|x| / 448) or int8 (scale = max|x| / 127), and the
//      codes are what is copied; MX rows are quantised per 32-value group.
// Row order inside an expert block is ascending t*k+j, a stable order; the
// pages leave the order to the implementation as long as it is fixed.
#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

// Scratch of the dispatch without a workspace (moe_permute_no_alloc), one
// copy per GPU: the error flag, the per-block expert counts and the in-block
// ranks of at most MOE_NO_ALLOC_MAX_ASSIGNMENTS assignments and kMaxExperts
// experts.
constexpr size_t kNoAllocFlagBytes = 256;
constexpr size_t kNoAllocBlkBytes =
    static_cast<size_t>((MOE_NO_ALLOC_MAX_ASSIGNMENTS + kPermChunk - 1) / kPermChunk) * kMaxExperts * 4;
constexpr size_t kNoAllocRankBytes = static_cast<size_t>(MOE_NO_ALLOC_MAX_ASSIGNMENTS) * 4;
constexpr size_t kNoAllocScratchBytes = kNoAllocFlagBytes + kNoAllocBlkBytes + kNoAllocRankBytes;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(kPermThreads) void count_rank_kernel(const int32_t* __restrict__ ids,
                                                                  int n, int E,
                                                                  int32_t* __restrict__ blk_cnt,
                                                                  int32_t* __restrict__ local_rank,
                                                                  uint8_t* __restrict__ blk_err) {
  constexpr int kGroups = kPermChunk / 64;  // groups of 64 assignments
  constexpr int kRounds = kPermChunk / kPermThreads;
  __shared__ int32_t s_cnt[kGroups][kMaxExperts];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int base = blockIdx.x * kPermChunk;
  for (int x = tid; x < kGroups * kMaxExperts; x += kPermThreads) (&s_cnt[0][0])[x] = 0;
  if (tid == 0) s_err = 0;
  int e[kRounds], rank[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = base + r * kPermThreads + tid;
    int v = -1;
    if (i < n) {
      v = ids[i];
      if (v < 0 || v >= E) v = -1;
    }
    e[r] = v;
  }
  __syncthreads();  // s_cnt and s_err cleared
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    if (e[r] < 0 && base + r * kPermThreads + tid < n) s_err = 1;  // every writer stores 1
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    // rank among the group's earlier lanes with the same expert, and the
    // group's count of that expert
    int rk = 0, cnt = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const int o = __builtin_amdgcn_readlane(e[r], j);
      const int eq = (o == e[r]) ? 1 : 0;
      rk += (j < lane) ? eq : 0;
      cnt += eq;
    }
    rank[r] = rk;
    if (e[r] >= 0 && rk == cnt - 1) s_cnt[r * (kPermThreads / 64) + wave][e[r]] = cnt;
  }
  __syncthreads();
  // this block's error byte (an expert id outside [0, E)), for the scan
  if (tid == 0) blk_err[blockIdx.x] = static_cast<uint8_t>(s_err);
  // per expert: exclusive scan over the groups, in group order
  for (int x = tid; x < E; x += kPermThreads) {
    int run = 0;
    for (int g = 0; g < kGroups; ++g) {
      const int c = s_cnt[g][x];
      s_cnt[g][x] = run;
      run += c;
    }
    blk_cnt[static_cast<size_t>(blockIdx.x) * E + x] = run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = base + r * kPermThreads + tid;
    if (i < n)
      local_rank[i] = (e[r] >= 0) ? s_cnt[r * (kPermThreads / 64) + wave][e[r]] + rank[r] : -1;
  }
}

// One block of 512 threads; E <= 512, one thread per expert.  The loops over
// the per-block counts load 8 blocks at a time so that the loads overlap.
// The prefix over the experts is a shuffle scan inside each wave plus the
// earlier waves' totals.  The device error flag: set when a counting block
// saw an expert id outside [0, E); with `clear` it is written either way
// (the dispatch is then the first step of its call that can raise it).
__global__ __launch_bounds__(kMaxExperts) void scan_kernel(int nblk, int E,
                                                           int32_t* __restrict__ blk_cnt,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           const uint8_t* __restrict__ blk_err,
                                                           int32_t* __restrict__ flag, int clear) {
  __shared__ int32_t s_wave[kMaxExperts / 64];
  constexpr int U = 8;
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  int my_err = 0;
  for (int b = e; b < nblk; b += kMaxExperts) my_err |= blk_err[b];
  const int err = __syncthreads_or(my_err);
  if (e == 0 && (clear || err)) flag[0] = err ? 1 : 0;
  int total = 0;
  if (e < E) {
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = blk_cnt[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) total += v[u];
    }
    for (; b < nblk; ++b) total += blk_cnt[static_cast<size_t>(b) * E + e];
  }
  // inclusive scan over the experts: inside the wave, then the waves before
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += s_wave[w];
  if (e < E) {
    int off = incl - total;
    counts[e] = total;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = incl;
    int run = off;
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = blk_cnt[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        blk_cnt[static_cast<size_t>(b + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; b < nblk; ++b) {
      const size_t at = static_cast<size_t>(b) * E + e;
      const int c = blk_cnt[at];
      blk_cnt[at] = run;
      run += c;
    }
  }
}

// One block (256 threads) per token.  VEC = 16-byte chunks of a row.
template <int PREC>
__global__ __launch_bounds__(256) void scatter_kernel(
    int T, int h, int E, int k, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ local_rank,
    const void* __restrict__ X, int32_t* __restrict__ dst_row, int32_t* __restrict__ src_tok,
    void* __restrict__ Xp, void* __restrict__ xp_scale_v, void* __restrict__ Xq,
    void* __restrict__ x_scale_v) {
  __shared__ int32_t s_dst[kMaxTopk];
  __shared__ float s_red[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    const int i = t * k + tid;
    const int e = ids[i];
    int d = -1;
    if (e >= 0 && e < E) {
      d = blk_base[static_cast<size_t>(i / kPermChunk) * E + e] + local_rank[i];
      src_tok[d] = t;
    }
    dst_row[i] = d;
    s_dst[tid] = d;
  }
  if (PREC == MOE_PREC_MXFP8 || PREC == MOE_PREC_MXFP4) {
    // MX: groups of 32 along h share an E8M0 scale, exponent floor(log2
    // amax) - emax (8 for e4m3, 2 for e2m1); 4 consecutive threads hold a
    // group's 32 values (8 each) and exchange their amax by xor shuffles;
    // codes = RNE_sat(x * 2^(127-code)).  e2m1 codes go two per byte.
    constexpr bool F4 = PREC == MOE_PREC_MXFP4;
    constexpr int EMAX = F4 ? 2 : 8;
    const size_t rb = F4 ? h / 2 : h;  // bytes of a quantised row
    __syncthreads();
    const uint16_t* xr = static_cast<const uint16_t*>(X) + static_cast<size_t>(t) * h;
    uint8_t* xq = static_cast<uint8_t*>(Xq) + static_cast<size_t>(t) * rb;
    uint8_t* xs = static_cast<uint8_t*>(x_scale_v) + static_cast<size_t>(t) * (h / 32);
    uint8_t* xps = static_cast<uint8_t*>(xp_scale_v);
    // the 4 threads of a group always make the same trips (h % 32 == 0)
    for (int c = tid * 8; c < h; c += 256 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(w[q] << 16);
        f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF);
      const uint32_t code = static_cast<uint32_t>(e > EMAX ? e - EMAX : 0);
      const float inv = __uint_as_float((254u - code) << 23);  // 2^(127 - code)
      const bool lead = (tid & 3) == 0;
      if (lead) xs[c / 32] = static_cast<uint8_t>(code);
      if constexpr (F4) {
        uint32_t qv = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) qv |= f32_to_e2m1(f[q] * inv) << (4 * q);
        *reinterpret_cast<uint32_t*>(xq + c / 2) = qv;
        for (int j = 0; j < k; ++j) {
          const int d = s_dst[j];
          if (d < 0) continue;
          *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(Xp) + static_cast<size_t>(d) * rb +
                                       c / 2) = qv;
          if (lead) xps[static_cast<size_t>(d) * (h / 32) + c / 32] = static_cast<uint8_t>(code);
        }
      } else {
        const uint2 qv =
            make_uint2(f32x4_to_e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                       f32x4_to_e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
        *reinterpret_cast<uint2*>(xq + c) = qv;
        for (int j = 0; j < k; ++j) {
          const int d = s_dst[j];
          if (d < 0) continue;
          *reinterpret_cast<uint2*>(static_cast<uint8_t*>(Xp) + static_cast<size_t>(d) * rb + c) =
              qv;
          if (lead) xps[static_cast<size_t>(d) * (h / 32) + c / 32] = static_cast<uint8_t>(code);
        }
      }
    }
  } else if (PREC != MOE_PREC_FP8 && PREC != MOE_PREC_INT8) {
    __syncthreads();
    const int esz = (PREC == MOE_PREC_F32) ? 4 : 2;
    const int nvec = h * esz / 16;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(X) +
                                                      static_cast<size_t>(t) * h * esz);
    // the token row is read once here: a non-temporal load (measured 5%
    // faster on the V4-Pro dispatch); the k copies are ordinary stores
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
    for (int v = tid; v < nvec; v += 256) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + v));
      const uint4 val = make_uint4(w[0], w[1], w[2], w[3]);
      for (int j = 0; j < k; ++j) {
        int d = s_dst[j];
        if (d >= 0)
          reinterpret_cast<uint4*>(static_cast<char*>(Xp) + static_cast<size_t>(d) * h * esz)[v] =
              val;
      }
    }
  } else {
    // A8W8: scale = max|x| / Q (1 for a zero row), codes of x / scale: e4m3
    // (Q = 448, RNE, saturating) or int8 (Q = 127, rounded half away from 0)
    constexpr bool I8 = PREC == MOE_PREC_INT8;
    constexpr float Q = I8 ? 127.0f : 448.0f;
    auto enc4 = [](float a, float b, float c, float d) {
      return I8 ? f32x4_to_i8x4(a, b, c, d) : f32x4_to_e4m3x4(a, b, c, d);
    };
    float* xp_scale = static_cast<float*>(xp_scale_v);
    float* x_scale = static_cast<float*>(x_scale_v);
    const uint16_t* xr = static_cast<const uint16_t*>(X) + static_cast<size_t>(t) * h;
    float amax = 0.0f;
    for (int c = tid * 8; c < h; c += 256 * 8) {
      uint4 v = *reinterpret_cast<const uint4*>(xr + c);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[q] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[q] & 0xffff0000u)));
      }
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) s_red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float s = amax > 0.0f ? amax / Q : 1.0f;
    if (tid == 0) x_scale[t] = s;
    if (tid < k && s_dst[tid] >= 0) xp_scale[s_dst[tid]] = s;
    uint8_t* xq = static_cast<uint8_t*>(Xq) + static_cast<size_t>(t) * h;
    for (int c = tid * 8; c < h; c += 256 * 8) {
      uint4 v = *reinterpret_cast<const uint4*>(xr + c);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t lo = enc4(__uint_as_float(w[0] << 16) / s,
                                    __uint_as_float(w[0] & 0xffff0000u) / s,
                                    __uint_as_float(w[1] << 16) / s,
                                    __uint_as_float(w[1] & 0xffff0000u) / s);
      uint32_t hi = enc4(__uint_as_float(w[2] << 16) / s,
                                    __uint_as_float(w[2] & 0xffff0000u) / s,
                                    __uint_as_float(w[3] << 16) / s,
                                    __uint_as_float(w[3] & 0xffff0000u) / s);
      uint2 q = make_uint2(lo, hi);
      *reinterpret_cast<uint2*>(xq + c) = q;
      for (int j = 0; j < k; ++j) {
        int d = s_dst[j];
        if (d >= 0)
          *reinterpret_cast<uint2*>(static_cast<uint8_t*>(Xp) + static_cast<size_t>(d) * h + c) =
              q;
      }
    }
  }
}

// The row maps alone (the dispatch without its row copies, for a consumer
// that gathers the token rows itself): one thread per assignment i = t k + j,
// the same destination row as scatter_kernel gives it.
__global__ __launch_bounds__(256) void row_maps_kernel(int n, int k, int E,
                                                       const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ blk_base,
                                                       const int32_t* __restrict__ local_rank,
                                                       int32_t* __restrict__ dst_row,
                                                       int32_t* __restrict__ src_tok) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = ids[i];
  int d = -1;
  if (e >= 0 && e < E) {
    d = blk_base[static_cast<size_t>(i / kPermChunk) * E + e] + local_rank[i];
    src_tok[d] = i / k;
  }
  dst_row[i] = d;
}

__global__ void clear_flag_kernel(int32_t* flag) { flag[0] = 0; }

// The device address of this device's `scratch` (in host code the array's
// name is only a stand-in), looked up once per device, with it current.
constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_of_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (q == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<char*>(q);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_permute_no_alloc(PermuteArgs a, hipStream_t stream) {
  if (static_cast<long long>(a.T) * a.k > MOE_NO_ALLOC_MAX_ASSIGNMENTS || a.E > kMaxExperts)
    return hipErrorInvalidValue;
  char* s = nullptr;
  hipError_t e = scratch_of_current_device(&s);
  if (e != hipSuccess) return e;
  a.flag = reinterpret_cast<int32_t*>(s);
  a.blk_cnt = reinterpret_cast<int32_t*>(s + kNoAllocFlagBytes);
  a.local_rank = reinterpret_cast<int32_t*>(s + kNoAllocFlagBytes + kNoAllocBlkBytes);
  // the flag is written by the scan kernel (no memset node under graph
  // capture); the counts, ranks and error bytes are written whole by every
  // call before they are read
  a.clear_flag = 1;
  return launch_permute(a, stream);
}

hipError_t launch_clear_flag(int32_t* flag, hipStream_t stream) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, stream, flag);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int n = a.T * a.k;
  // the per-block error bytes follow the flag word in its region
  uint8_t* blk_err = reinterpret_cast<uint8_t*>(a.flag + 1);
  hipLaunchKernelGGL(count_rank_kernel, dim3(a.nblk), dim3(kPermThreads), 0, stream, a.ids, n,
                     a.E, a.blk_cnt, a.local_rank, blk_err);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kMaxExperts), 0, stream, a.nblk, a.E, a.blk_cnt,
                     a.counts, a.offsets, blk_err, a.flag, a.clear_flag);
  if (a.maps_only) {
    hipLaunchKernelGGL(row_maps_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, n, a.k, a.E,
                       a.ids, a.blk_cnt, a.local_rank, a.dst_row, a.src_tok);
    return hipGetLastError();
  }
  switch (a.precision) {
    case MOE_PREC_F32:
      hipLaunchKernelGGL(scatter_kernel<MOE_PREC_F32>, dim3(a.T), dim3(256), 0, stream, a.T, a.h,
                         a.E, a.k, a.ids, a.blk_cnt, a.local_rank, a.X, a.dst_row, a.src_tok, a.Xp,
                         a.xp_scale, a.Xq, a.x_scale);
      break;
    case MOE_PREC_BF16:
      hipLaunchKernelGGL(scatter_kernel<MOE_PREC_BF16>, dim3(a.T), dim3(256), 0, stream, a.T, a.h,
                         a.E, a.k, a.ids, a.blk_cnt, a.local_rank, a.X, a.dst_row, a.src_tok, a.Xp,
                         a.xp_scale, a.Xq, a.x_scale);
      break;
    case MOE_PREC_MXFP4:
      hipLaunchKernelGGL(scatter_kernel<MOE_PREC_MXFP4>, dim3(a.T), dim3(256), 0, stream, a.T,
                         a.h, a.E, a.k, a.ids, a.blk_cnt, a.local_rank, a.X, a.dst_row, a.src_tok,
                         a.Xp, a.xp_scale, a.Xq, a.x_scale);
      break;
    case MOE_PREC_MXFP8:
      hipLaunchKernelGGL(scatter_kernel<MOE_PREC_MXFP8>, dim3(a.T), dim3(256), 0, stream, a.T,
                         a.h, a.E, a.k, a.ids, a.blk_cnt, a.local_rank, a.X, a.dst_row, a.src_tok,
                         a.Xp, a.xp_scale, a.Xq, a.x_scale);
      break;
    case MOE_PREC_INT8:
      hipLaunchKernelGGL(scatter_kernel<MOE_PREC_INT8>, dim3(a.T), dim3(256), 0, stream, a.T, a.h,
                         a.E, a.k, a.ids, a.blk_cnt, a.local_rank, a.X, a.dst_row, a.src_tok, a.Xp,
                         a.xp_scale, a.Xq, a.x_scale);
      break;
    default:
      hipLaunchKernelGGL(scatter_kernel<MOE_PREC_FP8>, dim3(a.T), dim3(256), 0, stream, a.T, a.h,
                         a.E, a.k, a.ids, a.blk_cnt, a.local_rank, a.X, a.dst_row, a.src_tok, a.Xp,
                         a.xp_scale, a.Xq, a.x_scale);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
