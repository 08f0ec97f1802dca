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
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;                  // K elements per LDS tile
constexpr int kARow = kBK * 2 + 16;      // bytes per padded token row

typedef __attribute__((ext_vector_type(8))) short i16x8_t;

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
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

// ------------------------------------------------------------ DMA gate GEMM
// bf16, E a multiple of 128 (E <= 512): a block of 8 waves owns BM (64 or
// 128) tokens and all E experts over one K range.  K-stages of 32 go global -> LDS by
// asynchronous DMA (global_load_lds_dwordx4) into a 3-stage ring with the
// waits written out (s_waitcnt vmcnt for the later stages, then s_barrier):
// token rows as 64-byte pieces, gate-weight rows ([h, E], E contiguous) as
// they are, read as MFMA B fragments by the transposing ds_read_b64_tr_b16.
// The waves split the tile 2 (tokens) x 4 (experts); each multiplies its
// BM / 64 x E / 128 tiles of 32 x 32 with two v_mfma_f32_32x32x16_bf16 per stage (a lane holds row or
// column lane % 32 at K 16 kh + 8 (lane / 32) + 0..7 of half kh, the same in
// A and B, so the instruction's own K order does not matter).  XOR chunk
// swizzles: token rows (r >> 2) & 3, weight rows 4 (r % 4) (a transposing
// read's half covers 4 consecutive K rows x 4 chunks; the XOR keeps a chunk
// inside its aligned group of 16, so rows of E / 8 chunks work).  Every block
// writes its fp32 partial logits part[split][t][e]; route_topk_kernel sums
// the splits and routes.
// The ring is as deep as 140 KB of LDS allows (up to 6 stages): a block
// streams its gate-weight slice from L2 and its token rows from HBM at
// latencies that only many stages in flight cover.  Block (0, 0) clears the
// device error flag first (route_topk_kernel, which runs after, may set it).
template <int EP, int BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void gate_dma_kernel(RouteArgs a, int kchunk, float* __restrict__ part) {
  constexpr int BK = 32, NW = 8, WN = 4;
  constexpr int MT = BM / 64;  // 32-row MFMA tiles per wave (2 x 4 waves)
  constexpr int STAGE_BYTES = BM * BK * 2 + BK * EP * 2;
  constexpr int STAGES = (143360 / STAGE_BYTES) < 6 ? (143360 / STAGE_BYTES) : 6;
  constexpr int NTW = EP / (32 * WN);  // 32-column MFMA tiles per wave
  constexpr int A_ROW = BK * 2;        // bytes of a token row piece
  constexpr int B_ROW = EP * 2;        // bytes of a gate-weight K row
  constexpr int A_BYTES = BM * A_ROW;
  constexpr int B_BYTES = BK * B_ROW;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTS = A_BYTES / 1024;
  constexpr int B_INSTS = B_BYTES / 1024;
  constexpr int INSTS = A_INSTS + B_INSTS;
  constexpr int MAX_OPS = (INSTS + NW - 1) / NW;
  constexpr int B_CHUNKS = B_ROW / 16;  // 16-byte chunks of a weight row
  static_assert(EP % 128 == 0 && EP <= 512 && B_CHUNKS % 16 == 0, "expert columns");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "DMA granularity");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.flag[0] = 0;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int wm = wave / WN, wn = wave % WN;
  const int T = a.T, h = a.h, E = a.E;
  const int m0 = blockIdx.x * BM;
  const int split = blockIdx.y;
  const int k0 = split * kchunk;
  const int KT = kchunk / BK;
  const size_t x_ld = static_cast<size_t>(h) * 2;
  const size_t w_ld = static_cast<size_t>(E) * 2;
  // DMA: instruction q of a stage (q < A_INSTS: token rows, else weight rows)
  // is issued by wave q % NW; this wave's per-lane source offsets
  const char* a_base = uniform_ptr(static_cast<const char*>(a.X) + static_cast<size_t>(m0) * x_ld +
                                   static_cast<size_t>(k0) * 2);
  const char* b_base = uniform_ptr(static_cast<const char*>(a.Wg) + static_cast<size_t>(k0) * w_ld);
  uint32_t voff[MAX_OPS];
  int ops = 0;
#pragma unroll
  for (int i = 0; i < MAX_OPS; ++i) {
    const int q = wave + i * NW;
    voff[i] = 0;
    if (q < A_INSTS) {
      const int r = q * (1024 / A_ROW) + lane / 4;
      const int c = (lane % 4) ^ ((r >> 2) & 3);
      voff[i] = static_cast<uint32_t>(min(m0 + r, T - 1) - m0) * static_cast<uint32_t>(x_ld) + c * 16;
      ++ops;
    } else if (q < INSTS) {
      const int s = (q - A_INSTS) * 64 + lane;
      const int r = s / B_CHUNKS;
      const int c = (s % B_CHUNKS) ^ (4 * (r & 3));
      voff[i] = static_cast<uint32_t>(r) * static_cast<uint32_t>(w_ld) + c * 16;
      ++ops;
    }
  }
  // DMA i of this wave for stage kt into ring slot `slot` (scalar LDS target)
  const uint32_t lds0 = lds_address(smem);
  auto issue_op = [&](int kt, int slot, int i) {
    const uint32_t st = lds0 + slot * STAGE;
    const int q = wave + i * NW;
    if (q < A_INSTS)
      dma16_at(a_base + static_cast<size_t>(kt) * A_ROW, voff[i], st + q * 1024);
    else if (q < INSTS)
      dma16_at(b_base + static_cast<size_t>(kt) * BK * w_ld, voff[i], st + q * 1024);
  };
  auto issue = [&](int kt, int slot) {
#pragma unroll
    for (int i = 0; i < MAX_OPS; ++i) issue_op(kt, slot, i);
  };
  // with INSTS a multiple of the wave count every wave issues MAX_OPS DMAs
  // per stage and the vmcnt waits are constants
  constexpr bool EVEN = INSTS % NW == 0;
  // fragment offsets (within a stage): A rows wm * BM / 2 + 32 i + lane % 32;
  // B columns of this wave's NTW tiles
  int a_off[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int ar = wm * (BM / 2) + 32 * i + (lane & 31);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      a_off[i][kh] = ar * A_ROW + (((2 * kh + (lane >> 5)) ^ ((ar >> 2) & 3)) << 4);
  }
  int b_off[NTW][4];
  {
    const int g = lane >> 4, p = lane & 15;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int col0 = wn * (EP / WN) + j * 32;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r = 16 * kh + 8 * (g >> 1) + 4 * hh + (p >> 2);
          const int col = col0 + 16 * (g & 1) + (p & 3) * 4;
          b_off[j][2 * kh + hh] = A_BYTES + r * B_ROW + (((col >> 3) ^ (4 * (r & 3))) << 4) + (col & 7) * 2;
        }
    }
  }
  f32x16_t acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x16_t{};
  auto tr_pair = [](const char* st, int o0, int o1) {
    const i16x4_t lo4 = ds_read_tr16(st + o0);
    const i16x4_t hi4 = ds_read_tr16(st + o1);
    const i16x8_t v = i16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };
  // the stage's MFMAs; with EVEN, this wave's DMAs of stage ikt (slot islot;
  // none if !more) go out one after each of the first MAX_OPS tile products:
  // a DMA can stall at issue while the memory pipeline is full, and ahead
  // of the MFMAs it would hold them back
  auto compute = [&](int slot, bool more, int ikt, int islot) {
    if (!EVEN && more) issue(ikt, islot);
    const char* st = smem + slot * STAGE;
    bf16x8_t bk0[NTW], bk1[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      bk0[j] = tr_pair(st, b_off[j][0], b_off[j][1]);
      bk1[j] = tr_pair(st, b_off[j][2], b_off[j][3]);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const bf16x8_t ak0 = *reinterpret_cast<const bf16x8_t*>(st + a_off[i][0]);
      const bf16x8_t ak1 = *reinterpret_cast<const bf16x8_t*>(st + a_off[i][1]);
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak0, bk0[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak1, bk1[j], acc[i][j], 0, 0, 0);
        const int idx = i * NTW + j;
        if (EVEN && idx < MAX_OPS && more) issue_op(ikt, islot, idx);
      }
    }
  };
  static_assert(!EVEN || MT * NTW >= MAX_OPS, "a tile product per DMA");
  // K loop, unrolled by STAGES so that every slot is a constant LDS range
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);
  for (int kt0 = 0; kt0 < KT; kt0 += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      const int kt = kt0 + s;
      if (kt < KT) {
        if constexpr (EVEN)
          wait_after<MAX_OPS, STAGES - 2>(KT - 1 - kt);
        else
          wait_vmcnt_rt(min(STAGES - 2, KT - 1 - kt) * ops);
        __builtin_amdgcn_s_barrier();
        compute(s, kt + STAGES - 1 < KT, kt + STAGES - 1, (s + STAGES - 1) % STAGES);
      }
    }
  }
  // partial logits: element v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4
  // of the wave's 32 rows, column l % 32 of tile j
  float* out = part + static_cast<size_t>(split) * T * E;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int e = wn * (EP / WN) + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = m0 + wm * (BM / 2) + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (t < T) out[static_cast<size_t>(t) * E + e] = acc[i][j][v];
      }
    }
}

// Routing of 4 tokens per wave (one wave per block, so that the blocks
// spread over every CU), 16 lanes per token.  E equals EP here (the DMA gate
// GEMM runs only for E a multiple of 128 up to 512, one instance per E).  Lane
// p of a token's group holds the 4 experts 64 q + 4 p + c (c < 4) of every
// 64-expert group q, in slot 4 q + c, so that its loads of partial logits
// are 16 bytes each.  Logits are the split partials summed in
// split order (+ the gating bias); affinity, key = a + beta; k rounds of a
// 16-lane argmax by xor shuffles (key descending, equal keys to the lower
// id), the winner's lane marks it taken; the weights' denominator sums the
// chosen affinities in choice order.  Hash routing reads the choice from
// tid2eid and takes the chosen affinities from their lanes.
template <int EP>
__global__ __launch_bounds__(64) void route_topk_kernel(RouteArgs a, int splits,
                                                        const float* __restrict__ part) {
  constexpr int G = EP / 64;  // 64-expert groups
  constexpr int Q = 4 * G;    // experts per lane
  static_assert(Q <= 32, "experts per lane");
  const int lane = threadIdx.x & 63;
  const int p = lane & 15;
  const int t = blockIdx.x * 4 + (lane >> 4);  // one wave (4 tokens) per block
  const int T = a.T, k = a.k;
  const bool live = t < T;  // not wave-uniform: every lane takes part in the shuffles
  const bool hash = (a.token_ids != nullptr && a.tid2eid != nullptr);
  const size_t tt = live ? t : 0;
  auto ld4 = [&](const float* row, int g) {
    return *reinterpret_cast<const f32x4_t*>(row + 64 * g + 4 * p);
  };
  float av[Q], key[Q];
#pragma unroll
  for (int s = 0; s < Q; ++s) av[s] = 0.0f;
  // four splits at a time, every load of the four issued before any add;
  // the adds go in split order
  int sp = 0;
  for (; sp + 3 < splits; sp += 4) {
    f32x4_t v[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* r = part + (static_cast<size_t>(sp + u) * T + tt) * EP;
#pragma unroll
      for (int g = 0; g < G; ++g) v[u][g] = ld4(r, g);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) av[4 * g + c] += v[u][g][c];
  }
  for (; sp < splits; ++sp) {
    const float* r = part + (static_cast<size_t>(sp) * T + tt) * EP;
    f32x4_t v0[G];
#pragma unroll
    for (int g = 0; g < G; ++g) v0[g] = ld4(r, g);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) av[4 * g + c] += v0[g][c];
  }
  if (a.gate_bias) {
#pragma unroll
    for (int s = 0; s < Q; ++s) av[s] += a.gate_bias[64 * (s >> 2) + 4 * p + (s & 3)];
  }
  // affinities with the hardware exp2 and reciprocal (a few ulp; the keys
  // stay within 1e-6 of the exact values)
  if (a.score_fn == MOE_SCORE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < Q; ++s) m = fmaxf(m, av[s]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    float z = 0.0f;
#pragma unroll
    for (int s = 0; s < Q; ++s) {
      av[s] = __expf(av[s] - m);
      z += av[s];
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 16);
    const float rz = __builtin_amdgcn_rcpf(z);
#pragma unroll
    for (int s = 0; s < Q; ++s) av[s] = av[s] * rz;
  } else if (a.score_fn == MOE_SCORE_SQRT_SOFTPLUS) {
#pragma unroll
    for (int s = 0; s < Q; ++s) {
      const float l = av[s];
      const float sp1 = l > 0.0f ? l + log1pf(expf(-l)) : log1pf(expf(l));
      av[s] = sqrtf(sp1);
    }
  } else {
#pragma unroll
    for (int s = 0; s < Q; ++s) av[s] = __builtin_amdgcn_rcpf(1.0f + __expf(-av[s]));
  }
  const bool use_beta = a.beta && !hash;
#pragma unroll
  for (int s = 0; s < Q; ++s)
    key[s] = av[s] + (use_beta ? a.beta[64 * (s >> 2) + 4 * p + (s & 3)] : 0.0f);
  if (a.keys && live) {
#pragma unroll
    for (int s = 0; s < Q; ++s) a.keys[static_cast<size_t>(t) * EP + 64 * (s >> 2) + 4 * p + (s & 3)] = key[s];
  }
  int my_id = -1;
  float my_a = 0.0f, den = 0.0f;
  if (!hash) {
    // branch-free selection: a taken expert competes with key -inf, which a
    // real key always beats in the group reduction (E >= k)
    uint32_t taken = 0u;
    for (int j = 0; j < k; ++j) {
      float bk = -INFINITY, ba = 0.0f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int s = 0; s < Q; ++s) {
        const int e = 64 * (s >> 2) + 4 * p + (s & 3);
        const float kq = ((taken >> s) & 1u) ? -INFINITY : key[s];
        const bool b = (kq > bk) || (kq == bk && e < bi);
        bk = b ? kq : bk;
        bi = b ? e : bi;
        ba = b ? av[s] : ba;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ok = __shfl_xor(bk, o, 16);
        const int oi = __shfl_xor(bi, o, 16);
        const float oa = __shfl_xor(ba, o, 16);
        if (better(ok, oi, bk, bi)) {
          bk = ok;
          bi = oi;
          ba = oa;
        }
      }
      taken |= (((bi >> 2) & 15) == p) ? (1u << ((4 * (bi >> 6) + (bi & 3)) & 31)) : 0u;
      den += ba;
      if (p == j) {
        my_id = bi;
        my_a = ba;
      }
    }
  } else {
    const int tok = live ? a.token_ids[t] : -1;
    const bool ok_tok = tok >= 0 && tok < a.vocab;
    for (int j = 0; j < k; ++j) {
      int e = ok_tok ? a.tid2eid[static_cast<size_t>(tok) * k + j] : -1;
      if (e < 0 || e >= EP) e = -1;
      const int se = e >= 0 ? 4 * (e >> 6) + (e & 3) : 0;
      float mine = 0.0f;
#pragma unroll
      for (int s = 0; s < Q; ++s)
        if (s == se) mine = av[s];
      float v = __shfl(mine, e >= 0 ? ((e >> 2) & 15) : 0, 16);
      if (e < 0) v = 0.0f;
      den += v;
      if (p == j) {
        my_id = e;
        my_a = v;
      }
    }
    if (live && p < k && my_id < 0) a.flag[0] = 1;
  }
  if (live && p < k) {
    a.ids[static_cast<size_t>(t) * k + p] = my_id;
    const float g = a.renorm ? a.alpha * my_a / den : a.alpha * my_a;
    a.G[static_cast<size_t>(t) * k + p] = (my_id >= 0) ? g : 0.0f;
  }
}

template <int EP>
hipError_t launch_dma_route(const RouteArgs& a, int bm, int splits, hipStream_t stream) {
  if (a.E != EP) return hipErrorInvalidValue;  // route_topk_kernel takes E == EP
  const int mtiles = (a.T + bm - 1) / bm;
  if (bm == 128)
    hipLaunchKernelGGL((gate_dma_kernel<EP, 128>), dim3(mtiles, splits), dim3(512), 0, stream, a,
                       a.h / splits, a.part);
  else
    hipLaunchKernelGGL((gate_dma_kernel<EP, 64>), dim3(mtiles, splits), dim3(512), 0, stream, a,
                       a.h / splits, a.part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_topk_kernel<EP>, dim3((a.T + 3) / 4), dim3(64), 0, stream, a, splits,
                     static_cast<const float*>(a.part));
  return hipGetLastError();
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
  const RoutePlan p = route_plan(a.T, a.h, a.E, a.precision);
  if (p.dma) {
    switch (a.E) {
      case 128: return launch_dma_route<128>(a, p.bm, p.splits, stream);
      case 256: return launch_dma_route<256>(a, p.bm, p.splits, stream);
      case 384: return launch_dma_route<384>(a, p.bm, p.splits, stream);
      default: return launch_dma_route<512>(a, p.bm, p.splits, stream);
    }
  }
  hipError_t e = launch_clear_flag(a.flag, stream);
  if (e != hipSuccess) return e;
  if (p.bm == 64) return launch_bm<64>(a, p.splits, stream);
  return p.bm == 32 ? launch_bm<32>(a, p.splits, stream) : launch_bm<16>(a, p.splits, stream);
}

}  // namespace moe
