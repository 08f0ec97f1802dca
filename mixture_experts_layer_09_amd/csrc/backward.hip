// backward.hip -- the layer's local backward on one GPU (bf16).
//
// The reverse chain of the blog "Megatron-LM 的 MoE 并行" (反向的通信) without
// its collectives: unpermute backward (the upstream gradient dY[t] goes to
// each of the token's k rows, weighted by G[t,j]; dG[t,j] = dY[t] . Yp[row]),
// the experts' dgrad (dX = Ȳ Wᵀ) and wgrad (dW = Xᵀ Ȳ), the SwiGLU backward
// of "Megatron 分布式训练全维度并行技术文档" §1.8 fused into the Linear2
// dgrad, the permute backward summing the k copies, and the router's
// backward through the chosen experts' continuous affinities.
//
// The gate weight is moved off the gradient rows: with U = dY[t] W2[e]ᵀ (the
// Linear2 dgrad of the unweighted row), dA = G U, and since Yp = A W2[e],
// dG = dY[t] . (A W2[e]) = U . A, a row sum that the Linear2 dgrad epilogue
// takes while it holds U and recomputes A for the SwiGLU backward; dW2 =
// Aᵀ (G dY) = (G A)ᵀ dY.  So the backward needs neither Yp nor the Linear2
// forward that makes it, and the rows of dY are copied, not scaled.
//
// Kernels:
//   dgrad_kernel  out[r] = dO[r] W[e]ᵀ over the expert blocks (ragged rows,
//                 as in the forward).  Both operands are K-contiguous rows
//                 (the gradient rows [rows, K] and the weights as stored,
//                 [N, K]), DMA'd to LDS in 32-value K-stages (64-byte rows,
//                 chunk swizzle (r >> 2) & 3) and read as plain 16-byte
//                 fragments of v_mfma_f32_32x32x16_bf16.  Optional epilogue:
//                 the SwiGLU backward, which reads the saved pre-activations.
//   wgrad_kernel  dW[e] = A_eᵀ B_e over the rows of expert e (ragged K).  Both
//                 operands are [rows, dim] (dim contiguous); chunks of 32 rows
//                 are DMA'd to LDS (rows past the expert's block cleared) and
//                 read with the transposing ds_read_b64_tr_b16 as fragments
//                 of v_mfma_f32_32x32x16_bf16.  Tiles are scheduled
//                 statically in groups of 64 per XCD so that the blocks
//                 sharing a chunk read it together; the dW stores are
//                 non-temporal.  An expert without rows gets zeros.
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) short i16x8s_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

__device__ __forceinline__ float bfv(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// ---------------------------------------------------------------- elementwise
// A = SiLU(H1[:, :f]) * H1[:, f:], 8 columns per thread, for `arows` rows:
// Aw = A * grow[r] on the first `rows` (dispatched) rows and A on the rest
// (the shared expert's); Af (may be NULL) = A.
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t* __restrict__ H1, int f,
                                                         long rows, long arows,
                                                         const float* __restrict__ grow,
                                                         uint16_t* __restrict__ Aw,
                                                         uint16_t* __restrict__ Af) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;  // 8-column group
  const long per = f / 8;
  if (i >= arows * per) return;
  const long r = i / per;
  const int c = static_cast<int>(i % per) * 8;
  const float gw = r < rows ? grow[r] : 1.0f;
  const uint4 g = *reinterpret_cast<const uint4*>(H1 + r * 2 * f + c);
  const uint4 u = *reinterpret_cast<const uint4*>(H1 + r * 2 * f + f + c);
  const uint32_t gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
  uint32_t ow[4], of[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a0 = silu(bfv(gv[q] & 0xFFFF)) * bfv(uv[q] & 0xFFFF);
    const float a1 = silu(bfv(gv[q] >> 16)) * bfv(uv[q] >> 16);
    ow[q] = f32_to_bf16(gw * a0) | (static_cast<uint32_t>(f32_to_bf16(gw * a1)) << 16);
    of[q] = f32_to_bf16(a0) | (static_cast<uint32_t>(f32_to_bf16(a1)) << 16);
  }
  *reinterpret_cast<uint4*>(Aw + r * f + c) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  if (Af) *reinterpret_cast<uint4*>(Af + r * f + c) = make_uint4(of[0], of[1], of[2], of[3]);
}

// The gate weight of each dispatched row: grow[dst_row[i]] = G[i].
__global__ __launch_bounds__(256) void row_gate_kernel(const int32_t* __restrict__ dst_row,
                                                       const float* __restrict__ G, int n,
                                                       float* __restrict__ grow) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = dst_row[i];
  if (r >= 0) grow[r] = G[i];
}

// Unpermute backward, one block (256 threads) per token: dYp[row(t,j)] =
// dY[t] for each of its k rows (unweighted: the gate weight goes onto A, and
// dG comes out of the Linear2 dgrad).  h % 8 == 0.
__global__ __launch_bounds__(256) void unpermute_backward_kernel(
    int h, int k, const uint16_t* __restrict__ dY, const int32_t* __restrict__ dst_row,
    uint16_t* __restrict__ dYp) {
  const int t = blockIdx.x;
  const uint16_t* dy = dY + static_cast<size_t>(t) * h;
  for (int c = threadIdx.x * 8; c < h; c += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(dy + c);
    for (int j = 0; j < k; ++j) {
      const int r = dst_row[static_cast<size_t>(t) * k + j];
      if (r >= 0) *reinterpret_cast<uint4*>(dYp + static_cast<size_t>(r) * h + c) = v;
    }
  }
}

// dG[t,j] = the sum of row(t,j)'s P partials, in column order (0 for a
// skipped assignment).
__global__ __launch_bounds__(256) void dg_reduce_kernel(int n, int P, const int32_t* __restrict__ dst_row,
                                                        const float* __restrict__ dgp,
                                                        float* __restrict__ dG) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = dst_row[i];
  float s = 0.0f;
  if (r >= 0) {
    const float* p = dgp + static_cast<size_t>(r) * P;
    for (int q = 0; q < P; ++q) s += p[q];
  }
  dG[i] = s;
}

// Router backward, one wave per token: affinities a from the recomputed keys
// (a + beta, or a for hash routing), the gradient of the mixing weights
// (G_j = alpha a_j / S with renorm, else alpha a_j) onto the chosen experts'
// affinities, then onto the logits: sigmoid a(1 - a), sqrt(softplus)
// sigma(l) / (2a) with sigma(l) = 1 - exp(-a^2), softmax a (da - sum da a).
__global__ __launch_bounds__(256) void route_backward_kernel(
    int T, int E, int k, const float* __restrict__ keys, const float* __restrict__ beta, int hash,
    int score_fn, int renorm, float alpha, const int32_t* __restrict__ ids,
    const float* __restrict__ dG, float* __restrict__ dl32, uint16_t* __restrict__ dl16) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int kQ = kMaxExperts / 64;
  const float* key = keys + static_cast<size_t>(t) * E;
  auto aff = [&](int e) { return key[e] - ((beta && !hash) ? beta[e] : 0.0f); };
  // lane j < k: choice j
  int my_id = 0;
  float my_g = 0.0f, my_a = 0.0f;
  if (lane < k) {
    my_id = ids[static_cast<size_t>(t) * k + lane];
    my_g = dG[static_cast<size_t>(t) * k + lane];
    my_a = (my_id >= 0 && my_id < E) ? aff(my_id) : 0.0f;
  }
  const float S = wave_sum(my_a);
  const float dGa = wave_sum(my_g * my_a);
  float a[kQ], da[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int e = lane + 64 * q;
    a[q] = (e < E) ? aff(e) : 0.0f;
    da[q] = 0.0f;
  }
  for (int j = 0; j < k; ++j) {
    const int id = __shfl(my_id, j, 64);
    const float g = __shfl(my_g, j, 64);
    const float d = renorm ? alpha * (g / S - dGa / (S * S)) : alpha * g;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (lane + 64 * q == id) da[q] += d;
  }
  float sda = 0.0f;
  if (score_fn == MOE_SCORE_SOFTMAX) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) sda += da[q] * a[q];
    sda = wave_sum(sda);
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int e = lane + 64 * q;
    if (e >= E) continue;
    float d;
    if (score_fn == MOE_SCORE_SOFTMAX)
      d = a[q] * (da[q] - sda);
    else if (score_fn == MOE_SCORE_SQRT_SOFTPLUS)
      d = da[q] == 0.0f ? 0.0f : da[q] * (1.0f - expf(-a[q] * a[q])) / (2.0f * a[q]);
    else
      d = da[q] * a[q] * (1.0f - a[q]);
    dl32[static_cast<size_t>(t) * E + e] = d;
    dl16[static_cast<size_t>(t) * E + e] = f32_to_bf16(d);
  }
}

// Permute backward, one block per token: dX[t] = sum_j dXp[row(t,j)] (+ the
// shared expert's row) (+ the router's dl Wgᵀ row), fp32 sums, bf16 out.
__global__ __launch_bounds__(256) void permute_backward_kernel(
    int h, int k, const uint16_t* __restrict__ dXp, const int32_t* __restrict__ dst_row,
    const uint16_t* __restrict__ dXs, const uint16_t* __restrict__ dXr, uint16_t* __restrict__ dX) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < h; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    auto add = [&](const uint16_t* p) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bfv(w[q] & 0xFFFF);
        acc[2 * q + 1] += bfv(w[q] >> 16);
      }
    };
    for (int j = 0; j < k; ++j) {
      const int r = dst_row[static_cast<size_t>(t) * k + j];
      if (r >= 0) add(dXp + static_cast<size_t>(r) * h);
    }
    if (dXs) add(dXs + static_cast<size_t>(t) * h);
    if (dXr) add(dXr + static_cast<size_t>(t) * h);
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = f32_to_bf16(acc[2 * q]) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * q + 1])) << 16);
    *reinterpret_cast<uint4*>(dX + static_cast<size_t>(t) * h + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// tile_off[e+1] = tile_off[e] + ceil(rows_e / BM) for e < E, then the shared
// rows (T_sh); E may be 0 (one plain segment of T_sh rows).
__global__ __launch_bounds__(kMaxExperts) void bwd_tile_offsets_kernel(
    const int32_t* __restrict__ offsets, int E, int T_sh, int BM, int32_t* __restrict__ tile_off) {
  __shared__ int32_t s[kMaxExperts];
  const int e = threadIdx.x;
  s[e] = (e < E) ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {
    const int v = (e >= o) ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) tile_off[e + 1] = s[e];
  if (e == 0) {
    tile_off[0] = 0;
    tile_off[E + 1] = (E > 0 ? s[E - 1] : 0) + (T_sh + BM - 1) / BM;
  }
}

// ---------------------------------------------------------------- dgrad
struct DgradArgs {
  const void* A;      // [rows, K] bf16 gradient rows (segment blocks by offsets)
  const void* A_sh;   // [T, K] shared rows
  const void* W;      // [E, N, K] bf16 (K contiguous)
  const void* W_sh;   // [N, K]
  void* out;          // [rows, N] (SWB: [rows, 2N])
  void* out_sh;
  const void* h1;     // SWB: [rows, 2N] bf16 pre-activations (gate, up)
  const void* h1_sh;
  const float* grow;  // SWB: [rows] gate weight of each routed row
  float* dgp;         // SWB: [rows, N / 64] partial dG per row and 64 columns
  const int32_t* offsets;
  const int32_t* tile_off;
  int E, K, N, T, n_tiles;
};

// The block's (segment, m-tile, n-tile): XCD x = blockIdx % 8 runs one
// contiguous range of items; items go in groups of 1024 / BM m-tiles, n-tile
// major (as the forward's grouped GEMM).
template <int BM>
__device__ __forceinline__ bool dgrad_item(const DgradArgs& g, int& seg, int& mtile, int& nt) {
  constexpr int GROUP_M = 1024 / BM;
  const int E = g.E, NT = g.n_tiles;
  const int total = g.tile_off[E + 1] * NT;
  if (static_cast<int>(blockIdx.x) >= total) return false;
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = total >> 3, rem = total & 7;
  const int item = x * per + min(x, rem) + slot;
  const int mq = item / NT;
  int lo = 0, hi = E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.tile_off[mid] <= mq)
      lo = mid;
    else
      hi = mid - 1;
  }
  seg = lo;
  const int mt_seg = g.tile_off[seg + 1] - g.tile_off[seg];
  const int local = item - g.tile_off[seg] * NT;
  const int grp = local / (GROUP_M * NT);
  const int gsz = min(GROUP_M, mt_seg - grp * GROUP_M);
  const int rin = local - grp * GROUP_M * NT;
  nt = rin / gsz;
  mtile = grp * GROUP_M + rin % gsz;
  return true;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool SWB>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(2)))
void dgrad_kernel(DgradArgs g) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int ROWB = 64;  // 32 bf16 of one row per stage
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTS = A_BYTES / 1024, B_INSTS = B_BYTES / 1024;  // 16 rows per DMA
  constexpr int A_OPS = A_INSTS / NW, B_OPS = B_INSTS / NW;
  // 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16, two per 32-value stage)
  constexpr int WM = BM / WAVES_M, MT = WM / 32, WN = BN / WAVES_N, NTW = WN / 32;
  static_assert(A_INSTS % NW == 0 && B_INSTS % NW == 0, "tiles must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int seg, mtile, nt;
  if (!dgrad_item<BM>(g, seg, mtile, nt)) return;
  const bool shared = (seg == g.E);
  const size_t ld = static_cast<size_t>(g.K) * 2;
  int row0, row_end;
  const char *Abase, *Wbase;
  if (!shared) {
    row0 = g.offsets[seg] + mtile * BM;
    row_end = g.offsets[seg + 1];
    Abase = static_cast<const char*>(g.A);
    Wbase = static_cast<const char*>(g.W) + static_cast<size_t>(seg) * g.N * ld;
  } else {
    row0 = mtile * BM;
    row_end = g.T;
    Abase = static_cast<const char*>(g.A_sh);
    Wbase = static_cast<const char*>(g.W_sh);
  }
  const int rows_valid = min(BM, row_end - row0);
  const int mt_live = __builtin_amdgcn_readfirstlane(max(0, min(MT, (rows_valid - wm * WM + 31) / 32)));
  auto swz = [](int r) { return (r >> 2) & 3; };

  const char* a_base = uniform_ptr(Abase + static_cast<size_t>(row0) * ld);
  const char* b_base = uniform_ptr(Wbase + static_cast<size_t>(nt) * BN * ld);
  uint32_t a_voff[A_OPS], b_voff[B_OPS];
#pragma unroll
  for (int q = 0; q < A_OPS; ++q) {
    const int r = (wave * A_OPS + q) * 16 + lane / 4;
    a_voff[q] = static_cast<uint32_t>(min(r, row_end - 1 - row0)) * static_cast<uint32_t>(ld) +
                ((lane % 4) ^ swz(r)) * 16;
  }
#pragma unroll
  for (int q = 0; q < B_OPS; ++q) {
    const int r = (wave * B_OPS + q) * 16 + lane / 4;
    b_voff[q] = static_cast<uint32_t>(r) * static_cast<uint32_t>(ld) + ((lane % 4) ^ swz(r)) * 16;
  }
  // every wave issues OPS DMAs per stage (A blocks past the segment's last
  // row fetch that row again), so the vmcnt waits are constants; the LDS
  // targets are scalar
  constexpr int OPS = A_OPS + B_OPS;
  const uint32_t lds0 = lds_address(smem);
  auto issue_op = [&](int kt, int slot, int q) {
    const uint32_t st = lds0 + slot * STAGE;
    if (q < A_OPS)
      dma16_at(a_base + static_cast<size_t>(kt) * ROWB, a_voff[q], st + (wave * A_OPS + q) * 1024);
    else
      dma16_at(b_base + static_cast<size_t>(kt) * ROWB, b_voff[q - A_OPS],
               st + A_BYTES + (wave * B_OPS + q - A_OPS) * 1024);
  };
  auto issue = [&](int kt, int slot) {
#pragma unroll
    for (int q = 0; q < OPS; ++q) issue_op(kt, slot, q);
  };

  f32x16_t acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x16_t{};
  // fragments: lane l holds row (or column) l % 32 at K 16 kh + 8 (l / 32)
  // + 0..7 of the stage, i.e. 16-byte chunk 2 kh + l / 32 of the row, for A
  // and W alike; element v of an accumulator is row 8 (v / 4) + 4 (l / 32) +
  // v % 4, column l % 32
  int a_off[MT][2], b_off[NTW][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int ch = 2 * kh + (lane >> 5);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int r = wm * WM + i * 32 + (lane & 31);
      a_off[i][kh] = r * ROWB + ((ch ^ swz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int r = wn * WN + j * 32 + (lane & 31);
      b_off[j][kh] = A_BYTES + r * ROWB + ((ch ^ swz(r)) << 4);
    }
  }
  static_assert(2 * MT * NTW >= OPS, "an MFMA per DMA");
  bf16x8_t bfr[NTW][2], af[MT][2];
  auto load_frags = [&](int slot) {
    const char* st = smem + slot * STAGE;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int j = 0; j < NTW; ++j) bfr[j][kh] = *reinterpret_cast<const bf16x8_t*>(st + b_off[j][kh]);
#pragma unroll
      for (int i = 0; i < MT; ++i) af[i][kh] = *reinterpret_cast<const bf16x8_t*>(st + a_off[i][kh]);
    }
  };
  // Without the SwiGLU backward, the transposed product (weight fragment
  // first): element v of lane l is row l % 32 of the tile and column
  // 8 (v / 4) + 4 (l / 32) + v % 4, stored 4 columns at a time.  With it,
  // element v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column
  // l % 32, the layout the staged SwiGLU-backward epilogue writes to LDS.
  // DMA idx of stage ikt (slot islot; none if !more) goes out after product
  // idx: a DMA can stall at issue while the memory pipeline is full, and
  // ahead of the MFMAs it would hold them back.
  auto mma_issue = [&](bool more, int ikt, int islot) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          acc[i][j] = SWB ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i][kh], bfr[j][kh], acc[i][j], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j][kh], af[i][kh], acc[i][j], 0, 0, 0);
          const int idx = (kh * MT + i) * NTW + j;
          if (idx < OPS && more) issue_op(ikt, islot, idx);
        }
  };

  const int KT = g.K / 32;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);
  const bool live = mt_live > 0;
  // Eight waves: ping-pong.  The two row halves (4 waves each, one of each
  // per SIMD) alternate: half 0 reads stage kt's fragments while half 1
  // multiplies stage kt - 1, then half 0 multiplies while half 1 reads, with
  // two barriers per stage; each half runs its own copy of the loop (the
  // same barriers in the same order).  Half 1 has read stage kt - 1 (and
  // waited for its reads) before the barrier after which that slot is
  // refilled.
  if constexpr (NW == 8 && WAVES_M == 2) {
    if (__builtin_amdgcn_readfirstlane(wm) == 0) {
      for (int k0 = 0; k0 < KT; k0 += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
          const int kt = k0 + s;
          if (kt < KT) {
            wait_after<OPS, STAGES - 2>(KT - 1 - kt);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const bool more = kt + STAGES - 1 < KT;
            if (live) load_frags(s);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (live)
              mma_issue(more, kt + STAGES - 1, (s + STAGES - 1) % STAGES);
            else if (more)
              issue(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
          }
        }
      }
    } else {
      for (int k0 = 0; k0 < KT; k0 += STAGES) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
          const int kt = k0 + s;
          if (kt < KT) {
            wait_after<OPS, STAGES - 2>(KT - 1 - kt);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const bool more = kt + STAGES - 1 < KT;
            if (live && kt > 0)
              mma_issue(more, kt + STAGES - 1, (s + STAGES - 1) % STAGES);
            else if (more)
              issue(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (live) {
              load_frags(s);
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
          }
        }
      }
      if (live) mma_issue(false, 0, 0);
    }
  } else {
    for (int k0 = 0; k0 < KT; k0 += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        const int kt = k0 + s;
        if (kt < KT) {
          // stage kt is in LDS once at most the stages issued after it are in flight
          wait_after<OPS, STAGES - 2>(KT - 1 - kt);
          __builtin_amdgcn_s_barrier();
          if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
          if (live) {
            load_frags(s);
            mma_issue(false, 0, 0);
          }
        }
      }
    }
  }

  // ------------------------------------------------ epilogue
  uint16_t* obase = static_cast<uint16_t*>(shared ? g.out_sh : g.out);
  if constexpr (SWB) {
    // acc = U, the dgrad of the unweighted rows.  Each wave stages its 64 x
    // 64 part of U in LDS (fp32), 32 rows at a time, and reads it back as 8
    // consecutive columns per lane, 8 lanes per row, so that H1 is read and
    // dH1 written in 16-byte pieces of whole 128-byte lines.  Then dA = G U,
    // the SwiGLU backward, and this wave's part of dG = U . A over its 64
    // columns of each row.  Element (r, c) of a staged 32 x 64 block is float
    // r * 64 + (c ^ 32 ((r >> 2) & 1)): the two half-waves of a write, rows
    // r and r + 4, then fall in different banks.
    static_assert(WN == 64 && NW * 8192 <= STAGES * STAGE, "staging: 32 x 64 fp32 per wave");
    __syncthreads();  // every wave is done with the ring
    float* wst = reinterpret_cast<float*>(smem + wave * 8192);
    const uint16_t* hbase = static_cast<const uint16_t*>(shared ? g.h1_sh : g.h1);
    const int P = g.N / 64, pcol = (nt * BN + wn * WN) / 64;
    const int cg = lane & 7;
    const int n0 = nt * BN + wn * WN + 8 * cg;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= mt_live) continue;  // wave-uniform
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), c = 32 * j + (lane & 31);
          wst[r * 64 + (c ^ (((r >> 2) & 1) << 5))] = acc[i][j][v];
        }
      // the wave's LDS operations run in order: once its writes are done,
      // its reads see them (the memory clobber keeps the compiler's order)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = (lane >> 3) + 8 * q;
        const float4* src = reinterpret_cast<const float4*>(wst + rr * 64 + ((8 * cg) ^ (((rr >> 2) & 1) << 5)));
        const float4 u0 = src[0], u1 = src[1];
        const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        const int row = row0 + wm * WM + i * 32 + rr;
        float part = 0.0f;
        if (row < row_end) {
          const float gw = shared ? 1.0f : g.grow[row];
          const size_t rb = static_cast<size_t>(row) * 2 * g.N;
          const uint4 gv = *reinterpret_cast<const uint4*>(hbase + rb + n0);
          const uint4 uv = *reinterpret_cast<const uint4*>(hbase + rb + g.N + n0);
          const uint32_t gq[4] = {gv.x, gv.y, gv.z, gv.w}, uq[4] = {uv.x, uv.y, uv.z, uv.w};
          uint32_t dg[4], du[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float og[2], ou[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              // dH = G U; H1 = (gate x, up y); A = SiLU(x) y: dy = dH SiLU(x)
              // and dx = dH y (sigma(x) + SiLU(x) (1 - sigma(x)))
              const float x = bfv(static_cast<uint16_t>(gq[e] >> (16 * hh)));
              const float y = bfv(static_cast<uint16_t>(uq[e] >> (16 * hh)));
              const float un = u[2 * e + hh], d = gw * un;
              const float sg = 1.0f / (1.0f + expf(-x));
              const float act = x * sg;
              og[hh] = d * y * (sg + act * (1.0f - sg));
              ou[hh] = d * act;
              // A as the forward's Linear2 multiplied it (bf16)
              part = fmaf(un, bfv(f32_to_bf16(act * y)), part);
            }
            dg[e] = pack_bf16x2(og[0], og[1]);
            du[e] = pack_bf16x2(ou[0], ou[1]);
          }
          *reinterpret_cast<uint4*>(obase + rb + n0) = make_uint4(dg[0], dg[1], dg[2], dg[3]);
          *reinterpret_cast<uint4*>(obase + rb + g.N + n0) = make_uint4(du[0], du[1], du[2], du[3]);
        }
        // the row's partial over its 8 lanes (every lane takes part)
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        if (!shared && cg == 0 && row < row_end) g.dgp[static_cast<size_t>(row) * P + pcol] = part;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
    }
    return;
  }
  // lane l holds row l % 32 of row tile i; 4 consecutive columns
  // 8 q + 4 (l / 32) + 0..3 of each n-tile leave as one 8-byte store
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i >= mt_live) continue;  // wave-uniform
    const int row = row0 + wm * WM + i * 32 + (lane & 31);
    if (row >= row_end) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int n = nt * BN + wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          w[e] = static_cast<uint32_t>(f32_to_bf16(acc[i][j][4 * q + 2 * e])) |
                 (static_cast<uint32_t>(f32_to_bf16(acc[i][j][4 * q + 2 * e + 1])) << 16);
        *reinterpret_cast<uint2*>(obase + static_cast<size_t>(row) * g.N + n) = make_uint2(w[0], w[1]);
      }
    }
  }
}

// ---------------------------------------------------------------- wgrad
struct WgradArgs {
  const void* A;     // [rows, M] bf16 (routed rows in expert blocks)
  const void* A_sh;  // [T, M]
  const void* B;     // [rows, N]
  const void* B_sh;  // [T, N]
  void* out;         // [E, M, N] bf16
  void* out_sh;      // [M, N]
  const int32_t* offsets;
  int E, M, N, T, has_shared;
  int strip_rows;  // routed segments of at most this many rows go to wgrad_strip_kernel (-1: none)
};

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63] (binary dispatch).
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID)
      wait_vm_range<LO, MID>(n);
    else
      wait_vm_range<MID + 1, HI>(n);
  }
}

// Swizzle of 16-byte chunks in a [rows][W] bf16 tile read by
// ds_read_b64_tr_b16 for 32x32 fragments (as the forward's B tiles): half a
// read is 4 consecutive K rows x 4 chunks, which must fall on distinct
// banks.  256-byte rows (CH = 16 chunks) all start on bank 0: XOR by
// 4 (r % 4).  128-byte rows (CH = 8): rows r and r + 1 already use opposite
// bank halves, so rows r and r + 2 get chunk sets 4 apart.
template <int CH>
__device__ __forceinline__ int wg_swz(int r) {
  return CH >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// dW[e] = A_eᵀ B_e, A_e and B_e the rows of segment e (the shared expert's
// segment: all T rows of A_sh and B_sh).  The 128 x BN output tiles of a
// segment are taken in groups of 8 m-tiles by 8 n-tiles, and the groups of
// all segments, shared expert first, are dealt round-robin to the 8 XCDs.
// Block b runs on XCD b % 8 and takes tile b / 8 of every group its XCD
// holds (m-tile (b / 8) % 8, n-tile b / 64 inside it): the 64 blocks of
// an XCD work through one group at a time, over the same rows at about the
// same time, so the 8 blocks that read a 32-row chunk of A or B do so while
// it is in that XCD's L2.  A block's tiles form one flat sequence of 32-row
// K chunks (a segment without rows counts one empty chunk), DMA'd into a
// STAGES-deep LDS ring; a chunk's rows past the segment are cleared in LDS
// before use.  v_mfma_f32_32x32x16_bf16, first operand the B tile (n), second
// the A tile (m).  A finished tile is staged, swizzled, in the ring stage
// just multiplied and leaves as non-temporal 16-byte stores of whole rows.
template <int BN, int STAGES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void wgrad_kernel(WgradArgs g) {
  constexpr int BM = 128, KC = 32;
  constexpr int TILE = KC * BM * 2;      // A: 8 KB
  constexpr int TILE_B = KC * BN * 2;    // B: 8 or 4 KB
  constexpr int STAGE = TILE + TILE_B;
  constexpr int A_OPS = TILE / 1024 / 4;    // A DMAs per wave per chunk
  constexpr int BCH = BN / 8;            // B chunks per row
  constexpr int B_RPI = 1024 / (BN * 2); // B rows per DMA instruction
  constexpr int B_OPS = TILE_B / 1024 / 4;  // B DMAs per wave per chunk
  constexpr int NB = BN / 64;            // 32-column n blocks per wave
  static_assert(BN == 256 || BN == 128 || BN == 64, "n-tile width");
  constexpr int OCH = BN / 8;                 // 16-byte chunks of an output row
  // a finished tile is staged in NPH phases of PR rows: halves, or quarters
  // where half a tile is more than a ring stage
  constexpr int NPH = (BM / 2) * BN * 2 <= STAGE ? 2 : 4;
  constexpr int PR = BM / NPH;
  constexpr int NSH = PR * OCH / 256;         // 16-byte stores of a phase, per thread
  constexpr int NST = NPH * NSH;
  constexpr int OPS = A_OPS + B_OPS;          // DMAs of one chunk, per wave
  static_assert((STAGES - 2) * OPS + (STAGES - 1) * NST <= 63, "vmcnt range");
  static_assert(PR * BN * 2 <= STAGE, "a staging phase fits in one ring stage");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves of 64 x BN / 2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;  // 512 blocks: 64 per XCD
  const int MTt = g.M / BM, NTt = g.N / BN;
  const int ngm = (MTt + 7) / 8, ngn = (NTt + 7) / 8;  // a segment's groups: ngm x ngn
  const int nseg = g.E + (g.has_shared ? 1 : 0);
  const int sm = slot & 7, sn = slot >> 3;  // this block's tile in a group
  const uint32_t lda = static_cast<uint32_t>(g.M) * 2, ldb = static_cast<uint32_t>(g.N) * 2;

  // position in the block's sequence: group (gm, gn) of segment sg (the
  // shared expert's first), whose tile for this block is m-tile 8 gm + sm,
  // n-tile 8 gn + sn of segment seg, and its chunk kc of nkc, which starts
  // at A row a and B row b with rem rows left in the segment.  This XCD's
  // groups are every 8th in (sg, gm, gn) order, so the walk is additions
  // with carries (no divisions in the loop).
  struct Cur {
    int sg, gm, gn, seg, nkc, kc, rem;  // sg >= nseg: past the end
    const char* a;
    const char* b;
  };
  auto carry = [&](Cur c) -> Cur {
    while (c.gn >= ngn) {
      c.gn -= ngn;
      ++c.gm;
    }
    while (c.gm >= ngm) {
      c.gm -= ngm;
      ++c.sg;
    }
    return c;
  };
  // from group (sg, gm, gn) on, this XCD's first group with a tile for this
  // block (a segment's last row or column of groups may be short), skipping
  // the routed segments that wgrad_strip_kernel takes
  auto settle = [&](Cur c) -> Cur {
    int k0 = 0, k1 = g.T;
    bool sh = false;
    for (;;) {
      if (c.sg >= nseg) return c;
      if (c.gm * 8 + sm < MTt && c.gn * 8 + sn < NTt) {
        sh = g.has_shared && c.sg == 0;
        c.seg = sh ? g.E : c.sg - (g.has_shared ? 1 : 0);
        k0 = 0;
        k1 = g.T;
        if (!sh)  // (the pointer made explicitly wave-uniform: an operand of a scalar load)
          scalar_load2(reinterpret_cast<const int32_t*>(
                           uniform_ptr(reinterpret_cast<const char*>(g.offsets + c.seg))),
                       k0, k1);
        if (sh || k1 - k0 > g.strip_rows) break;
        // on to this XCD's first group past the segment
        const int left = ngm * ngn - (c.gm * ngn + c.gn);
        c.gn += 8 * ((left + 7) / 8);
        c = carry(c);
        continue;
      }
      c.gn += 8;
      c = carry(c);
    }
    c.rem = k1 - k0;
    c.nkc = max(1, (c.rem + KC - 1) / KC);
    c.kc = 0;
    if (c.rem == 0) k0 = 0;  // no rows: the chunk's DMA reads row 0 (not multiplied)
    c.a = static_cast<const char*>(sh ? g.A_sh : g.A) + static_cast<size_t>(k0) * lda +
          static_cast<size_t>(c.gm * 8 + sm) * BM * 2;
    c.b = static_cast<const char*>(sh ? g.B_sh : g.B) + static_cast<size_t>(k0) * ldb +
          static_cast<size_t>(c.gn * 8 + sn) * BN * 2;
    return c;
  };
  auto advance = [&](Cur c) -> Cur {
    if (++c.kc < c.nkc) {
      c.rem -= KC;
      c.a += static_cast<size_t>(KC) * lda;
      c.b += static_cast<size_t>(KC) * ldb;
      return c;
    }
    c.gn += 8;
    return settle(carry(c));
  };

  // DMA of one chunk: A 8 instructions of 4 rows x 256 B (2 per wave), B 8 or
  // 4 of 4 or 8 rows (2 or 1 per wave), each lane one swizzled 16-byte piece.
  // Rows past the chunk's valid ones repeat its last valid row; a segment
  // without rows reads row 0 (the chunk is not multiplied).
  uint32_t a_off[A_OPS], b_off[B_OPS];  // a full chunk's per-lane offsets
#pragma unroll
  for (int q = 0; q < A_OPS; ++q) {
    const int r = (wave * A_OPS + q) * 4 + lane / 16;
    a_off[q] = r * lda + (((lane & 15) ^ wg_swz<16>(r)) << 4);
  }
#pragma unroll
  for (int q = 0; q < B_OPS; ++q) {
    const int r = (wave * B_OPS + q) * B_RPI + lane / BCH;
    b_off[q] = r * ldb + (((lane % BCH) ^ wg_swz<BCH>(r)) << 4);
  }
  const uint32_t lds0 = lds_address(smem);
  auto issue = [&](Cur c, int st) {
    const int kv = max(1, min(KC, c.rem));
    const uint32_t dst = lds0 + st * STAGE;
    if (kv == KC) {
#pragma unroll
      for (int q = 0; q < A_OPS; ++q) dma16_at(c.a, a_off[q], dst + (wave * A_OPS + q) * 1024);
#pragma unroll
      for (int q = 0; q < B_OPS; ++q) dma16_at(c.b, b_off[q], dst + TILE + (wave * B_OPS + q) * 1024);
    } else {
#pragma unroll
      for (int q = 0; q < A_OPS; ++q) {
        const int r = (wave * A_OPS + q) * 4 + lane / 16;
        const uint32_t rr = static_cast<uint32_t>(min(r, kv - 1));
        dma16_at(c.a, rr * lda + (((lane & 15) ^ wg_swz<16>(r)) << 4), dst + (wave * A_OPS + q) * 1024);
      }
#pragma unroll
      for (int q = 0; q < B_OPS; ++q) {
        const int r = (wave * B_OPS + q) * B_RPI + lane / BCH;
        const uint32_t rr = static_cast<uint32_t>(min(r, kv - 1));
        dma16_at(c.b, rr * ldb + (((lane % BCH) ^ wg_swz<BCH>(r)) << 4), dst + TILE + (wave * B_OPS + q) * 1024);
      }
    }
  };
  // v_mfma_f32_32x32x16_bf16 fragments (8 K-consecutive values per lane) by
  // transposing reads: 32 columns from col0 and the 16 K rows from 16 kh;
  // lane group g = lane / 16 reads rows 8 (g >> 1) + 4 h + p / 4 of the 16
  // columns from col0 + 16 (g & 1), so lane l holds column col0 + l % 32 at
  // K rows 16 kh + 8 (l / 32) + 0..7 (the same for both operands).  The
  // per-lane offsets inside a stage are computed once.
  const int kgr = lane >> 4, p = lane & 15;
  auto toff = [&](int col0, int kh, int h, int W) {
    const int r = 16 * kh + 8 * (kgr >> 1) + 4 * h + (p >> 2);
    const int col = col0 + 16 * (kgr & 1) + (p & 3) * 4;
    const int sw = W >= 128 ? wg_swz<16>(r) : wg_swz<8>(r);  // 256 or 512-byte rows alike
    return r * W * 2 + (((col >> 3) ^ sw) << 4) + (col & 7) * 2;
  };
  int offB[2][NB][2], offA[2][2][2];  // [kh][block][h]
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < NB; ++i) offB[kh][i][h] = TILE + toff(wn * (BN / 2) + i * 32, kh, h, BN);
#pragma unroll
      for (int j = 0; j < 2; ++j) offA[kh][j][h] = toff(wm * 64 + j * 32, kh, h, 128);
    }
  auto frag = [&](const char* base, int o0, int o1) {
    const i16x4_t lo4 = ds_read_tr16(base + o0);
    const i16x4_t hi4 = ds_read_tr16(base + o1);
    const i16x8s_t v = i16x8s_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };

  // acc[i][j]: the 32 x 32 block (n block i, m block j); lane l holds m =
  // l % 32 and, in elements 4 q .. 4 q + 3, the 4 consecutive n from
  // 8 q + 4 (l / 32)
  f32x16_t acc[NB][2];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  };
  // a finished tile, in two halves of 64 rows (the waves with wm = 0, then
  // wm = 1): acc -> swizzled staging rows in the ring stage just multiplied
  // (its next DMA is issued after the step's barrier) -> 16-byte stores of
  // whole rows.  Sharing the ring leaves LDS for a deeper ring, and so more
  // steps between a tile's stores and the first wait on a DMA issued after
  // them (stores and DMAs share vmcnt, in issue order).
  auto store = [&](Cur c, char* stg) {
    uint16_t* ob = static_cast<uint16_t*>(c.seg == g.E ? g.out_sh : g.out) +
                   (c.seg == g.E ? 0 : static_cast<size_t>(c.seg) * g.M * g.N);
    __syncthreads();  // every wave is done reading the stage
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      if (wm == ph / (NPH / 2)) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (NPH == 4 && j != (ph & 1)) continue;
          const int ml = (NPH == 4 ? 0 : j * 32) + (lane & 31);  // row inside the phase
#pragma unroll
          for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nl = wn * (BN / 2) + i * 32 + 8 * q + 4 * (lane >> 5);
              const uint32_t lo = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
              const uint32_t hi = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              *reinterpret_cast<uint2*>(stg + ml * BN * 2 + (((nl >> 3) ^ (ml & (OCH - 1))) << 4) +
                                        (nl & 7) * 2) = make_uint2(lo, hi);
            }
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < NSH; ++q) {
        const int idx = tid + q * 256, r = idx / OCH, cc = idx % OCH;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * BN * 2 + ((cc ^ (r & (OCH - 1))) << 4));
        // non-temporal: the dW stream would otherwise evict the A and B
        // chunks that the group's other blocks are about to read from L2
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<u32x4_t*>(ob + static_cast<size_t>((c.gm * 8 + sm) * BM + ph * PR + r) * g.N +
                                                               (c.gn * 8 + sn) * BN + cc * 8));
      }
      __syncthreads();  // the staging rows are free again
    }
  };

  Cur ci = settle(carry(Cur{0, 0, xcd, 0, 0, 0, 0, nullptr, nullptr}));  // the next chunk to DMA
  if (ci.sg >= nseg) return;  // no tile for this block
  Cur cc = ci;             // the next chunk to multiply
  zero_acc();
  int n_iss = 0;  // chunks DMA'd so far
#pragma unroll
  for (int q = 0; q < STAGES - 1; ++q)
    if (ci.sg < nseg) {
      issue(ci, q);
      ci = advance(ci);
      ++n_iss;
    }
  uint32_t ends = 0;  // bit d - 1: the chunk d steps back ended a tile (its stores follow)
  for (int s = 0;; ++s) {
    const int st = s % STAGES;
    // chunk s is in LDS once at most the memory operations issued after its
    // DMAs are in flight: the later chunks' DMAs and the tile stores of the
    // STAGES - 1 steps since (stores count in vmcnt too, in issue order)
    const int after = (n_iss - 1 - s) * OPS + NST * __builtin_popcount(ends & ((1u << (STAGES - 1)) - 1));
    wait_vm_range<0, 63>(after);
    __builtin_amdgcn_s_barrier();  // ... for every wave; all are done with chunk s - 1
    if (ci.sg < nseg) {
      issue(ci, (s + STAGES - 1) % STAGES);
      ci = advance(ci);
      ++n_iss;
    }
    const int kv = min(KC, cc.rem);
    char* base = smem + st * STAGE;
    if (kv > 0) {
      if (kv < KC) {  // rows past the segment: clear the A rows
        for (int i = tid; i < (KC - kv) * 16; i += 256)
          *reinterpret_cast<uint4*>(base + (kv + i / 16) * 256 + (i % 16) * 16) = make_uint4(0, 0, 0, 0);
        __syncthreads();
      }
      bf16x8_t bn[2][NB], am[2][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int i = 0; i < NB; ++i) bn[kh][i] = frag(base, offB[kh][i][0], offB[kh][i][1]);
#pragma unroll
        for (int j = 0; j < 2; ++j) am[kh][j] = frag(base, offA[kh][j][0], offA[kh][j][1]);
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bn[kh][i], am[kh][j], acc[i][j], 0, 0, 0);
    }
    const bool end = cc.kc == cc.nkc - 1;
    if (end) {
      store(cc, base);
      zero_acc();
    }
    ends = (ends << 1) | (end ? 1u : 0u);
    cc = advance(cc);
    if (cc.sg >= nseg) break;
  }
}

// dW[e] for the routed segments of at most strip_rows (<= 128) rows, most of
// the experts of a prefill batch.  A 128 x 128 tile over K = such a
// segment's rows reads about as many bytes of A and B as it writes, so a
// tile-by-tile walk reads about as much as it writes unless L2 catches the
// re-reads.  Here a block takes a strip: one m-tile of one segment (128
// columns of A_e).  The strip's rows of A_e are DMA'd into LDS once and kept
// there while the block walks every n-tile of dW[e], streaming 32-row chunks
// of B_e (the segment's rows, the n-tile's columns) through a STAGES-deep
// ring; each wave stages its part of a finished tile in LDS of its own and
// stores it as whole 128-byte lines.  The small segments are
// dealt to the 8 XCDs in turn (block b runs on XCD b % 8) and an XCD's 64
// blocks take its strips in order, so a segment's strips (M / 128 of them)
// run together on one XCD and read the same B_e rows, at most 128 x N
// values, through its L2.  A segment without rows gets zero tiles.
template <int STAGES, int RS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void wgrad_strip_kernel(WgradArgs g) {
  constexpr int BM = 128, BN = 128, KC = 32;
  constexpr int CH = KC * 256;                // one 32-row chunk of 256-byte rows (A or B)
  constexpr int OPS = CH / 1024 / 4;          // DMAs per wave per chunk
  constexpr int NA = RS / KC;                 // A chunks of a strip, at most
  constexpr int NB = BN / 64;                 // 32-column n blocks per wave
  constexpr int NST = 8;                      // 16-byte stores of a tile, per thread
  constexpr int B_OFF = NA * CH;
  constexpr int STG_OFF = B_OFF + STAGES * CH;
  constexpr int LDS_BYTES = STG_OFF + 4 * 4096;  // a 32 x 64 staging block per wave
  static_assert(RS % KC == 0 && BM == 128 && BN == 128, "strip shape");
  static_assert((STAGES - 2) * OPS + (STAGES - 1) * NST <= 63, "vmcnt range");
  static_assert(LDS_BYTES + kMaxExperts / 8 * 4 + 16 <= 81920, "two blocks per CU");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  __shared__ int list[kMaxExperts / 8];  // this XCD's segments, in order
  __shared__ int wsum[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves of 64 x 64
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;  // 512 blocks: 64 per XCD
  const int MTt = g.M / BM, NTt = g.N / BN;
  const uint32_t lda = static_cast<uint32_t>(g.M) * 2, ldb = static_cast<uint32_t>(g.N) * 2;

  // the small segments, numbered in expert order by a block-wide scan (two
  // experts per thread); number i goes to XCD i % 8
  const int e0 = 2 * tid, e1 = e0 + 1;
  const int f0 = (e0 < g.E && g.offsets[e0 + 1] - g.offsets[e0] <= g.strip_rows) ? 1 : 0;
  const int f1 = (e1 < g.E && g.offsets[e1 + 1] - g.offsets[e1] <= g.strip_rows) ? 1 : 0;
  int v = f0 + f1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int i0 = before + v - f0 - f1;  // number of e0 among the small segments
  if (f0 && i0 % 8 == xcd) list[i0 / 8] = e0;
  if (f1 && (i0 + f0) % 8 == xcd) list[(i0 + f0) / 8] = e1;
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int nlist = (total - xcd + 7) / 8;  // numbers i < total with i % 8 == xcd
  __syncthreads();

  // per-lane DMA and fragment offsets, as in wgrad_kernel: rows of 16
  // swizzled 16-byte chunks; lane l holds column l % 32 at K rows
  // 16 kh + 8 (l / 32) + 0..7 of both operands
  int rq[OPS];
  uint32_t cq[OPS];
#pragma unroll
  for (int q = 0; q < OPS; ++q) {
    rq[q] = (wave * OPS + q) * 4 + lane / 16;
    cq[q] = static_cast<uint32_t>(((lane & 15) ^ wg_swz<16>(rq[q])) << 4);
  }
  const uint32_t lds0 = lds_address(smem);
  const int kgr = lane >> 4, p = lane & 15;
  auto toff = [&](int col0, int kh, int h) {
    const int r = 16 * kh + 8 * (kgr >> 1) + 4 * h + (p >> 2);
    const int col = col0 + 16 * (kgr & 1) + (p & 3) * 4;
    return r * 256 + (((col >> 3) ^ wg_swz<16>(r)) << 4) + (col & 7) * 2;
  };
  int offB[2][NB][2], offA[2][2][2];  // [kh][block][h]
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < NB; ++i) offB[kh][i][h] = B_OFF + toff(wn * (BN / 2) + i * 32, kh, h);
#pragma unroll
      for (int j = 0; j < 2; ++j) offA[kh][j][h] = toff(wm * 64 + j * 32, kh, h);
    }
  auto frag = [&](const char* base, int o0, int o1) {
    const i16x4_t lo4 = ds_read_tr16(base + o0);
    const i16x4_t hi4 = ds_read_tr16(base + o1);
    const i16x8s_t w = i16x8s_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8_t, w);
  };
  f32x16_t acc[NB][2];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  };
  // tile (mt, n) of dW[e] at ob.  Each wave stages its own 64 x 64 part, 32
  // rows at a time, in its own 4 KB of LDS (128-byte rows, 16-byte chunk c
  // of row r at c ^ ((r >> 1) & 7), which keeps both the 8-byte writes and
  // the 16-byte reads free of bank conflicts) and stores it as whole 128-byte
  // lines, non-temporal; no block-wide barrier.
  char* wstg = smem + STG_OFF + wave * 4096;
  auto store = [&](uint16_t* ob, int mt, int n) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ml = lane & 31;
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 4 * i + q;  // columns 8 c .. 8 c + 7 of the wave's 64
          const uint32_t lo = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<uint2*>(wstg + ml * 128 + ((c ^ ((ml >> 1) & 7)) << 4) + (lane >> 5) * 8) =
              make_uint2(lo, hi);
        }
      // the wave's LDS operations run in order: once its writes are done,
      // its reads see them (the memory clobber keeps the compiler's order)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = (lane >> 3) + 8 * k, ch = lane & 7;
        const uint4 w = *reinterpret_cast<const uint4*>(wstg + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4));
        __builtin_nontemporal_store(u32x4_t{w.x, w.y, w.z, w.w},
                                    reinterpret_cast<u32x4_t*>(ob + static_cast<size_t>(mt * BM + wm * 64 + j * 32 + r) * g.N +
                                                               n * BN + wn * 64 + ch * 8));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
    }
  };

  const int nstrips = nlist * MTt;
  for (int s = slot; s < nstrips; s += 64) {
    const int li = s / MTt, mt = s - li * MTt;
    const int e = __builtin_amdgcn_readfirstlane(list[li]);
    int k0, k1;
    scalar_load2(g.offsets + e, k0, k1);
    const int R = k1 - k0;
    uint16_t* ob = static_cast<uint16_t*>(g.out) + static_cast<size_t>(e) * g.M * g.N;
    zero_acc();
    if (R == 0) {
      for (int n = 0; n < NTt; ++n) store(ob, mt, n);
      continue;
    }
    const int nkc = (R + KC - 1) / KC;
    // the strip's A rows (rows past the segment repeat its last row and are
    // cleared below, before the first multiply)
    const char* a_src = uniform_ptr(static_cast<const char*>(g.A) + static_cast<size_t>(k0) * lda + mt * BM * 2);
    for (int kc = 0; kc < nkc; ++kc) {
      const int kv = min(KC, R - kc * KC);
#pragma unroll
      for (int q = 0; q < OPS; ++q)
        dma16_at(uniform_ptr(a_src + static_cast<size_t>(kc) * KC * lda),
                 static_cast<uint32_t>(min(rq[q], kv - 1)) * lda + cq[q],
                 lds0 + kc * CH + (wave * OPS + q) * 1024);
    }
    // B chunks in (n-tile, chunk) order: chunk kc of n-tile n is rows
    // 32 kc .. of the segment, columns n BN ..
    const char* b_src = uniform_ptr(static_cast<const char*>(g.B) + static_cast<size_t>(k0) * ldb);
    auto issue = [&](int n, int kc, int st) {
      const int kv = min(KC, R - kc * KC);
#pragma unroll
      for (int q = 0; q < OPS; ++q)
        dma16_at(uniform_ptr(b_src + static_cast<size_t>(kc) * KC * ldb + n * BN * 2),
                 static_cast<uint32_t>(min(rq[q], kv - 1)) * ldb + cq[q],
                 lds0 + B_OFF + st * CH + (wave * OPS + q) * 1024);
    };
    const int nsteps = NTt * nkc;
    int in_ = 0, ikc = 0, n_iss = 0;  // the next chunk to DMA
#pragma unroll
    for (int q = 0; q < STAGES - 1; ++q)
      if (n_iss < nsteps) {
        issue(in_, ikc, q);
        if (++ikc == nkc) {
          ikc = 0;
          ++in_;
        }
        ++n_iss;
      }
    int cn = 0, ckc = 0;  // the chunk to multiply
    uint32_t ends = 0;    // bit d - 1: the step d back ended a tile (its stores follow)
    for (int t = 0; t < nsteps; ++t) {
      const int st = t % STAGES;
      // chunk t (and, issued before it, the strip's A rows) is in LDS once at
      // most the memory operations issued after it are in flight
      const int after = (n_iss - 1 - t) * OPS + NST * __builtin_popcount(ends & ((1u << (STAGES - 1)) - 1));
      wait_vm_range<0, 63>(after);
      __builtin_amdgcn_s_barrier();  // ... for every wave; all are done with chunk t - 1
      if (t == 0 && R % KC != 0) {  // A rows past the segment: clear
        const int kv = R % KC;
        char* al = smem + (nkc - 1) * CH;
        for (int i = tid; i < (KC - kv) * 16; i += 256)
          *reinterpret_cast<uint4*>(al + (kv + i / 16) * 256 + (i % 16) * 16) = make_uint4(0, 0, 0, 0);
        __syncthreads();
      }
      if (n_iss < nsteps) {
        issue(in_, ikc, (t + STAGES - 1) % STAGES);
        if (++ikc == nkc) {
          ikc = 0;
          ++in_;
        }
        ++n_iss;
      }
      const char* abase = smem + ckc * CH;
      const char* bbase = smem + st * CH;
      bf16x8_t bn[2][NB], am[2][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int i = 0; i < NB; ++i) bn[kh][i] = frag(bbase, offB[kh][i][0], offB[kh][i][1]);
#pragma unroll
        for (int j = 0; j < 2; ++j) am[kh][j] = frag(abase, offA[kh][j][0], offA[kh][j][1]);
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bn[kh][i], am[kh][j], acc[i][j], 0, 0, 0);
      const bool end = ckc == nkc - 1;
      if (end) {
        store(ob, mt, cn);
        zero_acc();
      }
      ends = (ends << 1) | (end ? 1u : 0u);
      if (++ckc == nkc) {
        ckc = 0;
        ++cn;
      }
    }
    __syncthreads();  // every wave is done with the strip's A rows and B chunks
  }
}

// Gating-bias gradient: column sums of dl [T, E] in two fixed-order passes.
// Pass 1: block (expert group of 64, 256-row chunk); wave w sums rows w, w +
// 4, ... of the chunk; the 4 wave sums are added in order.
__global__ __launch_bounds__(256) void colsum_partial_kernel(int T, int E, const float* __restrict__ dl,
                                                             float* __restrict__ part) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int t0 = blockIdx.y * 256;
  float s = 0.0f;
  if (e < E)
    for (int t = t0 + w; t < min(T, t0 + 256); t += 4) s += dl[static_cast<size_t>(t) * E + e];
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && e < E)
    part[static_cast<size_t>(blockIdx.y) * E + e] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// Pass 2: out[e] = sum over the chunks, in chunk order.
__global__ __launch_bounds__(256) void colsum_final_kernel(int nchunk, int E, const float* __restrict__ part,
                                                           float* __restrict__ out) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  float s = 0.0f;
  for (int c = 0; c < nchunk; ++c) s += part[static_cast<size_t>(c) * E + e];
  out[e] = s;
}

// ---------------------------------------------------------------- launches
constexpr int kDgradBM = 128;

hipError_t dgrad(const DgradArgs& in, int rows, int T_sh, bool swb, hipStream_t stream) {
  DgradArgs g = in;
  hipLaunchKernelGGL(bwd_tile_offsets_kernel, dim3(1), dim3(kMaxExperts), 0, stream, g.offsets,
                     g.E, T_sh, kDgradBM, const_cast<int32_t*>(g.tile_off));
  const long ub_m = (rows + kDgradBM - 1) / kDgradBM + (g.E < rows ? g.E : rows) +
                    (T_sh + kDgradBM - 1) / kDgradBM;
  if (!swb && g.N % 512 == 0 && static_cast<long>(rows) < 256L * g.E) {
    // about one m-tile of rows per expert: 512-wide n-tiles halve the
    // re-reads of the gradient rows (one per n-tile), as in the forward
    // (measured slower for Linear2's dgrad, whose N = inter gives 6 n-tiles)
    g.n_tiles = g.N / 512;
    const dim3 grid(static_cast<unsigned>(ub_m * g.n_tiles));
    hipLaunchKernelGGL((dgrad_kernel<kDgradBM, 512, 2, 4, 3, false>), grid, dim3(512), 0, stream, g);
  } else if (g.N % 256 == 0) {
    g.n_tiles = g.N / 256;
    const dim3 grid(static_cast<unsigned>(ub_m * g.n_tiles));
    if (swb)
      hipLaunchKernelGGL((dgrad_kernel<kDgradBM, 256, 2, 4, 3, true>), grid, dim3(512), 0, stream, g);
    else
      hipLaunchKernelGGL((dgrad_kernel<kDgradBM, 256, 2, 4, 3, false>), grid, dim3(512), 0, stream, g);
  } else {
    g.n_tiles = g.N / 128;
    const dim3 grid(static_cast<unsigned>(ub_m * g.n_tiles));
    if (swb)
      hipLaunchKernelGGL((dgrad_kernel<kDgradBM, 128, 2, 2, 3, true>), grid, dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((dgrad_kernel<kDgradBM, 128, 2, 2, 3, false>), grid, dim3(256), 0, stream, g);
  }
  return hipGetLastError();
}

// The strip kernel: ring depth and the most rows of a segment it takes.
constexpr int kStripStages = 3, kStripRows = 128;

hipError_t wgrad(const WgradArgs& in, hipStream_t stream) {
  constexpr unsigned kBlocks = 512;  // 64 per XCD, two per CU
  WgradArgs g = in;
  const bool strips = g.E > 0 && g.N % 128 == 0 && g.M % 128 == 0;
  g.strip_rows = strips ? kStripRows : -1;
  if (strips && g.N % 256 == 0)  // the experts above strip_rows and the shared expert: long K
    hipLaunchKernelGGL((wgrad_kernel<256, 3>), dim3(kBlocks), dim3(256), 0, stream, g);
  else if (g.N % 128 == 0)
    hipLaunchKernelGGL((wgrad_kernel<128, 5>), dim3(kBlocks), dim3(256), 0, stream, g);
  else  // N % 64 == 0 (the router's experts)
    hipLaunchKernelGGL((wgrad_kernel<64, 5>), dim3(kBlocks), dim3(256), 0, stream, g);
  if (strips)
    hipLaunchKernelGGL((wgrad_strip_kernel<kStripStages, kStripRows>), dim3(kBlocks), dim3(256), 0,
                       stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu_bf16(const void* H1, int f, long rows, long arows, const float* grow,
                              void* Aw, void* Af, hipStream_t stream) {
  const long n = arows * (f / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(H1), f, rows, arows, grow,
                     static_cast<uint16_t*>(Aw), static_cast<uint16_t*>(Af));
  return hipGetLastError();
}

hipError_t launch_row_gate(const int32_t* dst_row, const float* G, int n, float* grow,
                           hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(row_gate_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, dst_row, G, n,
                     grow);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  const int rows = a.T * a.k;
  const int T_sh = a.has_shared ? a.T : 0;
  const size_t h = a.h, f = a.f;
  hipError_t e;
  // unpermute backward: dY copied to each of its token's rows
  if (rows > 0) {
    hipLaunchKernelGGL(unpermute_backward_kernel, dim3(a.T), dim3(256), 0, stream, a.h, a.k,
                       static_cast<const uint16_t*>(a.dY), a.dst_row, static_cast<uint16_t*>(a.dYp));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // Linear2 dgrad of the unweighted rows with the SwiGLU backward: dH1 and
  // the partial dG of every routed row (the shared expert's upstream
  // gradient is dY itself)
  DgradArgs d2{};
  d2.A = a.dYp;
  d2.A_sh = a.dY;
  d2.W = a.W2;
  d2.W_sh = a.Ws2;
  d2.out = a.dH1;
  d2.out_sh = static_cast<char*>(a.dH1) + static_cast<size_t>(rows) * 2 * f * 2;
  d2.h1 = a.H1;
  d2.h1_sh = static_cast<const char*>(a.H1) + static_cast<size_t>(rows) * 2 * f * 2;
  d2.grow = a.grow;
  d2.dgp = a.dGp;
  d2.offsets = a.offsets;
  d2.tile_off = a.tile_b;
  d2.E = a.E;
  d2.K = a.h;
  d2.N = a.f;
  d2.T = a.T;
  if ((e = dgrad(d2, rows, T_sh, true, stream)) != hipSuccess) return e;
  // dG = the sum of each row's partials
  if (rows > 0) {
    hipLaunchKernelGGL(dg_reduce_kernel, dim3((rows + 255) / 256), dim3(256), 0, stream, rows,
                       a.f / 64, a.dst_row, static_cast<const float*>(a.dGp), a.dG);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // Linear2 wgrad: dW2[e] = (G A)_eᵀ dYp_e (shared: Aᵀ dY)
  WgradArgs w2{};
  w2.A = a.Aact;
  w2.A_sh = static_cast<const char*>(a.Aact) + static_cast<size_t>(rows) * f * 2;
  w2.B = a.dYp;
  w2.B_sh = a.dY;
  w2.out = a.dW2;
  w2.out_sh = a.dWs2;
  w2.offsets = a.offsets;
  w2.E = a.E;
  w2.M = a.f;
  w2.N = a.h;
  w2.T = a.T;
  w2.has_shared = a.has_shared;
  if ((e = wgrad(w2, stream)) != hipSuccess) return e;
  // Linear1 dgrad: dXp = dH1 W1ᵀ (shared rows after the routed ones)
  DgradArgs d1{};
  d1.A = a.dH1;
  d1.A_sh = d2.out_sh;
  d1.W = a.W1;
  d1.W_sh = a.Ws1;
  d1.out = a.dXp;
  d1.out_sh = static_cast<char*>(a.dXp) + static_cast<size_t>(rows) * h * 2;
  d1.offsets = a.offsets;
  d1.tile_off = a.tile_b;
  d1.E = a.E;
  d1.K = 2 * a.f;
  d1.N = a.h;
  d1.T = a.T;
  if ((e = dgrad(d1, rows, T_sh, false, stream)) != hipSuccess) return e;
  // Linear1 wgrad: dW1[e] = Xp_eᵀ dH1_e (shared: Xᵀ dH1_sh)
  WgradArgs w1{};
  w1.A = a.Xp;
  w1.A_sh = a.X;
  w1.B = a.dH1;
  w1.B_sh = d2.out_sh;
  w1.out = a.dW1;
  w1.out_sh = a.dWs1;
  w1.offsets = a.offsets;
  w1.E = a.E;
  w1.M = a.h;
  w1.N = 2 * a.f;
  w1.T = a.T;
  w1.has_shared = a.has_shared;
  if ((e = wgrad(w1, stream)) != hipSuccess) return e;
  // router: dl, dWg = Xᵀ dl, dgate_bias, dXr = dl Wgᵀ
  const void* dXr = nullptr;
  if (a.route) {
    hipLaunchKernelGGL(route_backward_kernel, dim3((a.T + 3) / 4), dim3(256), 0, stream, a.T, a.E,
                       a.k, a.keys, a.beta, a.hash, a.score_fn, a.renorm, a.alpha, a.ids, a.dG,
                       a.dl32, static_cast<uint16_t*>(a.dl16));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.dgate_bias) {  // partial sums in a region of their own: the saved keys stay intact
      const int nchunk = (a.T + 255) / 256;
      float* part = a.colsum;
      hipLaunchKernelGGL(colsum_partial_kernel, dim3((a.E + 63) / 64, nchunk), dim3(256), 0, stream,
                         a.T, a.E, a.dl32, part);
      hipLaunchKernelGGL(colsum_final_kernel, dim3((a.E + 255) / 256), dim3(256), 0, stream, nchunk,
                         a.E, part, a.dgate_bias);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.dWg) {
      WgradArgs wr{};
      wr.A_sh = a.X;
      wr.B_sh = a.dl16;
      wr.out_sh = a.dWg;
      wr.E = 0;
      wr.M = a.h;
      wr.N = a.E;
      wr.T = a.T;
      wr.has_shared = 1;
      if ((e = wgrad(wr, stream)) != hipSuccess) return e;
    }
    DgradArgs dr{};
    dr.A_sh = a.dl16;
    dr.W_sh = a.Wg;  // [h, E] = [N, K]
    dr.out_sh = a.dXr;
    dr.offsets = a.offsets;  // not read with E = 0
    dr.tile_off = a.tile_b;
    dr.E = 0;
    dr.K = a.E;
    dr.N = a.h;
    dr.T = a.T;
    if ((e = dgrad(dr, 0, a.T, false, stream)) != hipSuccess) return e;
    dXr = a.dXr;
  }
  // permute backward: dX = sum of the k rows + shared + router
  hipLaunchKernelGGL(permute_backward_kernel, dim3(a.T), dim3(256), 0, stream, a.h, a.k,
                     static_cast<const uint16_t*>(a.dXp), a.dst_row,
                     a.has_shared ? static_cast<const uint16_t*>(d1.out_sh) : nullptr,
                     static_cast<const uint16_t*>(dXr), static_cast<uint16_t*>(a.dX));
  return hipGetLastError();
}

}  // namespace moe
