// grouped_gemm.hip -- the expert FFN of the routed MoE layer as two grouped
// GEMMs over ragged per-expert row blocks (CANN "mega_moe" page, §计算过程
// Expert Compute: Linear1, SwiGLU, Linear2, and its A8W8 block; DeepSeek-V4
// blog post, §ETP 里的矩阵 for F(X) = (SiLU(X Wg) * X Wu) Wd).
//
//   Linear1 + SwiGLU:  A[r, n] = SiLU(H[r, n]) * H[r, f + n],  H = Xp[r] W1[e]
//   Linear2:           Yp[r]  = A[r] W2[e]
// for every row r of expert e's block [offsets[e], offsets[e+1]); the shared
// expert is one more segment whose rows are the T tokens themselves (input
// Xs, output rows T*k.. of A and Ys).
//
// Tile schedule (device side, no host sync): tile_off[e] is the prefix sum of
// ceil(rows_e / BM) over segments 0..E (E = shared).  The grid is an upper
// bound of m-tiles times the n-tiles; blocks past the real count exit at
// once.  A block renumbers itself so that each of the 8 XCDs (blocks are dealt
// to them round-robin) runs runs of consecutive work items (one contiguous
// range, or chunks of two m-tiles' items dealt to the XCDs in turn), and
// inside a segment items go in groups of m-tiles (1024 rows), n-tile major:
// the blocks an XCD runs together share weight columns and token rows in its
// L2.  16-row
// MFMA tiles past a segment's last row are skipped, so a cold expert's tile
// costs only the rows it has, and padding rows are never stored.
//
// Prefill (grouped_gemm_dma_kernel): operands go global -> LDS by DMA
// (global_load_lds_dwordx4) into a 3-stage ring, with waits written out as
// s_waitcnt vmcnt + s_barrier.  Weights are [K, N] row-major and stay so in
// LDS; the MFMA's K-consecutive B fragments come from transposing LDS reads
// (ds_read_b64_tr_b16 / _tr_b8).  Tiles: bf16 128 x 256 on 4 waves, two
// blocks per CU, or 128 x 512 on 8 waves when experts hold about one m-tile
// of rows (its two row halves of 4 waves take turns at reading fragments and
// multiplying); e4m3 128 x 256 on 8 waves.
// Decode (grouped_gemm_kernel, a few rows per expert): 16 x 256 tiles on 4
// waves with one LDS stage, which fits more blocks per CU and so keeps more
// weight bytes in flight; each thread loads a 4 x 16-byte weight block into
// registers and writes it transposed (v_perm byte shuffles), and the next
// K-tile is prefetched into registers while the current one is multiplied.
//   bf16: v_mfma_f32_16x16x32_bf16 (decode) and v_mfma_f32_32x32x16_bf16
//         (prefill; twice the rate), a lane holding 8 K-consecutive elements
//   e4m3: v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (32 per lane)
// For SwiGLU an N-tile of BN columns holds BN/2 gate columns and the
// matching BN/2 up columns, and each wave owns equal gate/up sub-tiles, so the
// gate and up accumulators of an output element sit in the same lane.
//
// A8W8 (e4m3, or INT8 with int32 products): H = C * w1_scale[e, n] *
// x_scale[r]; the SwiGLU output is written in fp32 and requantised per row
// (scale = max|A[r]| / 448, or / 127 for INT8) by requant_kernel; Linear2
// dequantises with w2_scale[e, n] * a_scale[r].
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBKBytes = 128;
constexpr int kRowBytes = kBKBytes;  // LDS row: one K-tile of one row, no padding

// LDS byte offset of 16-byte chunk `chunk` (0..7) of row `row`.  Chunks are
// XOR-swizzled by f(row) = ((row >> 1) & 7) ^ (((row >> 5) & 1) << 2), which
// is constant on no two rows of equal parity within an aligned group of 16:
//   - an MFMA operand read (16 consecutive rows, one logical chunk) hits 16
//     distinct 4-bank groups;
//   - 16-byte row writes (8 lanes per row) fill all 64 banks;
//   - the transposed weight writes below (see store_bt) are conflict-free.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  const int f = ((row >> 1) & 7) ^ (((row >> 5) & 1) << 2);
  return row * kRowBytes + ((chunk ^ f) << 4);
}

struct GemmArgs {
  const void* A;         // routed input rows [M, K]
  const void* A_sh;      // shared-expert input rows [T, K] (or null)
  const void* a_scale;  // FP8: fp32 per routed row; MX: E8M0 [rows, K/32]
  const void* a_scale_sh;
  const void* W;         // [E, K, Nw]
  const void* W_sh;      // [K, Nw]
  const void* w_scale;  // FP8: fp32 [E, Nw]; MX: E8M0 [E, K/32, Nw]
  const void* w_scale_sh;
  void* out_scale;      // MX SwiGLU: E8M0 scales [rows, Nout/32] of the output codes
  void* out_scale_sh;
  void* out;             // routed rows [M, Nout]
  void* out_sh;          // shared rows [T, Nout]
  const int32_t* offsets;
  const int32_t* tile_off;
  int E, K, Nw, Nout, f, T, n_tiles;
  int chunk;  // DMA kernel: items per XCD chunk (0: one contiguous range per XCD)
  // DMA kernel, bf16: routed row r is row gather[r] of A (null: row r of A)
  const int32_t* gather;
};

template <int PREC>
struct Mfma;

template <>
struct Mfma<MOE_PREC_BF16> {
  static constexpr int kEsz = 2;
  static constexpr int kStepBytes = 64;  // K bytes per MFMA (32 bf16)
  typedef bf16x8_t frag;
  // lane's 8 K-consecutive elements: chunk (kstep * 4 + lane / 16) of the row
  __device__ static frag load(const char* base, int row, int kstep, int lane) {
    return *reinterpret_cast<const bf16x8_t*>(base + lds_off(row, kstep * 4 + (lane >> 4)));
  }
  __device__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<MOE_PREC_FP8> {
  static constexpr int kEsz = 1;
  static constexpr int kStepBytes = 128;  // K bytes per MFMA (128 e4m3)
  typedef i32x8_t frag;
  // lane's 32 K-consecutive elements: chunks 2 * (lane / 16) and the next
  __device__ static frag load(const char* base, int row, int kstep, int lane) {
    const int c = (lane >> 4) * 2;
    i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + lds_off(row, c));
    i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + lds_off(row, c + 1));
    (void)kstep;
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    // formats 0/0 = e4m3 for both operands; E8M0 scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// Transposed store of a 4(k) x 16-byte block of weights: r[q] holds K-row
// kb*4+q, columns nl.. of the tile.  Writes each column's 4 K-values (8 bytes
// of bf16, 4 of e4m3) into its LDS row.  A wave's lanes hold 16 K-groups x 4
// column chunks; lanes of odd chunks write their columns in the order c ^ 1
// (`rot`), so at every write half the wave is on even rows and half on odd
// rows, which with the swizzle spreads one write instruction over all banks.
template <int ESZ>
__device__ __forceinline__ void store_bt(char* Bs, int nl, int kb, int rot,
                                         const uint32_t (&r)[4][4]) {
  const int kbyte = kb * 4 * ESZ;
  const int chunk = kbyte >> 4, within = kbyte & 15;
  if (ESZ == 2) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int cc = c ^ rot;
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      uint32_t d0 = __builtin_amdgcn_perm(r[1][c >> 1], r[0][c >> 1], sel);
      uint32_t d1 = __builtin_amdgcn_perm(r[3][c >> 1], r[2][c >> 1], sel);
      *reinterpret_cast<uint2*>(Bs + lds_off(nl + cc, chunk) + within) = make_uint2(d0, d1);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int cc = c ^ rot;
      const uint32_t b = cc & 3;
      const uint32_t sel = b | ((4u + b) << 8) | (b << 16) | ((4u + b) << 24);
      uint32_t t01 = __builtin_amdgcn_perm(r[1][c >> 2], r[0][c >> 2], sel);
      uint32_t t23 = __builtin_amdgcn_perm(r[3][c >> 2], r[2][c >> 2], sel);
      *reinterpret_cast<uint32_t*>(Bs + lds_off(nl + cc, chunk) + within) =
          __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    }
  }
}

template <int PREC, int BM, int BN, int WAVES_M, int WAVES_N, bool SWIGLU, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void grouped_gemm_kernel(GemmArgs g) {
  using M = Mfma<PREC>;
  constexpr int NTHR = 64 * WAVES_M * WAVES_N;
  constexpr int ESZ = M::kEsz;
  constexpr int kColsPer16B = 16 / ESZ;           // elements per 16-byte load
  constexpr int WM = BM / WAVES_M;
  constexpr int MT = WM / 16;
  constexpr int NTW = BN / WAVES_N / 16;          // n-tiles per wave
  constexpr int kAChunks = BM * kBKBytes / 16;
  constexpr int kAPer = (kAChunks + NTHR - 1) / NTHR;
  constexpr int kBBlocks = (kBKBytes / ESZ / 4) * (BN / kColsPer16B);
  constexpr int kBPer = (kBBlocks + NTHR - 1) / NTHR;
  constexpr int kBKRows = kBKBytes / ESZ / 4;  // 4-row K groups per tile (16 or 32)
  constexpr int kKGroups = kBKRows / 16;        // 16-lane K spans per tile
  static_assert((BN / kColsPer16B) % 4 == 0, "B mapping needs 4 column chunks per wave");
  static_assert(MT >= 1 && NTW >= 1, "tile shape");
  static_assert(!SWIGLU || (NTW % 2 == 0), "SwiGLU needs gate/up pairs per wave");

  __shared__ __attribute__((aligned(16))) char As[STAGES][BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) char Bs[STAGES][BN * kRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // ------------------------------------------------ tile -> segment
  // Work items: (m-tile, n-tile) pairs, m-tiles ordered by segment.  Blocks
  // are dealt round-robin to the 8 XCDs, so block b is renumbered such that
  // each XCD runs one contiguous range of work items; inside a segment, items
  // go in groups of GROUP_M m-tiles, n-tile major, so the blocks an XCD runs
  // at the same time share both their weight columns and their rows in L2.
  constexpr int GROUP_M = 4;
  const int E = g.E;
  const int NT = g.n_tiles;
  const int total = g.tile_off[E + 1] * NT;
  if (static_cast<int>(blockIdx.x) >= total) return;
  int item;
  {
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = total >> 3, rem = total & 7;
    item = x * per + min(x, rem) + slot;
  }
  const int mq = item / NT;  // segment search key: m-tile index of the item's group row
  int lo = 0, hi = E;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (g.tile_off[mid] <= mq)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int seg = lo;
  const int mt_seg = g.tile_off[seg + 1] - g.tile_off[seg];
  const int local = item - g.tile_off[seg] * NT;
  const int grp = local / (GROUP_M * NT);
  const int gsz = min(GROUP_M, mt_seg - grp * GROUP_M);
  const int rin = local - grp * GROUP_M * NT;
  const int nt = rin / gsz;
  const int mtile = grp * GROUP_M + rin % gsz;

  const bool shared = (seg == E);
  int row0, row_end;
  const char* Abase;
  const char* Wbase;
  const float* wsc;
  const float* asc;
  char* obase;
  if (!shared) {
    row0 = g.offsets[seg] + mtile * BM;
    row_end = g.offsets[seg + 1];
    Abase = static_cast<const char*>(g.A);
    Wbase = static_cast<const char*>(g.W) + static_cast<size_t>(seg) * g.K * g.Nw * ESZ;
    wsc = g.w_scale ? static_cast<const float*>(g.w_scale) + static_cast<size_t>(seg) * g.Nw
                    : nullptr;
    asc = static_cast<const float*>(g.a_scale);
    obase = static_cast<char*>(g.out);
  } else {
    row0 = mtile * BM;
    row_end = g.T;
    Abase = static_cast<const char*>(g.A_sh);
    Wbase = static_cast<const char*>(g.W_sh);
    wsc = static_cast<const float*>(g.w_scale_sh);
    asc = static_cast<const float*>(g.a_scale_sh);
    obase = static_cast<char*>(g.out_sh);
  }
  const int rows_valid = min(BM, row_end - row0);
  // number of this wave's 16-row tiles that hold at least one valid row
  const int mt_live = max(0, min(MT, (rows_valid - wm * WM + 15) / 16));
  const int K = g.K;
  const size_t a_ld = static_cast<size_t>(K) * ESZ;    // bytes per A row
  const size_t w_ld = static_cast<size_t>(g.Nw) * ESZ;  // bytes per W row

  // column of LDS row n (0..BN-1) in the weight matrix
  auto wcol = [&](int nl) -> int {
    if (SWIGLU) {
      const int half = BN / 2;
      return nl < half ? nt * half + nl : g.f + nt * half + (nl - half);
    }
    return nt * BN + nl;
  };

  // Loads are unconditional (rows clamped into the segment, surplus threads
  // repeat a chunk and store the same bytes) so that no branch separates a
  // load from its use and all of a tile's loads are in flight together.
  i32x4_t ra[kAPer];
  uint32_t rb[kBPer][4][4];
  auto gload = [&](int kt) {
    const size_t kb0 = static_cast<size_t>(kt) * kBKBytes;
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int c = (tid + q * NTHR) % kAChunks;
      const int r = c / (kBKBytes / 16), c16 = c % (kBKBytes / 16);
      const int row = min(row0 + r, row_end - 1);
      ra[q] = *reinterpret_cast<const i32x4_t*>(Abase + row * a_ld + kb0 + c16 * 16);
    }
#pragma unroll
    for (int q = 0; q < kBPer; ++q) {
      const int b = (tid + q * NTHR) % kBBlocks;
      const int kb = ((b >> 6) % kKGroups) * 16 + (b & 15);
      const int nb = ((b >> 6) / kKGroups) * 4 + ((b >> 4) & 3);
      const char* p = Wbase + (static_cast<size_t>(kt) * (kBKBytes / ESZ) + kb * 4) * w_ld +
                      static_cast<size_t>(wcol(nb * kColsPer16B)) * ESZ;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        i32x4_t v = *reinterpret_cast<const i32x4_t*>(p + r * w_ld);
        rb[q][r][0] = v[0];
        rb[q][r][1] = v[1];
        rb[q][r][2] = v[2];
        rb[q][r][3] = v[3];
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kAPer; ++q) {
      const int c = (tid + q * NTHR) % kAChunks;
      const int r = c / (kBKBytes / 16), c16 = c % (kBKBytes / 16);
      *reinterpret_cast<i32x4_t*>(&As[buf][lds_off(r, c16)]) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < kBPer; ++q) {
      const int b = (tid + q * NTHR) % kBBlocks;
      const int kb = ((b >> 6) % kKGroups) * 16 + (b & 15);
      const int nb = ((b >> 6) / kKGroups) * 4 + ((b >> 4) & 3);
      store_bt<ESZ>(Bs[buf], nb * kColsPer16B, kb, nb & 1, rb[q]);
    }
  };

  f32x4_t acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LDS row of this wave's n-tile j
  auto brow = [&](int j) -> int {
    if (SWIGLU) {
      const int half = BN / 2, per = BN / 2 / WAVES_N;
      return j < NTW / 2 ? wn * per + j * 16 : half + wn * per + (j - NTW / 2) * 16;
    }
    return wn * (BN / WAVES_N) + j * 16;
  };

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kBKBytes / M::kStepBytes; ++ks) {
      typename M::frag bfr[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) bfr[j] = M::load(Bs[buf], brow(j) + (lane & 15), ks, lane);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i < mt_live) {
          typename M::frag af = M::load(As[buf], wm * WM + i * 16 + (lane & 15), ks, lane);
#pragma unroll
          for (int j = 0; j < NTW; ++j) acc[i][j] = M::mma(af, bfr[j], acc[i][j]);
        }
      }
    }
  };

  const int KT = K * ESZ / kBKBytes;
  gload(0);
  sstore(0);
  __syncthreads();
  // steady state without conditionals (the last K-tile is peeled off)
  for (int kt = 0; kt < KT - 1; ++kt) {
    const int buf = (STAGES == 2) ? (kt & 1) : 0;
    gload(kt + 1);
    compute(buf);
    if (STAGES == 1) __syncthreads();  // the single buffer is about to be overwritten
    sstore(STAGES == 2 ? (buf ^ 1) : 0);
    __syncthreads();
  }
  compute(STAGES == 2 ? ((KT - 1) & 1) : 0);

  // ------------------------------------------------ epilogue
  // lane holds column (lane & 15) and rows 4*(lane >> 4) + v of each 16x16 tile
  const int col_in = lane & 15;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i >= mt_live) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + wm * WM + i * 16 + (lane >> 4) * 4 + v;
      if (row >= row_end) continue;
      const float rs = (PREC == MOE_PREC_FP8) ? asc[row] : 1.0f;
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < NTW / 2; ++j) {
          const int nl = brow(j) + col_in;  // gate LDS row; output column inside the tile
          const int ncol = nt * (BN / 2) + nl;
          float hg = acc[i][j][v];
          float hu = acc[i][j + NTW / 2][v];
          if (PREC == MOE_PREC_FP8) {
            hg *= wsc[ncol] * rs;
            hu *= wsc[g.f + ncol] * rs;
            static_cast<float*>(static_cast<void*>(obase))[static_cast<size_t>(row) * g.Nout + ncol] =
                silu(hg) * hu;
          } else {
            reinterpret_cast<uint16_t*>(obase)[static_cast<size_t>(row) * g.Nout + ncol] =
                f32_to_bf16(silu(hg) * hu);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int ncol = nt * BN + brow(j) + col_in;
          float y = acc[i][j][v];
          if (PREC == MOE_PREC_FP8) y *= wsc[ncol] * rs;
          reinterpret_cast<uint16_t*>(obase)[static_cast<size_t>(row) * g.Nout + ncol] =
              f32_to_bf16(y);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 DMA path
// The bf16 grouped GEMM with both operands brought into LDS by asynchronous
// global->LDS DMA (global_load_lds_dwordx4: each lane's 16 bytes land at
// base + 16 * lane) into a ring of STAGES K-slices of 32 elements, so that
// STAGES-1 slices are in flight while one is multiplied.  Weights stay in
// their [K, N] layout in LDS; the MFMA B fragments are read with gfx950's
// transposing LDS load ds_read_b64_tr_b16: in each 16-lane group, output
// lane i, element q, is element i % 4 of the 8-byte piece addressed by lane
// 4q + i / 4, so lane p addresses row k0 + p / 4, columns n0 + 4 (p % 4) and
// receives column n0 + i of rows k0..k0+3.  Two such loads give the 8
// K-consecutive values of one lane's B fragment.
//
// LDS layout of one stage:
//   A: BM rows x 64 bytes; 16-byte chunk c of row r at c ^ ((r >> 2) & 3)
//      (an MFMA read of 16 consecutive rows then covers all 64 banks);
//   B: 32 rows (k) x BN*2 bytes; chunk c of row r at c ^ 4 (r & 3), so that
//      each half of a transposing load (4 K rows x 64 bytes) touches every
//      bank once.
// The swizzles are applied on the global side: lane i of a DMA instruction
// fetches the chunk that belongs at LDS position i.
//
// The DMA writes LDS outside the compiler's view, so every wait is explicit:
// s_waitcnt vmcnt(n) leaves exactly the later stages in flight, then a plain
// s_barrier (no fence, which would drain all of them) publishes the stage.

// (dma16, dma4, uniform_ptr, wait_vmcnt, ds_read_tr16/8: lds_dma.h)

// Operand layout of one precision in the DMA pipeline (see above).
//   bf16: K-stage 32 elements; A rows 64 B (4 chunks, swizzle (r>>2)&3); B
//         fragments from 2 transposing 16-bit reads of 4 K-rows each.
//   e4m3: K-stage 128 elements; A rows 128 B (8 chunks, swizzle (r>>1)&7); B
//         fragments from 4 transposing 8-bit reads of 8 K-rows each; in a
//         16-lane group, output lane i byte q is byte i % 8 of the piece
//         addressed by lane 2q + i / 8, so lane p addresses row k0 + p / 2,
//         columns n0 + 8 (p % 2), and receives column n0 + i of 8 rows.
// B chunk swizzles spread each transposing read over all banks (twice).
template <int PREC, int BN>
struct DmaOps;

// bf16 multiplies 32 x 32 output tiles with v_mfma_f32_32x32x16_bf16 (twice
// the rate of the 16x16x32 form on gfx950): a stage's 32 K-values are two
// 16-deep halves kh, and in each a lane holds row (or column) lane % 32 at K
// 16 kh + 8 (lane / 32) + 0..7, for A and for B alike.  The accumulator's
// element v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
struct Bf16Pair {
  bf16x8_t k0, k1;
};

template <int BN>
struct DmaOps<MOE_PREC_BF16, BN> {
  static constexpr int ESZ = 2, BK = 32, A_CHUNKS = 4;
  static constexpr int TM = 32, NV = 16;  // MFMA tile and accumulator elements per lane
  typedef Bf16Pair frag;
  typedef f32x16_t acc_t;
  __device__ static int row_of(int lane, int v) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
  __device__ static int col_of(int lane) { return lane & 31; }
  __device__ static int swz_a(int r) { return (r >> 2) & 3; }
  // B chunk swizzle: a transposing read's 32-lane half covers 4 consecutive
  // K rows x 4 chunks (64 bytes); XOR by 4 (r % 4) gives the 4 rows disjoint
  // chunk sets, 16 chunks on 64 distinct banks (rows start on bank 0)
  __device__ static int swz_b(int r) { return 4 * (r & 3); }
  // byte offsets (inside a stage's B region) of this lane's transposing
  // reads: lane group g reads rows 16 kh + 8 (g >> 1) + 4 h + p / 4 of the
  // 16 columns from col0 + 16 (g & 1)
  template <int B_ROW>
  __device__ static void b_offsets(int lane, int col0, int (&o)[4]) {
    const int g = lane >> 4, p = lane & 15;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * kh + 8 * (g >> 1) + 4 * h + (p >> 2);
        const int col = col0 + 16 * (g & 1) + (p & 3) * 4;  // element
        o[2 * kh + h] = r * B_ROW + (((col >> 3) ^ swz_b(r)) << 4) + (col & 7) * 2;
      }
  }
  __device__ static bf16x8_t tr_pair(const char* st, int o0, int o1) {
    const i16x4_t lo4 = ds_read_tr16(st + o0);
    const i16x4_t hi4 = ds_read_tr16(st + o1);
    typedef __attribute__((ext_vector_type(8))) short i16x8_t;
    const i16x8_t v = i16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
  __device__ static frag load_b(const char* st, const int (&o)[4]) {
    return frag{tr_pair(st, o[0], o[1]), tr_pair(st, o[2], o[3])};
  }
  // row r of the tile: 16-byte chunk 2 kh + lane / 32 (K 16 kh + 8 (lane / 32))
  template <int A_ROW>
  __device__ static void a_offsets(int r, int lane, int (&o)[2]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) o[kh] = r * A_ROW + (((2 * kh + (lane >> 5)) ^ swz_a(r)) << 4);
  }
  __device__ static frag load_a(const char* st, const int (&o)[2]) {
    return frag{*reinterpret_cast<const bf16x8_t*>(st + o[0]), *reinterpret_cast<const bf16x8_t*>(st + o[1])};
  }
  __device__ static f32x16_t mma(frag a, frag b, f32x16_t c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.k0, b.k0, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.k1, b.k1, c, 0, 0, 0);
  }
};

template <int BN>
struct DmaOps<MOE_PREC_FP8, BN> {
  static constexpr int ESZ = 1, BK = 128, A_CHUNKS = 8;
  // 16 x 16 tiles: element v of lane l is row 4 (l / 16) + v, column l % 16
  static constexpr int TM = 16, NV = 4;
  typedef i32x8_t frag;
  typedef f32x4_t acc_t;
  __device__ static int row_of(int lane, int v) { return 4 * (lane >> 4) + v; }
  __device__ static int col_of(int lane) { return lane & 15; }
  __device__ static int swz_a(int r) { return (r >> 1) & 7; }
  __device__ static int swz_b(int r) {
    return BN >= 256 ? (r & 7) + 8 * ((r >> 5) & 1) : ((r & 7) >> 1) + 4 * ((r >> 5) & 1);
  }
  // K placement of the 16x16x128 8-bit MFMA: byte j of lane group g is K
  // index (j < 16 ? 0 : 64) + 16 g + j % 16, and the E8M0 scale of lane group
  // s covers K 32 s .. 32 s + 31 (read off the instruction on the GPU with
  // one-hot operands).  Both fragments follow it, so a lane group's scale is
  // the scale of the K-group it holds.
  __device__ static int k_of(int g, int half) { return (half ? 64 : 0) + 16 * g; }
  template <int B_ROW>
  __device__ static void b_offsets(int lane, int col0, int (&o)[4]) {
    const int g = lane >> 4, p = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = k_of(g, h >> 1) + 8 * (h & 1) + (p >> 1);
      const int col = col0 + (p & 1) * 8;  // byte
      o[h] = r * B_ROW + (((col >> 4) ^ swz_b(r)) << 4) + (col & 15);
    }
  }
  __device__ static frag load_b(const char* st, const int (&o)[4]) {
    const i32x2v_t a = ds_read_tr8(st + o[0]);
    const i32x2v_t b = ds_read_tr8(st + o[1]);
    const i32x2v_t c = ds_read_tr8(st + o[2]);
    const i32x2v_t d = ds_read_tr8(st + o[3]);
    return i32x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  template <int A_ROW>
  __device__ static void a_offsets(int r, int lane, int (&o)[2]) {
    const int g = lane >> 4;  // 16-byte chunks k_of(g, 0) / 16 and k_of(g, 1) / 16
    o[0] = r * A_ROW + (((k_of(g, 0) >> 4) ^ swz_a(r)) << 4);
    o[1] = r * A_ROW + (((k_of(g, 1) >> 4) ^ swz_a(r)) << 4);
  }
  __device__ static frag load_a(const char* st, const int (&o)[2]) {
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(st + o[0]);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(st + o[1]);
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// e4m3 with 512-wide n-tiles: 32 x 32 tiles on the scaled 32x32x64 MFMA
// (unit scales), K-stages of 64 values, so that a stage (8 KB of A, 32 KB of
// B) is the bf16 512-wide kernel's and three fit in LDS.  A lane holds row
// (or column) lane % 32 at K 32 (lane / 32) + 0..31: for A two 16-byte chunks
// of its 64-byte row, for B four transposing 8-bit reads of 8 K-rows each,
// byte j of either at K 32 (lane / 32) + j; with unit scales the MFMA's own
// K order does not matter, only that A and B agree.  B rows are 512 bytes
// (32 chunks); half a transposing read covers 8 consecutive K-rows x 2
// chunks, which the swizzle chunk ^ 2 (r % 8) puts on 64 distinct banks.
template <>
struct DmaOps<MOE_PREC_FP8, 512> {
  static constexpr int ESZ = 1, BK = 64, A_CHUNKS = 4;
  static constexpr int TM = 32, NV = 16;
  typedef i32x8_t frag;
  typedef f32x16_t acc_t;
  __device__ static int row_of(int lane, int v) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
  __device__ static int col_of(int lane) { return lane & 31; }
  __device__ static int swz_a(int r) { return (r >> 2) & 3; }
  __device__ static int swz_b(int r) { return 2 * (r & 7); }
  template <int B_ROW>
  __device__ static void b_offsets(int lane, int col0, int (&o)[4]) {
    const int g = lane >> 4, p = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = 32 * (g >> 1) + 8 * h + (p >> 1);
      const int col = col0 + 16 * (g & 1) + 8 * (p & 1);  // byte
      o[h] = r * B_ROW + (((col >> 4) ^ swz_b(r)) << 4) + (col & 15);
    }
  }
  __device__ static frag load_b(const char* st, const int (&o)[4]) {
    const i32x2v_t a = ds_read_tr8(st + o[0]);
    const i32x2v_t b = ds_read_tr8(st + o[1]);
    const i32x2v_t c = ds_read_tr8(st + o[2]);
    const i32x2v_t d = ds_read_tr8(st + o[3]);
    return i32x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  template <int A_ROW>
  __device__ static void a_offsets(int r, int lane, int (&o)[2]) {
    const int c0 = 2 * (lane >> 5);
    o[0] = r * A_ROW + ((c0 ^ swz_a(r)) << 4);
    o[1] = r * A_ROW + (((c0 + 1) ^ swz_a(r)) << 4);
  }
  __device__ static frag load_a(const char* st, const int (&o)[2]) {
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(st + o[0]);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(st + o[1]);
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// The work item of this block: its segment, m-tile and n-tile (false when
// the block has none).  Blocks are dealt to the 8 XCDs round-robin; XCD x
// runs either one contiguous range of items or (g.chunk > 0) chunks of
// g.chunk items dealt to the XCDs in turn.  Items are (m-tile, n-tile) pairs,
// m-tiles ordered by segment (tile_off); inside a segment they go in groups
// of 1024 / BM m-tiles, n-tile major.
template <int BM>
__device__ __forceinline__ bool block_item(const GemmArgs& g, int& seg, int& mtile, int& nt) {
  constexpr int GROUP_M = 1024 / BM;
  const int E = g.E;
  const int NT = g.n_tiles;
  const int total = g.tile_off[E + 1] * NT;
  int item;
  if (g.chunk > 0) {
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3, C = g.chunk;
    item = (slot / C) * (8 * C) + x * C + slot % C;
    if (item >= total) return false;
  } else {
    if (static_cast<int>(blockIdx.x) >= total) return false;
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = total >> 3, rem = total & 7;
    item = x * per + min(x, rem) + slot;
  }
  const int mq = item / NT;
  int lo = 0, hi = E;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
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

// MXFP8 shares the e4m3 operand layout; its MFMA takes each lane's E8M0
// scale byte (the lane's 32 K-values are one MX group) for A and for B.
template <int BN>
struct DmaOps<MOE_PREC_MXFP8, BN> : DmaOps<MOE_PREC_FP8, BN> {
  __device__ static f32x4_t mma_mx(i32x8_t a, i32x8_t b, f32x4_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  }
};

// MXFP8 on the 128 x 512 tiles.  The scaled 32x32x64 form takes K 0..31 of
// the stage from bytes 0-15 of both lane groups and K 32..63 from bytes
// 16-31, and lane l's scale for row (column) l % 32 and K group l / 32
// (measured on the GPU with one-hot operands and per-lane scales).  So lane
// group G holds K 16 G .. 16 G + 15 in bytes 0-15 and K 32 + 16 G .. in bytes
// 16-31 (A: 16-byte chunks G and G + 2 of the row; B: the transposing reads
// from those K rows), and each lane passes the scale of its row or column
// and group l / 32.
template <>
struct DmaOps<MOE_PREC_MXFP8, 512> : DmaOps<MOE_PREC_FP8, 512> {
  template <int B_ROW>
  __device__ static void b_offsets(int lane, int col0, int (&o)[4]) {
    const int g = lane >> 4, p = lane & 15, G = g >> 1;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int r = 8 * h + 16 * G + 16 * (h >> 1) + (p >> 1);
      const int col = col0 + 16 * (g & 1) + 8 * (p & 1);  // byte
      o[h] = r * B_ROW + (((col >> 4) ^ swz_b(r)) << 4) + (col & 15);
    }
  }
  template <int A_ROW>
  __device__ static void a_offsets(int r, int lane, int (&o)[2]) {
    const int G = lane >> 5;
    o[0] = r * A_ROW + ((G ^ swz_a(r)) << 4);
    o[1] = r * A_ROW + (((G + 2) ^ swz_a(r)) << 4);
  }
  __device__ static f32x16_t mma_mx(i32x8_t a, i32x8_t b, f32x16_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  }
};

// INT8 (the A8W8 block as printed) shares the 8-bit operand layout: a stage's
// 128 K-values per lane pair go through two 16x16x64 int8 MFMAs, the first
// on bytes 0-15 of both fragments and the second on bytes 16-31.  A and B
// fragments hold the same K indices at the same (lane group, byte), and an
// MFMA pairs A and B bytes that way, so the two MFMAs sum exactly the
// stage's 128 products, into int32.
template <int BN>
struct DmaOps<MOE_PREC_INT8, BN> : DmaOps<MOE_PREC_FP8, BN> {
  typedef i32x4_t acc_t;
  __device__ static i32x4_t mma(i32x8_t a, i32x8_t b, i32x4_t c) {
    const i32x4_t alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
    const i32x4_t blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi, c, 0, 0, 0);
  }
};

typedef __attribute__((ext_vector_type(16))) int i32x16_t;

// INT8 on the 128 x 512 tiles: the e4m3 32x32 operand layout, a stage's 64
// K-values per lane pair through two 32x32x32 int8 MFMAs (bytes 0-15 of both
// fragments, then bytes 16-31).  As for the 16x16 form, A and B hold the same
// K index at the same (lane, byte), so the pair sums exactly the stage's
// products, into int32.
template <>
struct DmaOps<MOE_PREC_INT8, 512> : DmaOps<MOE_PREC_FP8, 512> {
  typedef i32x16_t acc_t;
  __device__ static i32x16_t mma(i32x8_t a, i32x8_t b, i32x16_t c) {
    const i32x4_t alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
    const i32x4_t blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo, blo, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi, bhi, c, 0, 0, 0);
  }
};

// E8M0 code of the MX group scale for an e4m3 group whose largest magnitude
// is amax (fp32): floor(log2 amax) - 8, i.e. the biased exponent minus 8,
// clamped at 0 (all-zero and tiny groups); and 2^(127 - code) as a float.
__device__ __forceinline__ uint32_t mx_e4m3_code(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF);
  return static_cast<uint32_t>(e > 8 ? e - 8 : 0);
}
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// Two waves per SIMD for bf16 (two 4-wave blocks that cover each other's
// stage barriers); e4m3 keeps one block of deeper stages per CU.
template <int PREC, int BM, int BN, int WAVES_M, int WAVES_N, bool SWIGLU, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
__attribute__((amdgpu_waves_per_eu((PREC == MOE_PREC_BF16 || WAVES_M * WAVES_N >= 8 || STAGES * (BM + BN) * 128 <= 81920) ? 2 : 1)))
void grouped_gemm_dma_kernel(GemmArgs g) {
  using O = DmaOps<PREC, BN>;
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int ESZ = O::ESZ;
  constexpr int BK = O::BK;               // K elements per stage (one MFMA step)
  constexpr int A_ROW = BK * ESZ;         // bytes
  constexpr int B_ROW = BN * ESZ;         // bytes
  constexpr int A_BYTES = BM * A_ROW;
  constexpr int B_BYTES = BK * B_ROW;
  constexpr bool MX = PREC == MOE_PREC_MXFP8;
  // A8W8 (e4m3 or INT8): per-channel and per-row fp32 scales in the epilogue
  constexpr bool A8W8 = PREC == MOE_PREC_FP8 || PREC == MOE_PREC_INT8;
  // MX: each stage also holds the E8M0 scales of its KG K-groups: A [BM][4]
  // (per row the aligned dword that holds them: K / 32 is a multiple of 4)
  // and B [KG][BN] (one byte per group row and column)
  constexpr int KG = BK / 32;
  constexpr int AS_OFF = A_BYTES + B_BYTES;
  constexpr int BS_OFF = AS_OFF + (MX ? BM * 4 : 0);
  constexpr int STAGE = BS_OFF + (MX ? KG * BN : 0);
  constexpr int AS_INSTS = MX ? BM / 64 : 0;  // dword DMA: 64 rows per instruction
  constexpr int A_INSTS = (A_BYTES + 1023) / 1024;
  constexpr int B_INSTS = B_BYTES / 1024;
  constexpr int A_OPS = (A_INSTS + NW - 1) / NW;  // DMA instructions per wave per stage
  constexpr int B_OPS = B_INSTS / NW;
  constexpr int A_RPI = 1024 / A_ROW;     // A rows per DMA instruction
  constexpr int B_CHUNKS = B_ROW / 16;    // 16-byte chunks per B row
  constexpr int B_RPI = 1024 / B_ROW;     // B rows per DMA instruction
  constexpr int TM = O::TM;  // MFMA tile (rows = columns)
  constexpr int WM = BM / WAVES_M;
  constexpr int MT = WM / TM;
  constexpr int NTW = BN / WAVES_N / TM;
  static_assert(WM % TM == 0 && (BN / WAVES_N) % TM == 0, "wave tile in MFMA tiles");
  static_assert(B_INSTS % NW == 0, "B stage must split evenly over the waves");
  static_assert(A_BYTES % 1024 == 0 || A_INSTS == 1, "A stage granularity");
  static_assert(!SWIGLU || (NTW % 2 == 0), "SwiGLU needs gate/up pairs per wave");
  static_assert(!MX || (KG * BN == 1024 && BM % 64 == 0 && NW > AS_INSTS && KG <= 4),
                "MX scale DMA: one 1 KB instruction for B, 64-row ones for A");
  static_assert(!MX || !SWIGLU || TM == 32 || (NTW / 2) % 2 == 0,
                "MX SwiGLU epilogue: whole 32-column groups per wave");
  // ping-pong K loop for two row halves of 4 waves (see the K loop); bf16
  // only (measured: V4-Pro bf16 0.7% faster, e4m3 0.6% slower)
  constexpr bool PP = (NW == 8) && (WAVES_M == 2) && PREC == MOE_PREC_BF16;
  // the ping-pong tile, and the 8-bit A8W8 128 x 512 tile: transposed
  // products and an epilogue staged through LDS (see the epilogue)
  constexpr bool STAGED =
      PP || (A8W8 && BM == 128 && BN == 512 && NW == 8 && WAVES_M == 2 && O::TM == 32);

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: DMA targets are SGPRs
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // ------------------------------------------------ tile -> segment (as above)
  const int E = g.E;
  int seg, mtile, nt;
  if (!block_item<BM>(g, seg, mtile, nt)) return;

  const bool shared = (seg == E);
  int row0, row_end;
  const char* Abase;
  const char* Wbase;
  const float* wsc;
  const float* asc;
  char* obase;
  if (!shared) {
    row0 = g.offsets[seg] + mtile * BM;
    row_end = g.offsets[seg + 1];
    Abase = static_cast<const char*>(g.A);
    Wbase = static_cast<const char*>(g.W) + static_cast<size_t>(seg) * g.K * g.Nw * ESZ;
    wsc = g.w_scale ? static_cast<const float*>(g.w_scale) + static_cast<size_t>(seg) * g.Nw
                    : nullptr;
    asc = static_cast<const float*>(g.a_scale);
    obase = static_cast<char*>(g.out);
  } else {
    row0 = mtile * BM;
    row_end = g.T;
    Abase = static_cast<const char*>(g.A_sh);
    Wbase = static_cast<const char*>(g.W_sh);
    wsc = static_cast<const float*>(g.w_scale_sh);
    asc = static_cast<const float*>(g.a_scale_sh);
    obase = static_cast<char*>(g.out_sh);
  }
  // MX scale arrays of this segment (E8M0 bytes)
  const uint8_t* asc8 = nullptr;
  const uint8_t* wsc8 = nullptr;
  uint8_t* osc8 = nullptr;
  if constexpr (MX) {
    asc8 = static_cast<const uint8_t*>(shared ? g.a_scale_sh : g.a_scale);
    wsc8 = static_cast<const uint8_t*>(shared ? g.w_scale_sh : g.w_scale) +
           (shared ? 0 : static_cast<size_t>(seg) * (g.K / 32) * g.Nw);
    osc8 = static_cast<uint8_t*>(shared ? g.out_scale_sh : g.out_scale);
  }
  const int rows_valid = min(BM, row_end - row0);
  // wave-uniform: keep it scalar so the skip below is a scalar branch
  const int mt_live =
      __builtin_amdgcn_readfirstlane(max(0, min(MT, (rows_valid - wm * WM + TM - 1) / TM)));
  const size_t a_ld = static_cast<size_t>(g.K) * ESZ;
  const size_t w_ld = static_cast<size_t>(g.Nw) * ESZ;

  // DMA sources: a wave-uniform base (the tile's first row and column, K
  // offset added per stage) plus a 32-bit per-lane offset.  A: instruction
  // blk covers rows A_RPI blk .. + A_RPI - 1 of the tile (clamped to the
  // segment's last row).
  // A gathered routed rows (bf16): the base is the first token row and each
  // lane's offset is its row's token times the row pitch (host-checked to
  // stay below 2^32).
  const int32_t* gat = nullptr;
  if constexpr (PREC == MOE_PREC_BF16) gat = shared ? nullptr : g.gather;
  const char* a_base = uniform_ptr(gat ? Abase : Abase + static_cast<size_t>(row0) * a_ld);
  uint32_t a_voff[A_OPS];
#pragma unroll
  for (int q = 0; q < A_OPS; ++q) {
    const int blk = (wave * A_OPS + q) % A_INSTS;
    const int r = blk * A_RPI + lane / O::A_CHUNKS;
    const int c = (lane % O::A_CHUNKS) ^ O::swz_a(r);
    const int rr = min(r, row_end - 1 - row0);
    const uint32_t row = gat ? static_cast<uint32_t>(gat[row0 + rr]) : static_cast<uint32_t>(rr);
    a_voff[q] = row * static_cast<uint32_t>(a_ld) + c * 16;
  }
  const char* b_base = uniform_ptr(
      Wbase + static_cast<size_t>(nt) * (SWIGLU ? BN / 2 : BN) * ESZ);
  uint32_t b_voff[B_OPS];
#pragma unroll
  for (int q = 0; q < B_OPS; ++q) {
    const int blk = wave * B_OPS + q;
    const int r = blk * B_RPI + lane / B_CHUNKS;
    const int c = (lane % B_CHUNKS) ^ O::swz_b(r);
    const int nl = c * (16 / ESZ);  // LDS column (element) of the chunk
    int col = nl;  // column relative to the tile's first gate (or plain) column
    if (SWIGLU && nl >= BN / 2) col = g.f + (nl - BN / 2);
    b_voff[q] = static_cast<uint32_t>(r) * static_cast<uint32_t>(w_ld) + col * ESZ;
  }
  // Only A blocks that hold a valid row are fetched; rows past them are never
  // read by a live MFMA.  The count is wave-uniform and so is this wave's
  // number of DMA instructions per stage.
  const int a_live =
      (A_INSTS == 1)
          ? A_OPS
          : __builtin_amdgcn_readfirstlane(
                max(0, min(A_OPS, ((rows_valid + A_RPI - 1) / A_RPI) - wave * A_OPS)));
  // MX scale DMA: waves 0 .. AS_INSTS-1 fetch 64 rows' A scale dwords each,
  // wave AS_INSTS the B scales (4 group rows of the tile's BN columns)
  const size_t sc_ld = static_cast<size_t>(g.K / 32);  // scale bytes per A row
  const char* as_base = nullptr;
  const char* bs_base = nullptr;
  uint32_t as_voff = 0, bs_voff = 0;
  int ops_sc = 0;
  if constexpr (MX) {
    as_base = uniform_ptr(reinterpret_cast<const char*>(asc8) + static_cast<size_t>(row0) * sc_ld);
    as_voff = static_cast<uint32_t>(min(wave * 64 + lane, row_end - 1 - row0)) *
              static_cast<uint32_t>(sc_ld);
    bs_base = uniform_ptr(reinterpret_cast<const char*>(wsc8) +
                          static_cast<size_t>(nt) * (SWIGLU ? BN / 2 : BN));
    constexpr int CPR = BN / 16;  // 16-byte chunks of a group row
    const int nl = (lane % CPR) * 16;
    const int col = (SWIGLU && nl >= BN / 2) ? g.f + (nl - BN / 2) : nl;
    bs_voff = static_cast<uint32_t>(lane / CPR) * static_cast<uint32_t>(g.Nw) + col;
    ops_sc = (wave <= AS_INSTS) ? 1 : 0;
  }
  // Without MX scales every wave issues the same number of DMAs per stage:
  // A blocks past the segment's last row are fetched too (their rows clamp
  // to that row, one L2 line), so the vmcnt waits below are constants.
  constexpr bool CONST_OPS = !MX;
  constexpr int OPS = A_OPS + B_OPS;
  const int ops_w = (CONST_OPS ? A_OPS : a_live) + B_OPS + ops_sc;
  const uint32_t lds0 = lds_address(smem);
  auto issue = [&](int kt, int slot) {
    char* st = smem + slot * STAGE;
    const uint32_t sl = lds0 + slot * STAGE;
#pragma unroll
    for (int q = 0; q < A_OPS; ++q) {
      const int blk = (wave * A_OPS + q) % A_INSTS;
      if (CONST_OPS || q < a_live)
        dma16_at(a_base + static_cast<size_t>(kt) * A_ROW, a_voff[q], sl + blk * 1024);
    }
#pragma unroll
    for (int q = 0; q < B_OPS; ++q) {
      const int blk = wave * B_OPS + q;
      dma16_at(b_base + static_cast<size_t>(kt) * BK * w_ld, b_voff[q], sl + A_BYTES + blk * 1024);
    }
    if constexpr (MX) {
      if (wave < AS_INSTS)
        dma4(as_base + ((static_cast<size_t>(kt) * KG) & ~static_cast<size_t>(3)), as_voff,
             st + AS_OFF + wave * 256);
      else if (wave == AS_INSTS)
        dma16(bs_base + static_cast<size_t>(kt) * KG * g.Nw, bs_voff, st + BS_OFF);
    }
  };

  // one of this wave's DMAs of stage kt (q < A_OPS: A, else B)
  auto issue_op = [&](int kt, int slot, int q) {
    const uint32_t sl = lds0 + slot * STAGE;
    if (q < A_OPS) {
      const int blk = (wave * A_OPS + q) % A_INSTS;
      dma16_at(a_base + static_cast<size_t>(kt) * A_ROW, a_voff[q], sl + blk * 1024);
    } else {
      const int blk = wave * B_OPS + (q - A_OPS);
      dma16_at(b_base + static_cast<size_t>(kt) * BK * w_ld, b_voff[q - A_OPS], sl + A_BYTES + blk * 1024);
    }
  };
  typename O::acc_t acc[MT][NTW];  // fp32, or int32 for INT8
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = typename O::acc_t{};

  auto bcol = [&](int j) -> int {  // first LDS column of this wave's n-tile j
    if (SWIGLU) {
      const int half = BN / 2, per = BN / 2 / WAVES_N;
      return j < NTW / 2 ? wn * per + j * TM : half + wn * per + (j - NTW / 2) * TM;
    }
    return wn * (BN / WAVES_N) + j * TM;
  };

  int b_off[NTW][4];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    O::template b_offsets<B_ROW>(lane, bcol(j), b_off[j]);
#pragma unroll
    for (int h = 0; h < 4; ++h) b_off[j][h] += A_BYTES;
  }
  int a_off[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) O::template a_offsets<A_ROW>(wm * WM + i * TM + (lane & (TM - 1)), lane, a_off[i]);
  // MX: LDS byte of this lane's scale for A row tile i / B column tile j
  int as_off[MT], bs_off[NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i) as_off[i] = AS_OFF + (wm * WM + i * TM + (lane & (TM - 1))) * 4 + lane / TM;
#pragma unroll
  for (int j = 0; j < NTW; ++j) bs_off[j] = BS_OFF + (lane / TM) * BN + bcol(j) + (lane & (TM - 1));

  // A wave with any live row multiplies all of its MT row tiles (rows past the
  // segment only feed accumulators that are never stored); a wave with none
  // skips the stage's reads and MFMAs.  A single branch lets every fragment
  // read of the stage issue before the first MFMA.
  auto compute = [&](int slot, int kt) {
    if (mt_live == 0) return;
    const char* st = smem + slot * STAGE;
    typename O::frag bfr[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) bfr[j] = O::load_b(st, b_off[j]);
    typename O::frag af[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) af[i] = O::load_a(st, a_off[i]);
    if constexpr (MX) {
      int sa[MT], sb[NTW];
      const int a_sub = (kt * KG) & 3;  // the stage's first group inside the row's dword
#pragma unroll
      for (int i = 0; i < MT; ++i) sa[i] = *reinterpret_cast<const uint8_t*>(st + as_off[i] + a_sub);
#pragma unroll
      for (int j = 0; j < NTW; ++j) sb[j] = *reinterpret_cast<const uint8_t*>(st + bs_off[j]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = O::mma_mx(af[i], bfr[j], acc[i][j], sa[i], sb[j]);
    } else {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = STAGED ? O::mma(bfr[j], af[i], acc[i][j]) : O::mma(af[i], bfr[j], acc[i][j]);
    }
  };


  // The K loop is unrolled by STAGES so that every stage slot is a constant
  // LDS range: the compiler then sees DMA targets and operand reads as
  // disjoint and leaves the waiting to the explicit vmcnt below.
  const int KT = g.K / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);
  if constexpr (PP) {
    // Ping-pong: the waves of row half 0 (one per SIMD) and of row half 1
    // take turns, so that on every SIMD one wave multiplies while the other
    // reads its fragments.  Each stage has two phases split by a barrier:
    //   phase 1: half 0 reads stage kt, half 1 multiplies stage kt - 1;
    //   phase 2: half 0 multiplies stage kt, half 1 reads stage kt.
    // Stage kt must be in LDS before phase 1 (vmcnt wait + barrier, as
    // above); the slot that half 1 read in phase 2 is refilled after the
    // next phase-1 barrier, so half 1 waits for its reads (lgkmcnt(0))
    // before that barrier.  A wave's DMAs of stage kt + STAGES - 1 go out
    // one by one between its MFMAs (half 1 in phase 1, half 0 in phase 2):
    // a DMA can stall at issue while the memory pipeline is full, and a
    // block of them issued ahead of the MFMAs held those back.
    static_assert(CONST_OPS, "ping-pong schedule: constant DMA count per wave");
    typename O::frag pb[NTW];
    typename O::frag pa[MT];
    auto load_frags = [&](int slot) {
      const char* st = smem + slot * STAGE;
#pragma unroll
      for (int j = 0; j < NTW; ++j) pb[j] = O::load_b(st, b_off[j]);
#pragma unroll
      for (int i = 0; i < MT; ++i) pa[i] = O::load_a(st, a_off[i]);
    };
    auto mma_frags = [&]() {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = O::mma(pb[j], pa[i], acc[i][j]);
    };
    // the MFMAs, with this wave's DMAs of stage ikt (slot islot; none if
    // !more) one after each of the first OPS tile products (measured
    // against spreading them over all products: 1.5% faster on V4-Pro)
    static_assert(MT * NTW >= OPS, "a tile product per DMA");
    auto mma_issue = [&](bool more, int ikt, int islot) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          acc[i][j] = O::mma(pb[j], pa[i], acc[i][j]);
          const int idx = i * NTW + j;
          if (idx < OPS && more) issue_op(ikt, islot, idx);
        }
    };
    // The products are transposed (weight fragment first): element v of lane
    // l is row l % 32 of the row tile and column O::row_of(l, v) of the
    // n-tile, i.e. 4 groups of 4 consecutive columns, for the staged
    // epilogue below.  Each half runs its own copy of the loop (the same
    // barriers in the same order), so that fragments flow from reads to
    // MFMAs without merges.
    const bool live = mt_live > 0;
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
            if (live && kt > 0) {
              mma_issue(more, kt + STAGES - 1, (s + STAGES - 1) % STAGES);
            } else if (more) {
              issue(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
            }
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (live) {
              load_frags(s);
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
          }
        }
      }
      if (live) mma_frags();
    }
  } else
  for (int k0 = 0; k0 < KT; k0 += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      const int kt = k0 + s;
      if (kt < KT) {
        // stage kt is in LDS once at most the stages issued after it are in flight
        if constexpr (CONST_OPS)
          wait_after<OPS, STAGES - 2>(KT - 1 - kt);
        else
          wait_vmcnt_rt(min(STAGES - 2, KT - 1 - kt) * ops_w);
        __builtin_amdgcn_s_barrier();
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
        compute(s, kt);
      }
    }
  }

  // ------------------------------------------------ epilogue
  if constexpr (STAGED) {
    // Staged through LDS so that the tile leaves as whole 128-byte lines.
    // Once a wave is past the first barrier of the last stage, no wave reads
    // the ring slots of stages KT - 2 and KT - 3 again and no DMA writes
    // them: waves 0-3 stage in the first, waves 4-7 in the second, 8 KB
    // each (64 rows x 128 bytes; 16-byte chunk c of row r at
    // c ^ ((r >> 1) & 7), which keeps the writes and the 16-byte reads free
    // of bank conflicts).  A pass is 128 bytes of each of the wave's 64
    // rows: 64 bf16 columns (the SwiGLU output of its gate/up tile pairs,
    // or two of its n-tiles) or 32 fp32 columns (the A8W8 SwiGLU output of
    // one gate/up pair).
    static_assert(WM == 64 && TM == 32 && MT == 2 && NTW == 4, "wave tile");
    if (mt_live == 0) return;
    const int sslot = ((KT - 2 - (wave >> 2)) % STAGES + STAGES) % STAGES;
    char* wst = smem + sslot * STAGE + (wave & 3) * 8192;
    const int ml = lane & 31;
    constexpr bool F32OUT = A8W8 && SWIGLU;
    constexpr int PASSES = SWIGLU ? (F32OUT ? 2 : 1) : 2;
    float rs[MT];  // A8W8: the rows' activation scales
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = min(row0 + wm * WM + i * TM + ml, row_end - 1);
      rs[i] = A8W8 ? asc[row] : 1.0f;
    }
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int r = i * TM + ml;
#pragma unroll
        for (int jj = 0; jj < (F32OUT ? 1 : 2); ++jj) {
          const int j = F32OUT ? pass : (SWIGLU ? jj : 2 * pass + jj);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // columns 8 q + 4 (l / 32) + 0..3 of tile j
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = static_cast<float>(acc[i][j][4 * q + e]);
              if (SWIGLU) {
                float u = static_cast<float>(acc[i][j + NTW / 2][4 * q + e]);
                if (A8W8) {
                  const int ncol = nt * (BN / 2) + bcol(j) + 8 * q + 4 * (lane >> 5) + e;
                  x *= wsc[ncol] * rs[i];
                  u *= wsc[g.f + ncol] * rs[i];
                }
                v4[e] = silu(x) * u;
              } else {
                if (A8W8) x *= wsc[nt * BN + bcol(j) + 8 * q + 4 * (lane >> 5) + e] * rs[i];
                v4[e] = x;
              }
            }
            if constexpr (F32OUT) {
              const int c = 2 * q + (lane >> 5);  // 16-byte chunk of the pass's 128 bytes
              *reinterpret_cast<float4*>(wst + r * 128 + ((c ^ ((r >> 1) & 7)) << 4)) =
                  make_float4(v4[0], v4[1], v4[2], v4[3]);
            } else {
              const int c = 4 * jj + q;
              *reinterpret_cast<uint2*>(wst + r * 128 + ((c ^ ((r >> 1) & 7)) << 4) + (lane >> 5) * 8) =
                  make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
            }
          }
        }
      }
      // a wave's LDS operations run in order: its reads see its writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // first output column of the pass and bytes per output element
      const int cbase = F32OUT ? nt * (BN / 2) + bcol(pass)
                               : (SWIGLU ? nt * (BN / 2) + bcol(0) : nt * BN + bcol(2 * pass));
      constexpr int OB = F32OUT ? 4 : 2;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = (lane >> 3) + 8 * k, ch = lane & 7;
        const uint4 w = *reinterpret_cast<const uint4*>(wst + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4));
        const int row = row0 + wm * WM + r;
        if (row < row_end)
          *reinterpret_cast<uint4*>(static_cast<char*>(obase) +
                                    (static_cast<size_t>(row) * g.Nout + cbase) * OB + ch * 16) = w;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next writes
    }
    return;
  }
  const int col_in = O::col_of(lane);
  if constexpr (MX && SWIGLU && TM == 32) {
    // SwiGLU, then MX quantisation in groups of 32 output columns: a group is
    // gate tile j of one row, one value in each of the 32 lanes that hold the
    // row (lanes 0-31 or 32-63); their amax goes round them by xor shuffles.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= mt_live) continue;  // wave-uniform
#pragma unroll
      for (int v = 0; v < O::NV; ++v) {
        const int row = row0 + wm * WM + i * TM + O::row_of(lane, v);
#pragma unroll
        for (int j = 0; j < NTW / 2; ++j) {
          const float u = silu(acc[i][j][v]) * acc[i][j + NTW / 2][v];
          float amax = fabsf(u);
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
          const uint32_t code = mx_e4m3_code(amax);
          const float inv = mx_inv_scale(code);
          if (row < row_end) {
            const int c0 = nt * (BN / 2) + bcol(j);  // first column of the group
            uint8_t* orow = reinterpret_cast<uint8_t*>(obase) + static_cast<size_t>(row) * g.Nout;
            orow[c0 + col_in] = static_cast<uint8_t>(f32_to_e4m3(u * inv));
            if (col_in == 0)
              osc8[static_cast<size_t>(row) * (g.Nout / 32) + c0 / 32] = static_cast<uint8_t>(code);
          }
        }
      }
    }
    return;
  }
  if constexpr (MX && SWIGLU) {
    // SwiGLU, then MX quantisation in groups of 32 output columns: a group is
    // gate tiles (j, j+1) of one row, i.e. 2 values in each of the 16 lanes
    // that hold the row; their amax goes round those lanes by xor shuffles.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= mt_live) continue;  // wave-uniform
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wm * WM + i * 16 + (lane >> 4) * 4 + v;
#pragma unroll
        for (int j = 0; j < NTW / 2; j += 2) {
          const float u0 = silu(acc[i][j][v]) * acc[i][j + NTW / 2][v];
          const float u1 = silu(acc[i][j + 1][v]) * acc[i][j + 1 + NTW / 2][v];
          float amax = fmaxf(fabsf(u0), fabsf(u1));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
          const uint32_t code = mx_e4m3_code(amax);
          const float inv = mx_inv_scale(code);
          if (row < row_end) {
            const int c0 = nt * (BN / 2) + bcol(j);  // first column of the group
            uint8_t* orow = reinterpret_cast<uint8_t*>(obase) + static_cast<size_t>(row) * g.Nout;
            orow[c0 + col_in] = static_cast<uint8_t>(f32_to_e4m3(u0 * inv));
            orow[c0 + 16 + col_in] = static_cast<uint8_t>(f32_to_e4m3(u1 * inv));
            if (col_in == 0)
              osc8[static_cast<size_t>(row) * (g.Nout / 32) + c0 / 32] = static_cast<uint8_t>(code);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i >= mt_live) continue;
#pragma unroll
    for (int v = 0; v < O::NV; ++v) {
      const int row = row0 + wm * WM + i * TM + O::row_of(lane, v);
      if (row >= row_end) continue;
      const float rs = A8W8 ? asc[row] : 1.0f;  // MX: scales are in the MFMA
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < NTW / 2; ++j) {
          const int ncol = nt * (BN / 2) + bcol(j) + col_in;
          float hg = static_cast<float>(acc[i][j][v]);
          float hu = static_cast<float>(acc[i][j + NTW / 2][v]);
          if (A8W8) {
            hg *= wsc[ncol] * rs;
            hu *= wsc[g.f + ncol] * rs;
            reinterpret_cast<float*>(obase)[static_cast<size_t>(row) * g.Nout + ncol] =
                silu(hg) * hu;
          } else {
            reinterpret_cast<uint16_t*>(obase)[static_cast<size_t>(row) * g.Nout + ncol] =
                f32_to_bf16(silu(hg) * hu);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int ncol = nt * BN + bcol(j) + col_in;
          float y = static_cast<float>(acc[i][j][v]);
          if (A8W8) y *= wsc[ncol] * rs;
          reinterpret_cast<uint16_t*>(obase)[static_cast<size_t>(row) * g.Nout + ncol] =
              f32_to_bf16(y);
        }
      }
    }
  }
}

// MXFP4 (e2m1 x e2m1, group-32 E8M0 scales; the mega_moe page's A4W4 MXFP
// scenario).  Both operands are K-contiguous rows: token rows [rows, K/2] and
// weights [N, K/2] as the page stores them, so weight fragments are read the
// way token-row fragments are, with no transposing LDS read.  A K-stage is
// KS x 128 elements, KS x 64 bytes of a row: with KS = 2 every row's DMA
// covers one whole 128-byte line, so no line is fetched for half its bytes
// and left in L2 for the next stage.  Both tiles go to LDS by DMA with a
// 16-byte-chunk swizzle (chunk ^ ((row >> 2) & 3) for 64-byte rows,
// chunk ^ ((row >> 1) & 7) for 128-byte rows), so a 16-lane fragment read of
// 16 consecutive rows covers all banks once.  Each stage also carries the
// rows' E8M0 scales, one [rows][4] plane (one dword per row) per 128-value
// K-step.  For 4-bit operands the 16x16x128 scaled MFMA reads lane group
// g's 16 bytes as K 32g .. 32g+31, low nibble first, and lane group g's scale
// covers exactly those (measured on the GPU with one-hot operands), so a
// lane's data and scale are one MX group.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool SWIGLU, int STAGES, int KS, bool SW>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(2)))
void grouped_gemm_mx4_kernel(GemmArgs g) {
  static_assert(KS == 1 || KS == 2, "one or two 128-value K-steps per stage");
  constexpr int WSTG = 4 / KS;  // SW: stages per 512-value scale window
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int ROWB = 64 * KS;     // bytes of one row's K-stage (KS = 2: a whole 128-byte line)
  constexpr int CH = ROWB / 16;     // 16-byte chunks of a row's K-stage
  constexpr int RPI = 1024 / ROWB;  // rows per 16-byte-lane DMA
  constexpr int A_BYTES = BM * ROWB;
  constexpr int B_BYTES = BN * ROWB;
  // scales, SW = false: one [rows][4] plane per K-step inside each stage;
  // SW = true: 512-value windows, [BM][16] then [BN][16] bytes, in two
  // buffers after the ring, each row's 16 bytes fetched by one 16-byte lane
  constexpr int AS_OFF = A_BYTES + B_BYTES;
  constexpr int BS_OFF = AS_OFF + KS * BM * 4;
  constexpr int STAGE = SW ? A_BYTES + B_BYTES : BS_OFF + KS * BN * 4;
  constexpr int SCW = (BM + BN) * 16;     // one scale window buffer
  constexpr int SC_BASE = STAGES * STAGE;
  constexpr int W_INSTS = (BM + BN) / 64;  // 16-byte-lane DMAs per window
  constexpr int W_OPS = (W_INSTS + NW - 1) / NW;
  constexpr int A_INSTS = A_BYTES / 1024;
  constexpr int B_INSTS = B_BYTES / 1024;
  constexpr int AS_INSTS = BM / 64;        // 64 rows per 4-byte-lane DMA
  constexpr int BS_INSTS = BN / 64;
  constexpr int A_OPS = A_INSTS / NW;
  constexpr int B_OPS = B_INSTS / NW;
  constexpr int WM = BM / WAVES_M;
  constexpr int MT = WM / 16;
  constexpr int NTW = BN / WAVES_N / 16;
  static_assert(A_INSTS % NW == 0 && B_INSTS % NW == 0, "tiles must split evenly over the waves");
  constexpr int SC_PER = AS_INSTS + BS_INSTS;       // scale DMAs of one K-step
  constexpr int SC_INSTS = KS * SC_PER;
  constexpr int SC_OPS = (SC_INSTS + NW - 1) / NW;  // scale DMAs per wave (dealt round-robin)
  static_assert(!SWIGLU || (NTW / 2) % 2 == 0, "MX SwiGLU epilogue: whole 32-column groups");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE + (SW ? 2 * SCW : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: wave-uniform choices
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int E = g.E;
  int seg, mtile, nt;
  if (!block_item<BM>(g, seg, mtile, nt)) return;

  const bool shared = (seg == E);
  const size_t rowb = static_cast<size_t>(g.K) / 2;   // bytes of a K-contiguous row
  const size_t sc_ld = static_cast<size_t>(g.K) / 32;  // scale bytes of a row
  int row0, row_end;
  const char* Abase;
  const char* Wbase;
  const uint8_t* asc8;
  const uint8_t* wsc8;
  char* obase;
  uint8_t* osc8;
  if (!shared) {
    row0 = g.offsets[seg] + mtile * BM;
    row_end = g.offsets[seg + 1];
    Abase = static_cast<const char*>(g.A);
    Wbase = static_cast<const char*>(g.W) + static_cast<size_t>(seg) * g.Nw * rowb;
    asc8 = static_cast<const uint8_t*>(g.a_scale);
    wsc8 = static_cast<const uint8_t*>(g.w_scale) + static_cast<size_t>(seg) * g.Nw * sc_ld;
    obase = static_cast<char*>(g.out);
    osc8 = static_cast<uint8_t*>(g.out_scale);
  } else {
    row0 = mtile * BM;
    row_end = g.T;
    Abase = static_cast<const char*>(g.A_sh);
    Wbase = static_cast<const char*>(g.W_sh);
    asc8 = static_cast<const uint8_t*>(g.a_scale_sh);
    wsc8 = static_cast<const uint8_t*>(g.w_scale_sh);
    obase = static_cast<char*>(g.out_sh);
    osc8 = static_cast<uint8_t*>(g.out_scale_sh);
  }
  const int rows_valid = min(BM, row_end - row0);
  const int mt_live =
      __builtin_amdgcn_readfirstlane(max(0, min(MT, (rows_valid - wm * WM + 15) / 16)));
  // 16-byte chunk swizzle: the 16 rows of one fragment read land on distinct
  // bank groups (4 rows of 64 bytes, or 2 rows of 128 bytes, span all banks)
  auto swz = [](int r) { return KS == 1 ? (r >> 2) & 3 : (r >> 1) & 7; };
  // weight row of LDS B row nl (SwiGLU tiles: BN/2 gate rows, then the
  // matching BN/2 up rows)
  auto wrow = [&](int nl) {
    if (SWIGLU) return nl < BN / 2 ? nt * (BN / 2) + nl : g.f + nt * (BN / 2) + (nl - BN / 2);
    return nt * BN + nl;
  };

  // DMA sources (wave-uniform base + 32-bit lane offset; K-stage offset
  // kt*ROWB for data, kt*4*KS for scales, added per stage)
  const char* a_base = uniform_ptr(Abase + static_cast<size_t>(row0) * rowb);
  uint32_t a_voff[A_OPS];
#pragma unroll
  for (int q = 0; q < A_OPS; ++q) {
    const int blk = wave * A_OPS + q;
    const int r = blk * RPI + lane / CH;
    const int c = (lane % CH) ^ swz(r);
    a_voff[q] = static_cast<uint32_t>(min(r, row_end - 1 - row0)) * static_cast<uint32_t>(rowb) +
                c * 16;
  }
  const char* b_base = uniform_ptr(Wbase);
  uint32_t b_voff[B_OPS];
#pragma unroll
  for (int q = 0; q < B_OPS; ++q) {
    const int blk = wave * B_OPS + q;
    const int r = blk * RPI + lane / CH;
    const int c = (lane % CH) ^ swz(r);
    b_voff[q] = static_cast<uint32_t>(wrow(r)) * static_cast<uint32_t>(rowb) + c * 16;
  }
  const char* as_base = uniform_ptr(reinterpret_cast<const char*>(asc8) + static_cast<size_t>(row0) * sc_ld);
  const char* bs_base = uniform_ptr(reinterpret_cast<const char*>(wsc8));
  // scale DMA q of this wave is instruction idx = q * NW + wave, of K-step
  // ks = idx / SC_PER; within it, j = idx % SC_PER: A rows 64 j .. for
  // j < AS_INSTS, else B rows 64 (j - AS_INSTS) ..
  uint32_t sc_voff[SC_OPS];
  int sc_lds[SC_OPS];
  bool sc_a[SC_OPS];
#pragma unroll
  for (int q = 0; q < SC_OPS; ++q) {
    const int idx = min(q * NW + wave, SC_INSTS - 1);  // (unused past SC_INSTS)
    const int ks = idx / SC_PER, j = idx % SC_PER;
    sc_a[q] = j < AS_INSTS;
    if (j < AS_INSTS) {
      sc_voff[q] = static_cast<uint32_t>(min(j * 64 + lane, row_end - 1 - row0)) *
                       static_cast<uint32_t>(sc_ld) + 4 * ks;
      sc_lds[q] = AS_OFF + ks * BM * 4 + j * 256;
    } else {
      const int b = j - AS_INSTS;
      sc_voff[q] = static_cast<uint32_t>(wrow(b * 64 + lane)) * static_cast<uint32_t>(sc_ld) + 4 * ks;
      sc_lds[q] = BS_OFF + ks * BN * 4 + b * 256;
    }
  }
  const int sc_ops = SW ? 0 : min(SC_OPS, max(0, (SC_INSTS - wave + NW - 1) / NW));  // wave-uniform
  // SW: window DMA q of this wave is instruction idx = q * NW + wave: A rows
  // 64 idx .. for idx < BM / 64, else B rows 64 (idx - BM / 64) ..
  uint32_t w_voff[W_OPS];
  int w_lds[W_OPS];
  bool w_a[W_OPS];
#pragma unroll
  for (int q = 0; q < W_OPS; ++q) {
    const int idx = min(q * NW + wave, W_INSTS - 1);  // (unused past W_INSTS)
    w_a[q] = idx < BM / 64;
    if (idx < BM / 64) {
      w_voff[q] = static_cast<uint32_t>(min(idx * 64 + lane, row_end - 1 - row0)) *
                  static_cast<uint32_t>(sc_ld);
    } else {
      w_voff[q] = static_cast<uint32_t>(wrow((idx - BM / 64) * 64 + lane)) * static_cast<uint32_t>(sc_ld);
    }
    w_lds[q] = idx * 1024;
  }
  const int w_ops = SW ? min(W_OPS, max(0, (W_INSTS - wave + NW - 1) / NW)) : 0;  // wave-uniform
  // only A blocks holding a valid row are fetched (wave-uniform count)
  const int a_live = __builtin_amdgcn_readfirstlane(
      max(0, min(A_OPS, (rows_valid + RPI - 1) / RPI - wave * A_OPS)));
  const int ops_w = a_live + B_OPS + sc_ops;  // DMAs per stage (SW: + w_ops at window starts)
  auto issue = [&](int kt, int slot) {
    char* st = smem + slot * STAGE;
    if (SW && kt % WSTG == 0) {  // the scale window of stages kt .. kt + WSTG - 1 goes first
      char* sw = smem + SC_BASE + ((kt / WSTG) & 1) * SCW;
#pragma unroll
      for (int q = 0; q < W_OPS; ++q) {
        if (q >= w_ops) break;
        dma16((w_a[q] ? as_base : bs_base) + static_cast<size_t>(kt / WSTG) * 16, w_voff[q],
              sw + w_lds[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < A_OPS; ++q)
      if (q < a_live)
        dma16(a_base + static_cast<size_t>(kt) * ROWB, a_voff[q], st + (wave * A_OPS + q) * 1024);
#pragma unroll
    for (int q = 0; q < B_OPS; ++q)
      dma16(b_base + static_cast<size_t>(kt) * ROWB, b_voff[q],
            st + A_BYTES + (wave * B_OPS + q) * 1024);
#pragma unroll
    for (int q = 0; q < SC_OPS; ++q) {
      if (q >= sc_ops) break;
      dma4((sc_a[q] ? as_base : bs_base) + static_cast<size_t>(kt) * 4 * KS, sc_voff[q],
           st + sc_lds[q]);
    }
  };

  f32x4_t acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto bcol = [&](int j) -> int {  // first LDS B row of this wave's n-tile j
    if (SWIGLU) {
      const int half = BN / 2, per = BN / 2 / WAVES_N;
      return j < NTW / 2 ? wn * per + j * 16 : half + wn * per + (j - NTW / 2) * 16;
    }
    return wn * (BN / WAVES_N) + j * 16;
  };
  const int kg = lane >> 4;  // K-group of this lane's fragment bytes
  int a_off[MT], as_off[MT], b_off[NTW], bs_off[NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = wm * WM + i * 16 + (lane & 15);
    a_off[i] = r * ROWB + ((kg ^ swz(r)) << 4);
    as_off[i] = SW ? SC_BASE + r * 16 + kg : AS_OFF + r * 4 + kg;
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int r = bcol(j) + (lane & 15);
    b_off[j] = A_BYTES + r * ROWB + ((kg ^ swz(r)) << 4);
    bs_off[j] = SW ? SC_BASE + BM * 16 + r * 16 + kg : BS_OFF + r * 4 + kg;
  }

  // K-step ks of a stage: logical chunks 4 ks .. 4 ks + 3 of the row, i.e. the
  // fragment offset with bit 6 flipped (rows are 128 bytes when KS = 2)
  auto compute = [&](int slot, int kt) {
    if (mt_live == 0) return;
    const char* st = smem + slot * STAGE;
    // scale bytes of K-step ks: SW: window buffer (kt / WSTG) % 2, byte
    // 4 KS (kt % WSTG) + 4 ks + kg of the row; else plane ks of the stage
    const char* sc = SW ? smem + ((kt / WSTG) & 1) * SCW + (kt % WSTG) * 4 * KS : st;
    constexpr int SA_STEP = SW ? 4 : BM * 4, SB_STEP = SW ? 4 : BN * 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4_t bfr[NTW], af[MT];
      int sb[NTW], sa[MT];
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        bfr[j] = *reinterpret_cast<const i32x4_t*>(st + (b_off[j] ^ (ks << 6)));
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *reinterpret_cast<const i32x4_t*>(st + (a_off[i] ^ (ks << 6)));
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        sb[j] = *reinterpret_cast<const uint8_t*>(sc + bs_off[j] + ks * SB_STEP);
#pragma unroll
      for (int i = 0; i < MT; ++i)
        sa[i] = *reinterpret_cast<const uint8_t*>(sc + as_off[i] + ks * SA_STEP);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const i32x8_t a8 = {af[i][0], af[i][1], af[i][2], af[i][3], 0, 0, 0, 0};
          const i32x8_t b8 = {bfr[j][0], bfr[j][1], bfr[j][2], bfr[j][3], 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[i][j], 4, 4, 0,
                                                                       sa[i], 0, sb[j]);
        }
    }
  };

  const int KT = g.K / (128 * KS);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);
  for (int k0 = 0; k0 < KT; k0 += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      const int kt = k0 + s;
      if (kt < KT) {
        // stage kt is in LDS once at most the DMAs of the stages issued after
        // it are in flight (vector memory loads complete in issue order)
        const int after = min(STAGES - 2, KT - 1 - kt);
        int pend = 0;
        for (int d = 1; d <= after; ++d) pend += ops_w + ((SW && (kt + d) % WSTG == 0) ? w_ops : 0);
        wait_vmcnt_rt(pend);
        __builtin_amdgcn_s_barrier();
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
        compute(s, kt);
      }
    }
  }

  // ------------------------------------------------ epilogue
  const int col_in = lane & 15;
  if constexpr (SWIGLU) {
    // SwiGLU, then MX e2m1 quantisation in groups of 32 output columns (gate
    // tiles j, j+1 of one row: 2 values in each of the row's 16 lanes); two
    // codes per byte, the even column's in the low nibble (its lane takes the
    // odd neighbour's code by a shuffle).
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= mt_live) continue;  // wave-uniform
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wm * WM + i * 16 + (lane >> 4) * 4 + v;
#pragma unroll
        for (int j = 0; j < NTW / 2; j += 2) {
          const float u0 = silu(acc[i][j][v]) * acc[i][j + NTW / 2][v];
          const float u1 = silu(acc[i][j + 1][v]) * acc[i][j + 1 + NTW / 2][v];
          float amax = fmaxf(fabsf(u0), fabsf(u1));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
          const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFF);
          const uint32_t code = static_cast<uint32_t>(e > 2 ? e - 2 : 0);
          const float inv = __uint_as_float((254u - code) << 23);  // 2^(127 - code)
          const uint32_t n0 = f32_to_e2m1(u0 * inv);
          const uint32_t n1 = f32_to_e2m1(u1 * inv);
          const uint32_t m0 = __shfl_xor(n0, 1, 64);
          const uint32_t m1 = __shfl_xor(n1, 1, 64);
          if (row < row_end) {
            const int c0 = nt * (BN / 2) + bcol(j);  // first column of the group
            uint8_t* orow = reinterpret_cast<uint8_t*>(obase) + static_cast<size_t>(row) * (g.Nout / 2);
            if ((col_in & 1) == 0) {
              orow[(c0 + col_in) / 2] = static_cast<uint8_t>(n0 | (m0 << 4));
              orow[(c0 + 16 + col_in) / 2] = static_cast<uint8_t>(n1 | (m1 << 4));
            }
            if (col_in == 0)
              osc8[static_cast<size_t>(row) * (g.Nout / 32) + c0 / 32] = static_cast<uint8_t>(code);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= mt_live) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + wm * WM + i * 16 + (lane >> 4) * 4 + v;
        if (row >= row_end) continue;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int ncol = nt * BN + bcol(j) + col_in;
          reinterpret_cast<uint16_t*>(obase)[static_cast<size_t>(row) * g.Nout + ncol] =
              f32_to_bf16(acc[i][j][v]);
        }
      }
    }
  }
}

// tile_off[e+1] = tile_off[e] + ceil(rows_e / BM), segment E = shared (T rows).
__global__ __launch_bounds__(kMaxExperts) void tile_offsets_kernel(const int32_t* __restrict__ offsets,
                                                                   int E, int T_shared, int BM,
                                                                   int32_t* __restrict__ tile_off) {
  __shared__ int32_t s[kMaxExperts];
  const int e = threadIdx.x;
  int t = 0;
  if (e < E) t = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  s[e] = t;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {
    int v = (e >= o) ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) tile_off[e + 1] = s[e];
  if (e == 0) tile_off[0] = 0;
  if (e == E - 1) tile_off[E + 1] = s[e] + (T_shared + BM - 1) / BM;
}

// A8W8: per-row requantisation of the fp32 SwiGLU output, scale = max|row| /
// Q and codes of a / scale: e4m3 (Q = 448) or int8 (Q = 127, half away from
// zero); one block per row.
template <bool I8>
__global__ __launch_bounds__(256) void requant_kernel(const float* __restrict__ A, int f,
                                                      uint8_t* __restrict__ Aq,
                                                      float* __restrict__ a_scale) {
  __shared__ float s_red[4];
  const size_t r = blockIdx.x;
  const float* a = A + r * f;
  float amax = 0.0f;
  for (int c = threadIdx.x * 4; c < f; c += 256 * 4) {
    float4 v = *reinterpret_cast<const float4*>(a + c);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float s = amax > 0.0f ? amax / (I8 ? 127.0f : 448.0f) : 1.0f;
  if (threadIdx.x == 0) a_scale[r] = s;
  for (int c = threadIdx.x * 4; c < f; c += 256 * 4) {
    float4 v = *reinterpret_cast<const float4*>(a + c);
    *reinterpret_cast<uint32_t*>(Aq + r * f + c) =
        I8 ? f32x4_to_i8x4(v.x / s, v.y / s, v.z / s, v.w / s)
           : f32x4_to_e4m3x4(v.x / s, v.y / s, v.z / s, v.w / s);
  }
}

// ---------------------------------------------------------------- fp32 path
// Plain FMA kernels for the fp32 layer (one output element per thread).
__device__ __forceinline__ int find_segment(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__global__ void l1_f32_kernel(FfnArgs a, int rows_routed) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int rows = rows_routed + (a.has_shared ? a.T : 0);
  if (idx >= static_cast<size_t>(rows) * a.f) return;
  const int r = static_cast<int>(idx / a.f), n = static_cast<int>(idx % a.f);
  const float* x;
  const float* W;
  if (r < rows_routed) {
    int e = find_segment(a.offsets, a.E, r);
    x = static_cast<const float*>(a.Xp) + static_cast<size_t>(r) * a.h;
    W = static_cast<const float*>(a.w.W1) + static_cast<size_t>(e) * a.h * 2 * a.f;
  } else {
    x = static_cast<const float*>(a.Xs) + static_cast<size_t>(r - rows_routed) * a.h;
    W = static_cast<const float*>(a.w.Ws1);
  }
  float hg = 0.0f, hu = 0.0f;
  for (int c = 0; c < a.h; ++c) {
    hg = fmaf(x[c], W[static_cast<size_t>(c) * 2 * a.f + n], hg);
    hu = fmaf(x[c], W[static_cast<size_t>(c) * 2 * a.f + a.f + n], hu);
  }
  static_cast<float*>(a.A)[idx] = silu(hg) * hu;
}

__global__ void l2_f32_kernel(FfnArgs a, int rows_routed) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int rows = rows_routed + (a.has_shared ? a.T : 0);
  if (idx >= static_cast<size_t>(rows) * a.h) return;
  const int r = static_cast<int>(idx / a.h), o = static_cast<int>(idx % a.h);
  const float* u = static_cast<const float*>(a.A) + static_cast<size_t>(r) * a.f;
  const float* W;
  float* out;
  if (r < rows_routed) {
    int e = find_segment(a.offsets, a.E, r);
    W = static_cast<const float*>(a.w.W2) + static_cast<size_t>(e) * a.f * a.h;
    out = static_cast<float*>(a.Yp) + static_cast<size_t>(r) * a.h;
  } else {
    W = static_cast<const float*>(a.w.Ws2);
    out = static_cast<float*>(a.Ys) + static_cast<size_t>(r - rows_routed) * a.h;
  }
  float y = 0.0f;
  for (int n = 0; n < a.f; ++n) y = fmaf(u[n], W[static_cast<size_t>(n) * a.h + o], y);
  out[o] = y;
}

template <int PREC, int BM, int BN, int WAVES_M, int WAVES_N, bool SWIGLU, int STAGES>
hipError_t launch_gemm(const GemmArgs& g, int ub_m, hipStream_t stream) {
  if constexpr (PREC == MOE_PREC_MXFP4) {
    // scales in 512-value windows (one 16-byte load per row) where K % 512
    // == 0, else per-stage 4-byte scale loads; 128-value K-stages (whole
    // 128-byte-line stages, KS = 2, need one block per CU and measured slower)
    const dim3 grid(ub_m * g.n_tiles), block(64 * WAVES_M * WAVES_N);
    if (g.K % 512 == 0)
      hipLaunchKernelGGL((grouped_gemm_mx4_kernel<BM, BN, WAVES_M, WAVES_N, SWIGLU, STAGES, 1, true>),
                         grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((grouped_gemm_mx4_kernel<BM, BN, WAVES_M, WAVES_N, SWIGLU, STAGES, 1, false>),
                         grid, block, 0, stream, g);
  } else if constexpr (STAGES >= 3) {
    // bf16: chunks of two m-tiles' worth of items are dealt to the XCDs in
    // turn, which evens out the XCDs' loads when a few segments (the shared
    // expert, hot experts) hold many m-tiles; e4m3 keeps contiguous ranges.
    GemmArgs gg = g;
    gg.chunk = (PREC == MOE_PREC_BF16) ? 2 * g.n_tiles : 0;
    long grid = static_cast<long>(ub_m) * g.n_tiles;
    if (gg.chunk > 0) grid = (grid + 8L * gg.chunk - 1) / (8L * gg.chunk) * (8L * gg.chunk);
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<PREC, BM, BN, WAVES_M, WAVES_N, SWIGLU, STAGES>),
                       dim3(grid), dim3(64 * WAVES_M * WAVES_N), 0, stream, gg);
  } else {
    dim3 grid(ub_m * g.n_tiles);
    hipLaunchKernelGGL((grouped_gemm_kernel<PREC, BM, BN, WAVES_M, WAVES_N, SWIGLU, STAGES>), grid,
                       dim3(64 * WAVES_M * WAVES_N), 0, stream, g);
  }
  return hipGetLastError();
}

template <int PREC, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
hipError_t run_ffn(const FfnArgs& a, hipStream_t stream) {
  const int rows = a.T * a.k;
  const int T_sh = a.has_shared ? a.T : 0;
  hipLaunchKernelGGL(tile_offsets_kernel, dim3(1), dim3(kMaxExperts), 0, stream, a.offsets, a.E,
                     T_sh, BM, a.tile_off);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ub_m = (rows + BM - 1) / BM + (a.E < rows ? a.E : rows) + (T_sh + BM - 1) / BM;
  constexpr bool MX = PREC == MOE_PREC_MXFP8 || PREC == MOE_PREC_MXFP4;
  constexpr bool A8W8 = PREC == MOE_PREC_FP8 || PREC == MOE_PREC_INT8;
  constexpr bool Q8 = A8W8 || MX;  // quantised activation codes into Linear2
  // bytes of one row of the SwiGLU output as Linear2 reads it
  const size_t arow_bytes = PREC == MOE_PREC_MXFP4 ? a.f / 2 : static_cast<size_t>(a.f) * (Q8 ? 1 : 2);

  GemmArgs g1{};
  g1.A = a.src_tok ? a.Xs : a.Xp;
  g1.gather = a.src_tok;
  g1.A_sh = a.Xs;
  g1.a_scale = a.xp_scale;
  g1.a_scale_sh = a.xs_scale;
  g1.W = a.w.W1;
  g1.W_sh = a.w.Ws1;
  g1.w_scale = a.w.w1_scale;
  g1.w_scale_sh = a.w.ws1_scale;
  if (MX) {  // the SwiGLU output is MX-quantised by the Linear1 epilogue
    g1.out = a.Aq;
    g1.out_sh = static_cast<char*>(a.Aq) + static_cast<size_t>(rows) * arow_bytes;
    g1.out_scale = a.a_scale;
    g1.out_scale_sh = static_cast<char*>(a.a_scale) + static_cast<size_t>(rows) * (a.f / 32);
  } else {
    g1.out = a.A;
    g1.out_sh = static_cast<char*>(a.A) +
                static_cast<size_t>(rows) * a.f * (A8W8 ? 4 : 2);
  }
  g1.offsets = a.offsets;
  g1.tile_off = a.tile_off;
  g1.E = a.E;
  g1.K = a.h;
  g1.Nw = 2 * a.f;
  g1.Nout = a.f;
  g1.f = a.f;
  g1.T = a.T;
  g1.n_tiles = 2 * a.f / BN;
  err = launch_gemm<PREC, BM, BN, WAVES_M, WAVES_N, true, STAGES>(g1, ub_m, stream);
  if (err != hipSuccess) return err;

  const void* A2 = a.A;
  const char* as2 = nullptr;
  if (A8W8) {
    const int arows = rows + T_sh;
    hipLaunchKernelGGL(requant_kernel<PREC == MOE_PREC_INT8>, dim3(arows), dim3(256), 0, stream,
                       static_cast<const float*>(a.A), a.f, static_cast<uint8_t*>(a.Aq),
                       static_cast<float*>(a.a_scale));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (Q8) {
    A2 = a.Aq;
    as2 = static_cast<const char*>(a.a_scale);
  }
  GemmArgs g2{};
  g2.A = A2;
  g2.A_sh = static_cast<const char*>(A2) + static_cast<size_t>(rows) * arow_bytes;
  g2.a_scale = as2;
  g2.a_scale_sh = as2 ? as2 + static_cast<size_t>(rows) * (MX ? a.f / 32 : 4) : nullptr;
  g2.W = a.w.W2;
  g2.W_sh = a.w.Ws2;
  g2.w_scale = a.w.w2_scale;
  g2.w_scale_sh = a.w.ws2_scale;
  g2.out = a.Yp;
  g2.out_sh = a.Ys;
  g2.offsets = a.offsets;
  g2.tile_off = a.tile_off;
  g2.E = a.E;
  g2.K = a.f;
  g2.Nw = a.h;
  g2.Nout = a.h;
  g2.f = a.f;
  g2.T = a.T;
  g2.n_tiles = a.h / BN;
  return launch_gemm<PREC, BM, BN, WAVES_M, WAVES_N, false, STAGES>(g2, ub_m, stream);
}

template <int PREC>
hipError_t dispatch_ffn(const FfnArgs& a, hipStream_t stream) {
  const int rows = a.T * a.k;
  // Decode-sized batches (a few rows per expert) are weight streams.  For
  // bf16 with 512-wide n-tiles the DMA pipeline streams them fastest (only an
  // expert's live rows are fetched and multiplied, and one block per CU keeps
  // three 40 KB stages of weight slices in flight); otherwise they run 16-row
  // tiles with one LDS stage, so more blocks fit on a CU.  N tiles of 256
  // need hidden and 2*inter to be multiples of 256, else 128.
  const bool w512 = (a.h % 512 == 0) && ((2 * a.f) % 512 == 0);
  const bool small = static_cast<long>(rows) < 16L * a.E && !(PREC == MOE_PREC_BF16 && w512);
  const bool wide = (a.h % 256 == 0) && ((2 * a.f) % 256 == 0);
  if (small)
    return wide ? run_ffn<PREC, 16, 256, 1, 4, 1>(a, stream)
                : run_ffn<PREC, 16, 128, 1, 4, 1>(a, stream);
  if constexpr (PREC == MOE_PREC_FP8) {
    // e4m3: 128 x 512 tiles on 8 waves (64 x 128 per wave, 32x32x64 MFMA,
    // 64-value stages) where hidden and 2 * inter allow, which halves the
    // re-reads of token-row tiles (one per n-tile) against 256-wide tiles;
    // else 128 x 256 (64 x 64 per wave, 16x16x128, 128-value stages).  Either
    // ring takes most of the LDS (120 / 144 KB): one block per CU, and its 8
    // waves are two per SIMD to cover each other's LDS and DMA waits
    if ((a.h % 512 == 0) && ((2 * a.f) % 512 == 0)) return run_ffn<PREC, 128, 512, 2, 4, 3>(a, stream);
    return run_ffn<PREC, 128, 256, 2, 4, 3>(a, stream);
  } else {
    if (!wide) return run_ffn<PREC, 128, 128, 2, 2, 2>(a, stream);
    // 128 x 512 tiles on 8 waves (the ping-pong schedule) wherever hidden and
    // 2 * inter allow: every m-tile's token rows are read once per n-tile,
    // and 512-wide n-tiles halve that against 256.  With DMAs issued between
    // the MFMAs they are also faster than two 4-wave 128 x 256 blocks per CU
    // on experts of many rows (measured: EP-share 2.94 -> 2.79 ms, Llama-
    // shaped 3.90 -> 3.29 ms).  Decode-sized batches are pure weight
    // streams: a 4-stage ring (all 160 KB of LDS) keeps a third stage in
    // flight (measured: decode 3.8% faster, V4-Pro prefill 2% slower).
    if (w512 && static_cast<long>(rows) < 16L * a.E)
      return run_ffn<PREC, 128, 512, 2, 4, 4>(a, stream);
    if (w512) return run_ffn<PREC, 128, 512, 2, 4, 3>(a, stream);
    return run_ffn<PREC, 128, 256, 2, 2, 3>(a, stream);
  }
}

}  // namespace

hipError_t launch_grouped_linear_bf16(const LinearArgs& a, hipStream_t stream) {
  constexpr int BM = 128;
  const int T_sh = a.has_shared ? a.T : 0;
  hipLaunchKernelGGL(tile_offsets_kernel, dim3(1), dim3(kMaxExperts), 0, stream, a.offsets, a.E,
                     T_sh, BM, a.tile_off);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ub_m = (a.rows + BM - 1) / BM + (a.E < a.rows ? a.E : a.rows) + (T_sh + BM - 1) / BM;
  GemmArgs g{};
  g.A = a.A;
  g.A_sh = a.A_sh;
  g.W = a.W;
  g.W_sh = a.W_sh;
  g.out = a.out;
  g.out_sh = a.out_sh;
  g.offsets = a.offsets;
  g.tile_off = a.tile_off;
  g.E = a.E;
  g.K = a.K;
  g.Nw = a.N;
  g.Nout = a.N;
  g.T = a.T;
  // tile width as the expert FFN chooses it (512-wide n-tiles on the
  // ping-pong schedule wherever N allows)
  if (a.N % 512 == 0) {
    g.n_tiles = a.N / 512;
    return launch_gemm<MOE_PREC_BF16, BM, 512, 2, 4, false, 3>(g, ub_m, stream);
  }
  if (a.N % 256 == 0) {
    g.n_tiles = a.N / 256;
    return launch_gemm<MOE_PREC_BF16, BM, 256, 2, 2, false, 3>(g, ub_m, stream);
  }
  g.n_tiles = a.N / 128;
  return launch_gemm<MOE_PREC_BF16, BM, 128, 2, 2, false, 2>(g, ub_m, stream);
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream) {
  if (a.src_tok && !ffn_gathers(a.precision, a.T, a.h, a.E, a.k, a.f)) return hipErrorInvalidValue;
  const int rows = a.T * a.k;
  if (a.precision == MOE_PREC_F32) {
    const int T_sh = a.has_shared ? a.T : 0;
    size_t n1 = static_cast<size_t>(rows + T_sh) * a.f;
    hipLaunchKernelGGL(l1_f32_kernel, dim3((n1 + 255) / 256), dim3(256), 0, stream, a, rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    size_t n2 = static_cast<size_t>(rows + T_sh) * a.h;
    hipLaunchKernelGGL(l2_f32_kernel, dim3((n2 + 255) / 256), dim3(256), 0, stream, a, rows);
    return hipGetLastError();
  }
  if (a.precision == MOE_PREC_BF16) return dispatch_ffn<MOE_PREC_BF16>(a, stream);
  // MX: the 3-stage DMA pipeline at every batch size (the 16-row decode
  // kernel has no per-group scales)
  if (a.precision == MOE_PREC_MXFP8) {
    // 128 x 512 tiles (32x32x64 scaled MFMA) where hidden and 2 * inter allow
    if ((a.h % 512 == 0) && ((2 * a.f) % 512 == 0))
      return run_ffn<MOE_PREC_MXFP8, 128, 512, 2, 4, 3>(a, stream);
    return run_ffn<MOE_PREC_MXFP8, 128, 256, 2, 4, 3>(a, stream);
  }
  // MXFP4: 128 x 256 tiles on 8 waves, a 2-stage ring of 128-value K-stages
  // plus two 6 KB scale windows (60 KB), two blocks per CU
  if (a.precision == MOE_PREC_MXFP4) return run_ffn<MOE_PREC_MXFP4, 128, 256, 2, 4, 2>(a, stream);
  // INT8: the e4m3 tiles (128 x 512 where hidden and 2 * inter allow, else
  // 128 x 256; 8 waves, 3-stage ring) at every batch size (the 16-row decode
  // kernel has no int8 form)
  if (a.precision == MOE_PREC_INT8) {
    if ((a.h % 512 == 0) && ((2 * a.f) % 512 == 0))
      return run_ffn<MOE_PREC_INT8, 128, 512, 2, 4, 3>(a, stream);
    return run_ffn<MOE_PREC_INT8, 128, 256, 2, 4, 3>(a, stream);
  }
  return dispatch_ffn<MOE_PREC_FP8>(a, stream);
}

}  // namespace moe
