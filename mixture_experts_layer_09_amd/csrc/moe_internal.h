// moe_internal.h -- types, device helpers, workspace layout and launcher
// declarations shared by the HIP kernels and the C ABI of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- vectors
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

// ---------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> bf16 (round to nearest even) packed low, high, by the
// hardware conversion v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

// fp32 -> OCP e4m3fn code, round to nearest even, saturating at +-448.  The
// clamp makes the hardware conversion's out-of-range behaviour irrelevant:
// every value that reaches it lies in [-448, 448].
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false)) & 0xffu;
}

// Four fp32 -> four e4m3 codes packed little-endian in one word.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// INT8 code of v (the A8W8 block's ⌊v⌉): rounded half away from zero
// (roundf), clamped to [-127, 127], as the low byte of the result.
__device__ __forceinline__ uint32_t f32_to_i8(float v) {
  const float r = fminf(fmaxf(roundf(v), -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
}
__device__ __forceinline__ uint32_t f32x4_to_i8x4(float a, float b, float c, float d) {
  return f32_to_i8(a) | (f32_to_i8(b) << 8) | (f32_to_i8(c) << 16) | (f32_to_i8(d) << 24);
}

// fp32 -> OCP e2m1 (FP4) code in the low 4 bits: nearest of 0, 0.5, 1, 1.5,
// 2, 3, 4, 6 with ties to the even code (the midpoints 0.25, 1.25, 2.5, 5
// round down, 0.75, 1.75, 3.5 round up), saturating at 6; the sign is bit 3.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------- workspace
constexpr size_t kAlign = 256;
constexpr int kPermChunk = 2048;   // assignments per counting block of the dispatch
constexpr int kPermThreads = 1024; // its threads: two assignments each
constexpr int kMaxExperts = 512;
constexpr int kMaxTopk = 16;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline size_t act_bytes(int precision) { return precision == MOE_PREC_F32 ? 4 : 2; }
// bytes of one dispatched (or quantised) row of n elements
inline size_t xrow_bytes(int precision, size_t n) {
  if (precision == MOE_PREC_F32) return 4 * n;
  if (precision == MOE_PREC_BF16) return 2 * n;
  return precision == MOE_PREC_MXFP4 ? n / 2 : n;
}
inline bool is_mx(int precision) {
  return precision == MOE_PREC_MXFP8 || precision == MOE_PREC_MXFP4;
}
// bytes of the activation scales of one row of `n` elements
inline size_t row_scale_bytes(int precision, size_t n) {
  if (is_mx(precision)) return n / 32;
  return (precision == MOE_PREC_FP8 || precision == MOE_PREC_INT8) ? 4 : 0;
}

// The router's launch plan: which gate kernel, tokens per block and
// K-splits of the gating linear (route_plan.cpp), and the bytes of fp32
// partial gate logits it uses in the workspace (0 if none).
struct RoutePlan {
  int dma;  // 1: DMA-fed bf16 gate GEMM + top-k kernel; 0: register-staged gate kernel
  int bm, splits;
};
RoutePlan route_plan(int T, int h, int E, int precision);
size_t route_partial_bytes(int T, int h, int E, int precision);

// Byte offsets of every region inside the caller's workspace.
struct Layout {
  size_t flag;        // int32 error flag, then one error byte per counting block (padded to 256 B)
  size_t part;        // router: fp32 partial logits [splits, T, E]
  size_t blk_cnt;     // [nblk, E] int32 per-block expert counts
  size_t local_rank;  // [T*k] int32 rank of an assignment inside its block
  size_t tile_off;    // [E+2] int32 m-tile prefix of the grouped GEMM
  size_t counts, offsets, dst_row, src_tok;  // forward-internal dispatch results
  size_t Xp, xp_scale, Xq, x_scale;          // forward-internal dispatched rows
  size_t A;                                  // [T*k + T*S, f] SwiGLU output (not for MX)
  size_t Aq, a_scale;                        // FP8 / MX: quantised SwiGLU output
  size_t Yp, Ys;                             // forward-internal expert outputs
  size_t total;
  int nblk;
};

inline Layout make_layout(const moe_shape& s) {
  Layout L{};
  size_t T = s.tokens, h = s.hidden, E = s.experts, k = s.topk, f = s.inter;
  size_t rows = T * k, arows = rows + (s.has_shared ? T : 0);
  L.nblk = static_cast<int>((rows + kPermChunk - 1) / kPermChunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.flag = take(4 + static_cast<size_t>(L.nblk));  // flag word + the dispatch's per-block error bytes
  L.part = take(route_partial_bytes(s.tokens, s.hidden, s.experts, s.precision));
  L.blk_cnt = take(static_cast<size_t>(L.nblk) * E * 4);
  L.local_rank = take(rows * 4);
  L.tile_off = take((E + 2) * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.dst_row = take(rows * 4);
  L.src_tok = take(rows * 4);
  L.Xp = take(rows * xrow_bytes(s.precision, h));
  const bool q8 = s.precision >= MOE_PREC_FP8;  // quantised activations (A8W8 or MX)
  const bool mx = is_mx(s.precision);
  L.xp_scale = take(rows * row_scale_bytes(s.precision, h));
  L.Xq = take(q8 ? T * xrow_bytes(s.precision, h) : 0);
  L.x_scale = take(T * row_scale_bytes(s.precision, h));
  L.A = take(mx ? 0 : arows * f * (q8 ? 4 : act_bytes(s.precision)));
  L.Aq = take(q8 ? arows * xrow_bytes(s.precision, f) : 0);
  L.a_scale = take(arows * row_scale_bytes(s.precision, f));
  L.Yp = take(rows * h * act_bytes(s.precision));
  L.Ys = take(s.has_shared ? T * h * act_bytes(s.precision) : 0);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already valid.
struct RouteArgs {
  int T, h, E, k, precision, score_fn, renorm;
  float alpha;
  const void* X;
  const void* Wg;
  const float* beta;
  const float* gate_bias;
  const int32_t* token_ids;
  const int32_t* tid2eid;
  int vocab;
  int32_t* ids;
  float* G;
  float* keys;
  int32_t* flag;
  float* part;  // workspace for split-K partial logits
};
// Clears the error flag a.flag, then routes (hash routing may set the flag).
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

struct PermuteArgs {
  int T, h, E, k, precision, nblk;
  const int32_t* ids;
  const void* X;
  int32_t* counts;
  int32_t* offsets;
  int32_t* dst_row;
  int32_t* src_tok;
  void* Xp;
  void* xp_scale;  // fp32 per row (FP8) or E8M0 bytes [rows, h/32] (MX)
  void* Xq;
  void* x_scale;
  int32_t* blk_cnt;
  int32_t* local_rank;
  int32_t* flag;
  int maps_only;  // 1: the row maps dst_row and src_tok only, no rows copied (Xp unused)
  int clear_flag;  // 1: the dispatch writes the error flag (clear unless a bad id); 0: only sets it
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);
// launch_permute with the flag, per-block counts and ranks in the library's
// static scratch of this device (a's workspace pointers are ignored).
hipError_t launch_permute_no_alloc(PermuteArgs a, hipStream_t stream);

struct FfnArgs {
  int T, h, E, k, f, has_shared, precision;
  const void* Xp;
  const void* xp_scale;
  const int32_t* offsets;
  const void* Xs;
  const void* xs_scale;
  moe_expert_weights w;
  void* Yp;
  void* Ys;
  void* A;  // [T*k + T*S, f] (fp32 for FP8; unused for MX)
  void* Aq;
  void* a_scale;
  int32_t* tile_off;
  // Non-null: Linear1 reads routed row r as token row src_tok[r] of Xs (the
  // layer input) instead of row r of Xp; only where ffn_gathers() allows it.
  const int32_t* src_tok;
};
hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream);
// Whether launch_expert_ffn can take its Linear1 rows from the layer input by
// the row -> token map (FfnArgs::src_tok) for this shape: bf16 where Linear1
// runs on the DMA kernel, with every byte offset into X below 2^32.
bool ffn_gathers(int precision, int T, int h, int E, int k, int f);

struct CombineArgs {
  int T, h, k, precision;
  const void* Yp;
  const int32_t* dst_row;
  const float* G;
  const void* Ys;
  void* Y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

hipError_t launch_clear_flag(int32_t* flag, hipStream_t stream);

// Plain grouped linear (bf16, fp32 accumulation, no activation): out[r] =
// A[r] W[e] for the rows r of expert e's block [offsets[e], offsets[e+1]),
// then the shared rows (A_sh, W_sh, out_sh; T rows) when has_shared.  W is
// [E, K, N] (N contiguous); A rows K, out rows N elements.
struct LinearArgs {
  const void* A;
  const void* A_sh;
  const void* W;
  const void* W_sh;
  void* out;
  void* out_sh;
  const int32_t* offsets;
  int32_t* tile_off;  // [E+2] scratch
  int E, K, N, T, rows, has_shared;
};
hipError_t launch_grouped_linear_bf16(const LinearArgs& a, hipStream_t stream);

// Workspace of the backward: the forward's regions (make_layout) followed by
// the recomputed activations and the gradients in flight.
struct BwdLayout {
  size_t H1;       // [arows, 2f] bf16: Linear1 pre-activations (gate, up)
  size_t Aact;     // [arows, f] bf16: SwiGLU output times the row's gate weight
                   // (shared rows: 1), the left operand of dW2
  size_t Afwd;     // [arows, f] bf16: SwiGLU output, the training forward's Linear2 input
  size_t grow;     // [rows] fp32: gate weight of each dispatched row
  size_t dGp;      // [rows, f/64] fp32: partial dG of each row per 64 columns of Linear2's dgrad
  size_t dYp;      // [rows, h] bf16: upstream gradient dY[t] copied to each row of token t
  size_t dH1;      // [arows, 2f] bf16: gradient of the pre-activations
  size_t dXp;      // [arows, h] bf16: dgrad of the dispatched rows (+ shared)
  size_t dXr;      // [T, h] bf16: router part of dX
  size_t keys;     // [T, E] fp32: recomputed router keys
  size_t ids_s;    // [T, k] int32 scratch of the recomputed router
  size_t G_s;      // [T, k] fp32 scratch
  size_t dG;       // [T, k] fp32
  size_t dl32;     // [T, E] fp32: gradient of the gating logits
  size_t dl16;     // [T, E] bf16
  size_t tile_b;   // [E+2] int32: m-tile prefix of the dgrad kernels
  size_t colsum;   // [ceil(T/256), E] fp32: partial column sums of dl (gating bias gradient)
  size_t total;
};
inline BwdLayout make_bwd_layout(const moe_shape& s) {
  const Layout F = make_layout(s);
  BwdLayout B{};
  size_t T = s.tokens, h = s.hidden, E = s.experts, k = s.topk, f = s.inter;
  size_t rows = T * k, arows = rows + (s.has_shared ? T : 0);
  size_t o = F.total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  B.H1 = take(arows * 2 * f * 2);
  B.Aact = take(arows * f * 2);
  B.Afwd = take(arows * f * 2);
  B.grow = take(rows * 4);
  B.dGp = take(rows * (f / 64) * 4);
  B.dYp = take(rows * h * 2);
  B.dH1 = take(arows * 2 * f * 2);
  B.dXp = take(arows * h * 2);
  B.dXr = take(T * h * 2);
  B.keys = take(T * E * 4);
  B.ids_s = take(T * k * 4);
  B.G_s = take(T * k * 4);
  B.dG = take(T * k * 4);
  B.dl32 = take(T * E * 4);
  B.dl16 = take(T * E * 2);
  B.tile_b = take((E + 2) * 4);
  B.colsum = take((T + 255) / 256 * E * 4);
  B.total = o;
  return B;
}

struct BackwardArgs {
  int T, h, E, k, f, has_shared;
  int route;  // 1: differentiate the router (score_fn, renorm, alpha, beta, hash below)
  int score_fn, renorm, hash;
  float alpha;
  const float* beta;
  const void* X;      // [T, h] bf16
  const void* Wg;     // [h, E] bf16
  const void* W1;     // [E, h, 2f]
  const void* W2;     // [E, f, h]
  const void* Ws1;
  const void* Ws2;
  const int32_t* ids; // [T, k] the forward's routing
  const float* G;     // [T, k]
  const void* dY;     // [T, h] bf16
  // the forward's dispatch and recomputed activations (workspace)
  const int32_t* offsets;
  const int32_t* dst_row;
  const void* Xp;
  const float* grow;  // [rows] gate weight of each dispatched row
  // workspace regions (BwdLayout)
  void* H1;
  void* Aact;
  float* dGp;
  void* dYp;
  void* dH1;
  void* dXp;
  void* dXr;
  const float* keys;
  float* dG;
  float* dl32;
  void* dl16;
  int32_t* tile_off;  // forward linears' m-tile prefix scratch
  int32_t* tile_b;
  float* colsum;      // [ceil(T/256), E] partial column sums of dl
  // outputs
  void* dX;
  void* dWg;
  float* dgate_bias;
  void* dW1;
  void* dW2;
  void* dWs1;
  void* dWs2;
};
// Everything after the forward recompute: unpermute backward, the experts'
// dgrad and wgrad, router backward (when route), permute backward.
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);
// grow[dst_row[i]] = G[i] for the n dispatched assignments (skipped ones have
// no row).
hipError_t launch_row_gate(const int32_t* dst_row, const float* G, int n, float* grow,
                           hipStream_t stream);
// A = SiLU(H1[:, :f]) * H1[:, f:] for `arows` rows (bf16): Aw gets A times
// grow[r] for the first `rows` rows and A itself for the rest; Af (if not
// NULL) gets A.
hipError_t launch_swiglu_bf16(const void* H1, int f, long rows, long arows, const float* grow,
                              void* Aw, void* Af, hipStream_t stream);

}  // namespace moe
