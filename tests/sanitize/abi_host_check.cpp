// abi_host_check.cpp -- the host side of libmoe's C ABI (moe_api.cpp, the
// workspace layout and the router's launch plan) under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU.
//
// The kernel launchers are replaced by stubs that read the first and the
// last byte of every buffer a launch would touch, at the sizes its kernels
// use; every "device" buffer, the workspace included, is a host allocation
// of exactly the size the header documents (the workspace: the size that
// moe_workspace_size / moe_backward_workspace_size report).  So a workspace
// region that runs past the workspace, or a buffer passed with the wrong
// size, is a heap overflow that the sanitizer reports; signed overflow or a
// misaligned access in the shape arithmetic is undefined behaviour it
// reports.  The entry points are called with valid arguments for every
// precision (and the backward), then with out-of-contract ones, whose
// status is checked.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../mixture_experts_layer_09_amd/csrc/moe_internal.h"

namespace {

int g_launches = 0;
int g_overlaps = 0;
int g_stub_fail = 0;  // a launch stub found its arguments inconsistent
// the workspace of the current calls, and the workspace regions one launch
// touches (they must be disjoint)
const unsigned char* g_ws_lo = nullptr;
const unsigned char* g_ws_hi = nullptr;
std::vector<std::pair<const unsigned char*, size_t>> g_regions;

void touch(const void* p, size_t bytes) {
  if (!p || bytes == 0) return;
  const volatile unsigned char* c = static_cast<const volatile unsigned char*>(p);
  (void)c[0];
  (void)c[bytes - 1];
  const unsigned char* q = static_cast<const unsigned char*>(p);
  if (q >= g_ws_lo && q < g_ws_hi) {
    for (const auto& r : g_regions)
      if (q < r.first + r.second && r.first < q + bytes) {
        std::fprintf(stderr, "FAIL workspace regions overlap: [%td, +%zu) and [%td, +%zu)\n",
                     r.first - g_ws_lo, r.second, q - g_ws_lo, bytes);
        ++g_overlaps;
      }
    g_regions.emplace_back(q, bytes);
  }
}

// called at the start of every launch stub
void new_launch() { g_regions.clear(); }

size_t act(int prec) { return prec == MOE_PREC_F32 ? 4 : 2; }
size_t wbytes(int prec) {
  return prec == MOE_PREC_F32 ? 4 : prec == MOE_PREC_BF16 ? 2 : 1;
}

}  // namespace

// ------------------------------------------------------------------ launcher stubs
namespace moe {

hipError_t launch_clear_flag(int32_t* flag, hipStream_t) {
  new_launch();
  touch(flag, 4);
  *flag = 0;  // what the kernel does
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t) {
  new_launch();
  const size_t T = a.T, h = a.h, E = a.E, k = a.k;
  touch(a.X, T * h * act(a.precision));
  touch(a.Wg, h * E * act(a.precision));
  touch(a.beta, a.beta ? E * 4 : 0);
  touch(a.gate_bias, a.gate_bias ? E * 4 : 0);
  touch(a.token_ids, a.token_ids ? T * 4 : 0);
  touch(a.tid2eid, a.tid2eid ? static_cast<size_t>(a.vocab) * k * 4 : 0);
  touch(a.ids, T * k * 4);
  touch(a.G, T * k * 4);
  touch(a.keys, a.keys ? T * E * 4 : 0);
  touch(a.flag, 4);
  *a.flag = 0;  // the router clears the error flag first
  touch(a.part, route_partial_bytes(a.T, a.h, a.E, a.precision));
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t) {
  new_launch();
  const size_t T = a.T, h = a.h, E = a.E, k = a.k, n = T * k;
  touch(a.ids, n * 4);
  touch(a.X, T * h * act(a.precision == MOE_PREC_F32 ? MOE_PREC_F32 : MOE_PREC_BF16));
  touch(a.counts, E * 4);
  touch(a.offsets, (E + 1) * 4);
  touch(a.dst_row, n * 4);
  touch(a.src_tok, n * 4);
  if (!a.maps_only) touch(a.Xp, n * xrow_bytes(a.precision, h));
  if (a.precision >= MOE_PREC_FP8) {
    touch(a.xp_scale, n * row_scale_bytes(a.precision, h));
    touch(a.Xq, T * xrow_bytes(a.precision, h));
    touch(a.x_scale, T * row_scale_bytes(a.precision, h));
  }
  touch(a.blk_cnt, static_cast<size_t>(a.nblk) * E * 4);
  touch(a.local_rank, n * 4);
  touch(a.flag, 4 + static_cast<size_t>(a.nblk));  // flag word + per-block error bytes
  if (a.clear_flag) *a.flag = 0;  // what the scan kernel writes when no id was bad
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_permute_no_alloc(PermuteArgs a, hipStream_t stream) {
  // the kernels' scratch is the library's static array, not a workspace
  static std::vector<int32_t> flag, blk, rank;
  flag.assign(1 + (static_cast<size_t>(a.nblk) + 3) / 4, 0);  // flag word + error bytes
  blk.assign(static_cast<size_t>(a.nblk) * a.E, 0);
  rank.assign(static_cast<size_t>(a.T) * a.k, 0);
  a.flag = flag.data();
  a.clear_flag = 1;
  a.blk_cnt = blk.data();
  a.local_rank = rank.data();
  return launch_permute(a, stream);
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t) {
  new_launch();
  const size_t T = a.T, h = a.h, E = a.E, k = a.k, f = a.f, rows = T * k;
  const size_t arows = rows + (a.has_shared ? T : 0);
  const int p = a.precision;
  const bool q8 = p >= MOE_PREC_FP8, mx = is_mx(p);
  if (a.src_tok) {  // Linear1 gathers token rows of Xs by the row -> token map
    if (!ffn_gathers(p, a.T, a.h, a.E, a.k, a.f)) {
      std::fprintf(stderr, "FAIL expert FFN gathers on a shape that does not allow it\n");
      ++g_stub_fail;
    }
    touch(a.src_tok, rows * 4);
    touch(a.Xs, T * xrow_bytes(p, h));
  } else {
    touch(a.Xp, rows * xrow_bytes(p, h));
  }
  if (q8) touch(a.xp_scale, rows * row_scale_bytes(p, h));
  touch(a.offsets, (E + 1) * 4);
  touch(a.w.W1, E * h * 2 * f * wbytes(p) / (p == MOE_PREC_MXFP4 ? 2 : 1));
  touch(a.w.W2, E * f * h * wbytes(p) / (p == MOE_PREC_MXFP4 ? 2 : 1));
  if (a.has_shared) {
    touch(a.Xs, T * xrow_bytes(p, h));
    if (q8) touch(a.xs_scale, T * row_scale_bytes(p, h));
    touch(a.w.Ws1, h * 2 * f * wbytes(p) / (p == MOE_PREC_MXFP4 ? 2 : 1));
    touch(a.w.Ws2, f * h * wbytes(p) / (p == MOE_PREC_MXFP4 ? 2 : 1));
    touch(a.Ys, T * h * act(p == MOE_PREC_F32 ? p : MOE_PREC_BF16));
  }
  touch(a.Yp, rows * h * act(p == MOE_PREC_F32 ? p : MOE_PREC_BF16));
  if (!mx) touch(a.A, arows * f * (q8 ? 4 : act(p)));
  if (q8) {
    touch(a.Aq, arows * xrow_bytes(p, f));
    touch(a.a_scale, arows * row_scale_bytes(p, f));
  }
  touch(a.tile_off, (E + 2) * 4);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t) {
  new_launch();
  const size_t T = a.T, h = a.h, k = a.k;
  const size_t ab = act(a.precision == MOE_PREC_F32 ? MOE_PREC_F32 : MOE_PREC_BF16);
  touch(a.Yp, T * k * h * ab);
  touch(a.dst_row, T * k * 4);
  touch(a.G, T * k * 4);
  touch(a.Ys, a.Ys ? T * h * ab : 0);
  touch(a.Y, T * h * ab);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_grouped_linear_bf16(const LinearArgs& a, hipStream_t) {
  new_launch();
  const size_t K = a.K, N = a.N, E = a.E, T = a.T;
  touch(a.A, static_cast<size_t>(a.rows) * K * 2);
  touch(a.W, E * K * N * 2);
  touch(a.out, static_cast<size_t>(a.rows) * N * 2);
  if (a.has_shared) {
    touch(a.A_sh, T * K * 2);
    touch(a.W_sh, K * N * 2);
    touch(a.out_sh, T * N * 2);
  }
  touch(a.offsets, (E + 1) * 4);
  touch(a.tile_off, (E + 2) * 4);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_swiglu_bf16(const void* H1, int f, long rows, long arows, const float* grow,
                              void* Aw, void* Af, hipStream_t) {
  new_launch();
  touch(H1, static_cast<size_t>(arows) * 2 * f * 2);
  touch(grow, static_cast<size_t>(rows) * 4);
  touch(Aw, static_cast<size_t>(arows) * f * 2);
  touch(Af, Af ? static_cast<size_t>(arows) * f * 2 : 0);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_row_gate(const int32_t* dst_row, const float* G, int n, float* grow, hipStream_t) {
  new_launch();
  touch(dst_row, static_cast<size_t>(n) * 4);
  touch(G, static_cast<size_t>(n) * 4);
  touch(grow, static_cast<size_t>(n) * 4);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t) {
  new_launch();
  const size_t T = a.T, h = a.h, E = a.E, k = a.k, f = a.f, rows = T * k;
  const size_t arows = rows + (a.has_shared ? T : 0);
  touch(a.X, T * h * 2);
  touch(a.W1, E * h * 2 * f * 2);
  touch(a.W2, E * f * h * 2);
  touch(a.ids, rows * 4);
  touch(a.G, rows * 4);
  touch(a.dY, T * h * 2);
  touch(a.offsets, (E + 1) * 4);
  touch(a.dst_row, rows * 4);
  touch(a.Xp, rows * h * 2);
  touch(a.grow, rows * 4);
  touch(a.H1, arows * 2 * f * 2);
  touch(a.Aact, arows * f * 2);
  touch(a.dGp, rows * (f / 64) * 4);
  touch(a.dYp, rows * h * 2);
  touch(a.dH1, arows * 2 * f * 2);
  touch(a.dXp, arows * h * 2);
  touch(a.dXr, T * h * 2);
  touch(a.keys, T * E * 4);
  touch(a.dG, rows * 4);
  touch(a.dl32, T * E * 4);
  touch(a.dl16, T * E * 2);
  touch(a.tile_off, (E + 2) * 4);
  touch(a.tile_b, (E + 2) * 4);
  touch(a.colsum, (T + 255) / 256 * E * 4);
  touch(a.dX, T * h * 2);
  touch(a.dW1, E * h * 2 * f * 2);
  touch(a.dW2, E * f * h * 2);
  if (a.has_shared) {
    touch(a.Ws1, h * 2 * f * 2);
    touch(a.Ws2, f * h * 2);
    touch(a.dWs1, h * 2 * f * 2);
    touch(a.dWs2, f * h * 2);
  }
  if (a.route) {
    touch(a.Wg, h * E * 2);
    touch(a.dWg, a.dWg ? h * E * 2 : 0);
    touch(a.dgate_bias, a.dgate_bias ? E * 4 : 0);
    touch(a.beta, a.beta ? E * 4 : 0);
  }
  ++g_launches;
  return hipSuccess;
}

}  // namespace moe

// moe_check_device_error's runtime calls, on host memory
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
extern "C" hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}

// ------------------------------------------------------------------ driver
namespace {

int g_fail = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++g_fail;
  }
}

// A host "device" buffer of `bytes` (256-byte aligned, zeroed).
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t bytes) {
    if (bytes) {
      p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
      std::memset(p, 0, (bytes + 255) / 256 * 256);
    }
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

void run_shape(int T, int h, int E, int k, int f, int shared, int prec, bool hash) {
  moe_shape s{T, h, E, k, f, shared, prec};
  const size_t ws_bytes = moe_workspace_size(&s);
  if (ws_bytes == 0) {
    std::fprintf(stderr, "FAIL moe_workspace_size == 0 for a valid shape\n");
    ++g_fail;
    return;
  }
  // the workspace: exactly ws_bytes (the layout rounds every region to 256
  // bytes, so the size is a multiple of the alignment and a read past the
  // last region is past the allocation)
  if (ws_bytes % 256 != 0) {
    std::fprintf(stderr, "FAIL workspace size %zu is not a multiple of 256\n", ws_bytes);
    ++g_fail;
  }
  void* W = std::aligned_alloc(256, ws_bytes);
  g_ws_lo = static_cast<unsigned char*>(W);
  g_ws_hi = g_ws_lo + ws_bytes;
  const size_t ab = prec == MOE_PREC_F32 ? 4 : 2;
  const size_t wb = wbytes(prec);
  const size_t n = static_cast<size_t>(T) * k;
  const bool fp4 = prec == MOE_PREC_MXFP4;
  Buf X(static_cast<size_t>(T) * h * ab), Wg(static_cast<size_t>(h) * E * ab);
  Buf ids(n * 4), G(n * 4), keys(static_cast<size_t>(T) * E * 4), beta(E * 4), gb(E * 4);
  Buf tok(T * 4), tid(static_cast<size_t>(1000) * k * 4);
  Buf counts(E * 4), offsets((E + 1) * 4), dst(n * 4), src(n * 4);
  Buf Xp(n * moe::xrow_bytes(prec, h)), xps(n * (moe::row_scale_bytes(prec, h) ? moe::row_scale_bytes(prec, h) : 4));
  Buf Xq(static_cast<size_t>(T) * moe::xrow_bytes(prec, h)),
      xs(static_cast<size_t>(T) * (moe::row_scale_bytes(prec, h) ? moe::row_scale_bytes(prec, h) : 4));
  const size_t w1 = static_cast<size_t>(E) * h * 2 * f * wb / (fp4 ? 2 : 1);
  const size_t w2 = static_cast<size_t>(E) * f * h * wb / (fp4 ? 2 : 1);
  Buf W1(w1), W2(w2), Ws1(w1 / E), Ws2(w2 / E);
  const size_t sc1 = moe::is_mx(prec) ? static_cast<size_t>(E) * h / 32 * 2 * f
                                      : static_cast<size_t>(E) * 2 * f * 4;
  const size_t sc2 = moe::is_mx(prec) ? static_cast<size_t>(E) * f / 32 * h
                                      : static_cast<size_t>(E) * h * 4;
  Buf s1(sc1), s2(sc2), ss1(sc1 / E), ss2(sc2 / E);
  Buf Yp(n * h * (prec == MOE_PREC_F32 ? 4 : 2)), Ys(static_cast<size_t>(T) * h * (prec == MOE_PREC_F32 ? 4 : 2)),
      Y(static_cast<size_t>(T) * h * (prec == MOE_PREC_F32 ? 4 : 2));
  moe_expert_weights w{W1.p, prec >= MOE_PREC_FP8 ? s1.p : nullptr, W2.p,
                       prec >= MOE_PREC_FP8 ? s2.p : nullptr, shared ? Ws1.p : nullptr,
                       shared && prec >= MOE_PREC_FP8 ? ss1.p : nullptr, shared ? Ws2.p : nullptr,
                       shared && prec >= MOE_PREC_FP8 ? ss2.p : nullptr};
  moe_route_opts o{MOE_SCORE_SIGMOID, 1, 2.5f, static_cast<float*>(beta.p),
                   static_cast<float*>(gb.p), hash ? static_cast<int32_t*>(tok.p) : nullptr,
                   hash ? static_cast<int32_t*>(tid.p) : nullptr, hash ? 1000 : 0};
  const bool q8 = prec >= MOE_PREC_FP8;
  expect(moe_route(&s, &o, X.p, Wg.p, static_cast<int32_t*>(ids.p), static_cast<float*>(G.p),
                   static_cast<float*>(keys.p), W, ws_bytes, nullptr), MOE_OK, "route");
  expect(moe_permute(&s, static_cast<int32_t*>(ids.p), X.p, static_cast<int32_t*>(counts.p),
                     static_cast<int32_t*>(offsets.p), static_cast<int32_t*>(dst.p),
                     static_cast<int32_t*>(src.p), Xp.p, q8 ? xps.p : nullptr, q8 ? Xq.p : nullptr,
                     q8 ? xs.p : nullptr, W, ws_bytes, nullptr), MOE_OK, "permute");
  expect(moe_permute_no_alloc(&s, static_cast<int32_t*>(ids.p), X.p, static_cast<int32_t*>(counts.p),
                              static_cast<int32_t*>(offsets.p), static_cast<int32_t*>(dst.p),
                              static_cast<int32_t*>(src.p), Xp.p, q8 ? xps.p : nullptr,
                              q8 ? Xq.p : nullptr, q8 ? xs.p : nullptr, nullptr),
         static_cast<long long>(T) * k <= MOE_NO_ALLOC_MAX_ASSIGNMENTS ? MOE_OK : MOE_ERR_SCRATCH,
         "permute_no_alloc");
  expect(moe_expert_ffn(&s, Xp.p, q8 ? xps.p : nullptr, static_cast<int32_t*>(offsets.p),
                        shared ? (q8 ? Xq.p : X.p) : nullptr, shared && q8 ? xs.p : nullptr, &w,
                        Yp.p, shared ? Ys.p : nullptr, W, ws_bytes, nullptr), MOE_OK, "expert_ffn");
  expect(moe_combine(&s, Yp.p, static_cast<int32_t*>(dst.p), static_cast<float*>(G.p),
                     shared ? Ys.p : nullptr, Y.p, nullptr), MOE_OK, "combine");
  expect(moe_forward(&s, &o, X.p, Wg.p, &w, static_cast<int32_t*>(ids.p), static_cast<float*>(G.p),
                     Y.p, W, ws_bytes, nullptr), MOE_OK, "forward");
  expect(moe_forward(&s, nullptr, X.p, nullptr, &w, static_cast<int32_t*>(ids.p),
                     static_cast<float*>(G.p), Y.p, W, ws_bytes, nullptr), MOE_OK, "forward, given routing");
  expect(moe_check_device_error(W, ws_bytes, nullptr), MOE_OK, "check_device_error");
  // out of contract
  expect(moe_route(&s, &o, X.p, Wg.p, static_cast<int32_t*>(ids.p), static_cast<float*>(G.p),
                   nullptr, W, ws_bytes - 1, nullptr), MOE_ERR_WORKSPACE, "route, small workspace");
  expect(moe_permute(&s, nullptr, X.p, static_cast<int32_t*>(counts.p),
                     static_cast<int32_t*>(offsets.p), static_cast<int32_t*>(dst.p),
                     static_cast<int32_t*>(src.p), Xp.p, xps.p, Xq.p, xs.p, W, ws_bytes, nullptr),
         MOE_ERR_INVALID_ARG, "permute, NULL ids");
  expect(moe_combine(&s, static_cast<char*>(Yp.p) + 2, static_cast<int32_t*>(dst.p),
                     static_cast<float*>(G.p), nullptr, Y.p, nullptr), MOE_ERR_INVALID_ARG,
         "combine, misaligned Yp");
  std::free(W);

  if (prec == MOE_PREC_BF16 && h % 256 == 0 && f % 128 == 0 && E % 64 == 0) {
    const size_t bws = moe_backward_workspace_size(&s);
    void* B = std::aligned_alloc(256, bws);
    g_ws_lo = static_cast<unsigned char*>(B);
    g_ws_hi = g_ws_lo + bws;
    Buf dY(static_cast<size_t>(T) * h * 2), dX(static_cast<size_t>(T) * h * 2), dW1(w1), dW2(w2),
        dWs1(w1 / E), dWs2(w2 / E), dWg(static_cast<size_t>(h) * E * 2), dgb(E * 4), dG(n * 4);
    moe_grads g{dX.p, dW1.p, dW2.p, shared ? dWs1.p : nullptr, shared ? dWs2.p : nullptr, dWg.p,
                static_cast<float*>(dgb.p), static_cast<float*>(dG.p)};
    expect(moe_backward(&s, &o, X.p, Wg.p, &w, static_cast<int32_t*>(ids.p),
                        static_cast<float*>(G.p), dY.p, &g, B, bws, nullptr), MOE_OK, "backward");
    expect(moe_forward_train(&s, &o, X.p, Wg.p, &w, static_cast<int32_t*>(ids.p),
                             static_cast<float*>(G.p), Y.p, B, bws, nullptr), MOE_OK,
           "forward_train");
    expect(moe_backward_saved(&s, &o, X.p, Wg.p, &w, static_cast<int32_t*>(ids.p),
                              static_cast<float*>(G.p), dY.p, &g, B, bws, nullptr), MOE_OK,
           "backward_saved");
    expect(moe_backward(&s, &o, X.p, Wg.p, &w, static_cast<int32_t*>(ids.p),
                        static_cast<float*>(G.p), dY.p, &g, B, bws - 256, nullptr),
           MOE_ERR_WORKSPACE, "backward, small workspace");
    std::free(B);
  }
}

}  // namespace

int main() {
  // shapes: several tiles, ragged T, every precision; a V4-like router with
  // 384 experts; hash routing; no shared expert
  const int precs[] = {MOE_PREC_F32, MOE_PREC_BF16, MOE_PREC_FP8, MOE_PREC_MXFP8, MOE_PREC_MXFP4,
                       MOE_PREC_INT8};
  for (int p : precs) {
    run_shape(257, 512, 64, 6, 256, 1, p, false);
    run_shape(3, 256, 8, 2, 128, 0, p, false);
  }
  run_shape(1000, 512, 384, 6, 256, 1, MOE_PREC_BF16, false);
  run_shape(130, 512, 64, 6, 256, 1, MOE_PREC_BF16, true);
  run_shape(8192, 256, 384, 6, 128, 1, MOE_PREC_BF16, false);
  // invalid shapes: no launch
  moe_shape bad{0, 128, 8, 2, 64, 0, MOE_PREC_BF16};
  expect(static_cast<int>(moe_workspace_size(&bad)), 0, "workspace size of T = 0");
  moe_shape huge{1 << 30, 128, 8, 2, 64, 0, MOE_PREC_BF16};
  expect(static_cast<int>(moe_workspace_size(&huge) == 0), 1, "workspace size beyond the limits");
  std::printf("launch stubs reached: %d, failures: %d, overlapping workspace regions: %d\n",
              g_launches, g_fail + g_stub_fail, g_overlaps);
  return g_fail + g_stub_fail == 0 && g_overlaps == 0 && g_launches > 0 ? 0 : 1;
}
