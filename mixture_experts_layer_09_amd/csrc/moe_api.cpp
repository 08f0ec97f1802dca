// moe_api.cpp -- the C ABI of libmoe (declared in include/moe.h): host-side
// validation, workspace carving and kernel launches.  No entry point reads
// device memory or synchronises, except moe_check_device_error.
#include <hip/hip_runtime.h>

#include <initializer_list>

#include "moe_internal.h"

using namespace moe;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The kernels move activations, weights and scales with 16-byte vector loads
// and global->LDS DMAs, so those arrays must be 16-byte aligned (NULL, an
// absent optional array, passes).
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 16)) return false;
  return true;
}

int check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->tokens < 1 || s->hidden < 1 || s->experts < 1 || s->topk < 1 || s->inter < 1)
    return MOE_ERR_INVALID_ARG;
  if (s->topk > s->experts || s->topk > kMaxTopk) return MOE_ERR_INVALID_ARG;
  if (s->has_shared != 0 && s->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (s->precision < MOE_PREC_F32 || s->precision > MOE_PREC_INT8) return MOE_ERR_INVALID_ARG;
  if (s->experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (s->hidden % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (s->inter % (s->precision >= MOE_PREC_FP8 ? 128 : 64) != 0) return MOE_ERR_UNSUPPORTED;
  // e4m3 grouped GEMMs use 256-column n-tiles for Linear2
  if (s->precision >= MOE_PREC_FP8 && s->hidden % 256 != 0) return MOE_ERR_UNSUPPORTED;
  // row and element counts must fit the kernels' 32-bit row indices
  const long long rows = static_cast<long long>(s->tokens) * (s->topk + 1);
  if (rows > (1LL << 30)) return MOE_ERR_UNSUPPORTED;
  if (rows * (s->hidden > s->inter ? s->hidden : s->inter) > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_ws(const moe_shape* s, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned(ws, kAlign)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < make_layout(*s).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_weights(const moe_shape* s, const moe_expert_weights* w) {
  if (!w || !w->W1 || !w->W2) return MOE_ERR_INVALID_ARG;
  const bool scaled = s->precision >= MOE_PREC_FP8;
  if (scaled && (!w->w1_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
  if (!aligned16({w->W1, w->w1_scale, w->W2, w->w2_scale, w->Ws1, w->ws1_scale, w->Ws2,
                  w->ws2_scale}))
    return MOE_ERR_INVALID_ARG;
  if (s->has_shared) {
    if (!w->Ws1 || !w->Ws2) return MOE_ERR_INVALID_ARG;
    if (scaled && (!w->ws1_scale || !w->ws2_scale))
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

int check_route_opts(const moe_route_opts* o) {
  if (!o) return MOE_ERR_INVALID_ARG;
  if (o->score_fn < MOE_SCORE_SIGMOID || o->score_fn > MOE_SCORE_SQRT_SOFTPLUS)
    return MOE_ERR_INVALID_ARG;
  if (o->renorm != 0 && o->renorm != 1) return MOE_ERR_INVALID_ARG;
  if ((o->token_ids == nullptr) != (o->tid2eid == nullptr)) return MOE_ERR_INVALID_ARG;
  if (o->tid2eid && o->vocab < 1) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

RouteArgs route_args(const moe_shape* s, const moe_route_opts* o, const void* X, const void* Wg,
                     int32_t* ids, float* G, float* keys, void* ws) {
  RouteArgs a{};
  a.T = s->tokens;
  a.h = s->hidden;
  a.E = s->experts;
  a.k = s->topk;
  a.precision = s->precision;
  a.score_fn = o->score_fn;
  a.renorm = o->renorm;
  a.alpha = o->alpha;
  a.X = X;
  a.Wg = Wg;
  a.beta = o->expert_bias;
  a.gate_bias = o->gate_bias;
  a.token_ids = o->token_ids;
  a.tid2eid = o->tid2eid;
  a.vocab = o->vocab;
  a.ids = ids;
  a.G = G;
  a.keys = keys;
  const Layout L = make_layout(*s);
  a.flag = at<int32_t>(ws, L.flag);
  a.part = at<float>(ws, L.part);
  return a;
}

PermuteArgs permute_args(const moe_shape* s, const int32_t* ids, const void* X, int32_t* counts,
                         int32_t* offsets, int32_t* dst_row, int32_t* src_tok, void* Xp,
                         void* xp_scale, void* Xq, void* x_scale, void* ws /* may be NULL */) {
  Layout L = make_layout(*s);
  PermuteArgs a{};
  a.T = s->tokens;
  a.h = s->hidden;
  a.E = s->experts;
  a.k = s->topk;
  a.precision = s->precision;
  a.nblk = L.nblk;
  a.ids = ids;
  a.X = X;
  a.counts = counts;
  a.offsets = offsets;
  a.dst_row = dst_row;
  a.src_tok = src_tok;
  a.Xp = Xp;
  a.xp_scale = xp_scale;
  a.Xq = Xq;
  a.x_scale = x_scale;
  if (ws) {
    a.blk_cnt = at<int32_t>(ws, L.blk_cnt);
    a.local_rank = at<int32_t>(ws, L.local_rank);
    a.flag = at<int32_t>(ws, L.flag);
  }
  return a;
}

FfnArgs ffn_args(const moe_shape* s, const void* Xp, const void* xp_scale, const int32_t* offsets,
                 const void* Xs, const void* xs_scale, const moe_expert_weights* w, void* Yp,
                 void* Ys, void* ws) {
  Layout L = make_layout(*s);
  FfnArgs a{};
  a.T = s->tokens;
  a.h = s->hidden;
  a.E = s->experts;
  a.k = s->topk;
  a.f = s->inter;
  a.has_shared = s->has_shared;
  a.precision = s->precision;
  a.Xp = Xp;
  a.xp_scale = xp_scale;
  a.offsets = offsets;
  a.Xs = Xs;
  a.xs_scale = xs_scale;
  a.w = *w;
  a.Yp = Yp;
  a.Ys = Ys;
  a.A = at<void>(ws, L.A);
  a.Aq = at<void>(ws, L.Aq);
  a.a_scale = at<void>(ws, L.a_scale);
  a.tile_off = at<int32_t>(ws, L.tile_off);
  return a;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return make_layout(*shape).total;
}

int moe_route(const moe_shape* shape, const moe_route_opts* opts, const void* X, const void* Wg,
              int32_t* expert_ids, float* gate_weights, float* keys_out, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_route_opts(opts)) != MOE_OK) return st;
  if (!X || !Wg || !expert_ids || !gate_weights) return MOE_ERR_INVALID_ARG;
  if (!aligned16({X, Wg})) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  RouteArgs a = route_args(shape, opts, X, Wg, expert_ids, gate_weights, keys_out, workspace);
  return hip_status(launch_route(a, stream));  // clears the error flag first
}

int moe_permute(const moe_shape* shape, const int32_t* expert_ids, const void* X,
                int32_t* counts, int32_t* offsets, int32_t* dst_row, int32_t* src_tok, void* Xp,
                void* xp_scale, void* Xq, void* x_scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!expert_ids || !X || !counts || !offsets || !dst_row || !src_tok || !Xp)
    return MOE_ERR_INVALID_ARG;
  if (shape->precision >= MOE_PREC_FP8 && (!xp_scale || !Xq || !x_scale))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16({X, Xp, xp_scale, Xq, x_scale})) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  PermuteArgs a = permute_args(shape, expert_ids, X, counts, offsets, dst_row, src_tok, Xp,
                               xp_scale, Xq, x_scale, workspace);
  a.clear_flag = 1;  // the call's only step that can raise the flag
  return hip_status(launch_permute(a, stream));
}

int moe_permute_no_alloc(const moe_shape* shape, const int32_t* expert_ids, const void* X,
                         int32_t* counts, int32_t* offsets, int32_t* dst_row, int32_t* src_tok,
                         void* Xp, void* xp_scale, void* Xq, void* x_scale, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!expert_ids || !X || !counts || !offsets || !dst_row || !src_tok || !Xp)
    return MOE_ERR_INVALID_ARG;
  if (shape->precision >= MOE_PREC_FP8 && (!xp_scale || !Xq || !x_scale))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16({X, Xp, xp_scale, Xq, x_scale})) return MOE_ERR_INVALID_ARG;
  if (static_cast<long long>(shape->tokens) * shape->topk > MOE_NO_ALLOC_MAX_ASSIGNMENTS)
    return MOE_ERR_SCRATCH;
  PermuteArgs a = permute_args(shape, expert_ids, X, counts, offsets, dst_row, src_tok, Xp,
                               xp_scale, Xq, x_scale, nullptr);
  return hip_status(launch_permute_no_alloc(a, stream));
}

int moe_expert_ffn(const moe_shape* shape, const void* Xp, const void* xp_scale,
                   const int32_t* offsets, const void* Xs, const void* xs_scale,
                   const moe_expert_weights* weights, void* Yp, void* Ys, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_weights(shape, weights)) != MOE_OK) return st;
  if (!Xp || !offsets || !Yp) return MOE_ERR_INVALID_ARG;
  if (shape->precision >= MOE_PREC_FP8 && !xp_scale) return MOE_ERR_INVALID_ARG;
  if (shape->has_shared) {
    if (!Xs || !Ys) return MOE_ERR_INVALID_ARG;
    if (shape->precision >= MOE_PREC_FP8 && !xs_scale) return MOE_ERR_INVALID_ARG;
  }
  if (!aligned16({Xp, xp_scale, Xs, xs_scale, Yp, Ys})) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  FfnArgs a = ffn_args(shape, Xp, xp_scale, offsets, Xs, xs_scale, weights, Yp, Ys, workspace);
  return hip_status(launch_expert_ffn(a, stream));
}

int moe_combine(const moe_shape* shape, const void* Yp, const int32_t* dst_row,
                const float* gate_weights, const void* Ys, void* Y, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!Yp || !dst_row || !gate_weights || !Y) return MOE_ERR_INVALID_ARG;
  if (!aligned16({Yp, Ys, Y})) return MOE_ERR_INVALID_ARG;
  CombineArgs a{};
  a.T = shape->tokens;
  a.h = shape->hidden;
  a.k = shape->topk;
  a.precision = shape->precision;
  a.Yp = Yp;
  a.dst_row = dst_row;
  a.G = gate_weights;
  a.Ys = Ys;
  a.Y = Y;
  return hip_status(launch_combine(a, stream));
}

int moe_forward(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                const void* Wg, const moe_expert_weights* weights, int32_t* expert_ids,
                float* gate_weights, void* Y, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_weights(shape, weights)) != MOE_OK) return st;
  if (!X || !expert_ids || !gate_weights || !Y) return MOE_ERR_INVALID_ARG;
  if (!aligned16({X, Wg, Y})) return MOE_ERR_INVALID_ARG;
  if (opts) {
    if ((st = check_route_opts(opts)) != MOE_OK) return st;
    if (!Wg) return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(shape, workspace, workspace_bytes)) != MOE_OK) return st;
  const Layout L = make_layout(*shape);
  void* ws = workspace;
  const bool fp8 = shape->precision >= MOE_PREC_FP8;  // quantised activations
  // the router clears the error flag when it starts; without it the
  // dispatch is the first step that can raise it and writes it whole
  hipError_t e = hipSuccess;
  if (opts) {
    RouteArgs r = route_args(shape, opts, X, Wg, expert_ids, gate_weights, nullptr, ws);
    e = launch_route(r, stream);
  }
  // Where Linear1 can gather its token rows from X by the row -> token map,
  // the dispatch writes the row maps only and no permuted copy of X.
  const bool gather = ffn_gathers(shape->precision, shape->tokens, shape->hidden, shape->experts,
                                  shape->topk, shape->inter);
  if (e == hipSuccess) {
    PermuteArgs p = permute_args(shape, expert_ids, X, at<int32_t>(ws, L.counts),
                                 at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.dst_row),
                                 at<int32_t>(ws, L.src_tok), at<void>(ws, L.Xp),
                                 fp8 ? at<void>(ws, L.xp_scale) : nullptr,
                                 fp8 ? at<void>(ws, L.Xq) : nullptr,
                                 fp8 ? at<void>(ws, L.x_scale) : nullptr, ws);
    p.maps_only = gather ? 1 : 0;
    p.clear_flag = opts ? 0 : 1;
    e = launch_permute(p, stream);
  }
  if (e == hipSuccess) {
    FfnArgs f = ffn_args(shape, at<void>(ws, L.Xp), fp8 ? at<void>(ws, L.xp_scale) : nullptr,
                         at<int32_t>(ws, L.offsets), fp8 ? at<void>(ws, L.Xq) : X,
                         fp8 ? at<void>(ws, L.x_scale) : nullptr, weights, at<void>(ws, L.Yp),
                         shape->has_shared ? at<void>(ws, L.Ys) : nullptr, ws);
    if (gather) f.src_tok = at<int32_t>(ws, L.src_tok);
    e = launch_expert_ffn(f, stream);
  }
  if (e == hipSuccess) {
    CombineArgs c{};
    c.T = shape->tokens;
    c.h = shape->hidden;
    c.k = shape->topk;
    c.precision = shape->precision;
    c.Yp = at<void>(ws, L.Yp);
    c.dst_row = at<int32_t>(ws, L.dst_row);
    c.G = gate_weights;
    c.Ys = shape->has_shared ? at<void>(ws, L.Ys) : nullptr;
    c.Y = Y;
    e = launch_combine(c, stream);
  }
  return hip_status(e);
}

size_t moe_backward_workspace_size(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return make_bwd_layout(*shape).total;
}

namespace {

// Shape, argument and workspace checks of moe_backward and its saved form.
int check_backward(const moe_shape* shape, const moe_route_opts* opts, const void* X, const void* Wg,
                   const moe_expert_weights* weights, const int32_t* expert_ids,
                   const float* gate_weights, const void* dY, const moe_grads* grads,
                   void* workspace, size_t workspace_bytes) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->precision != MOE_PREC_BF16) return MOE_ERR_UNSUPPORTED;
  // the backward GEMMs' tiles: 256-column Linear1 outputs, 128-row weight tiles
  if (shape->hidden % 256 != 0 || shape->inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((st = check_weights(shape, weights)) != MOE_OK) return st;
  if (!X || !expert_ids || !gate_weights || !dY || !grads) return MOE_ERR_INVALID_ARG;
  if (!grads->dX || !grads->dW1 || !grads->dW2) return MOE_ERR_INVALID_ARG;
  if (shape->has_shared && (!grads->dWs1 || !grads->dWs2)) return MOE_ERR_INVALID_ARG;
  if (opts) {
    if ((st = check_route_opts(opts)) != MOE_OK) return st;
    if (!Wg) return MOE_ERR_INVALID_ARG;
    // the router's dWg tiles are 64 experts wide, its dgrad K-stages 32
    if (shape->experts % 64 != 0) return MOE_ERR_UNSUPPORTED;
  }
  if (!aligned16({X, Wg, dY, grads->dX, grads->dW1, grads->dW2, grads->dWs1, grads->dWs2,
                  grads->dWg}))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kAlign)) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < make_bwd_layout(*shape).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// The dispatch, the router keys (with opts), the gate weight of each row,
// H1 = Xp W1 (routed and shared rows) and A = SwiGLU(H1) weighted by the
// row's gate weight (what the backward reads) into a backward workspace.
// Routing: with ids_out the router runs and writes it and G (the training
// forward), else it runs into scratch for its keys only and G is the
// caller's (the recompute).  The training forward (train) also keeps A
// unweighted and runs Linear2: Yp = A W2 for the routed rows and, with Ys !=
// NULL, the shared expert's output.
hipError_t recompute(const moe_shape* shape, const moe_route_opts* opts, const void* X, const void* Wg,
                     const moe_expert_weights* weights, const int32_t* expert_ids,
                     const float* G, int32_t* ids_out, float* g_out, bool train, void* Ys,
                     void* ws, hipStream_t stream) {
  const Layout L = make_layout(*shape);
  const BwdLayout B = make_bwd_layout(*shape);
  const int T = shape->tokens, k = shape->topk, E = shape->experts;
  const int rows = T * k;
  const size_t f = shape->inter;
  hipError_t e = hipSuccess;
  // router keys (a + beta) for the router's backward; the training forward's
  // routing itself
  if (opts) {
    RouteArgs r = route_args(shape, opts, X, Wg, ids_out ? ids_out : at<int32_t>(ws, B.ids_s),
                             g_out ? g_out : at<float>(ws, B.G_s), at<float>(ws, B.keys), ws);
    e = launch_route(r, stream);
  }
  if (e == hipSuccess) {
    PermuteArgs p = permute_args(shape, ids_out ? ids_out : expert_ids, X, at<int32_t>(ws, L.counts),
                                 at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.dst_row),
                                 at<int32_t>(ws, L.src_tok), at<void>(ws, L.Xp), nullptr, nullptr,
                                 nullptr, ws);
    e = launch_permute(p, stream);
  }
  if (e == hipSuccess) {
    LinearArgs l1{};
    l1.A = at<void>(ws, L.Xp);
    l1.A_sh = X;
    l1.W = weights->W1;
    l1.W_sh = weights->Ws1;
    l1.out = at<void>(ws, B.H1);
    l1.out_sh = at<char>(ws, B.H1) + static_cast<size_t>(rows) * 2 * f * 2;
    l1.offsets = at<int32_t>(ws, L.offsets);
    l1.tile_off = at<int32_t>(ws, L.tile_off);
    l1.E = E;
    l1.K = shape->hidden;
    l1.N = 2 * shape->inter;
    l1.T = T;
    l1.rows = rows;
    l1.has_shared = shape->has_shared;
    e = launch_grouped_linear_bf16(l1, stream);
  }
  if (e == hipSuccess)
    e = launch_row_gate(at<int32_t>(ws, L.dst_row), g_out ? g_out : G, rows,
                        at<float>(ws, B.grow), stream);
  if (e == hipSuccess)
    e = launch_swiglu_bf16(at<void>(ws, B.H1), shape->inter, rows,
                           static_cast<long>(rows) + (shape->has_shared ? T : 0),
                           at<float>(ws, B.grow), at<void>(ws, B.Aact),
                           train ? at<void>(ws, B.Afwd) : nullptr, stream);
  if (e == hipSuccess && train) {
    LinearArgs l2{};
    l2.A = at<void>(ws, B.Afwd);
    l2.A_sh = at<char>(ws, B.Afwd) + static_cast<size_t>(rows) * f * 2;
    l2.W = weights->W2;
    l2.W_sh = weights->Ws2;
    l2.out = at<void>(ws, L.Yp);
    l2.out_sh = Ys;
    l2.offsets = at<int32_t>(ws, L.offsets);
    l2.tile_off = at<int32_t>(ws, L.tile_off);
    l2.E = E;
    l2.K = shape->inter;
    l2.N = shape->hidden;
    l2.T = T;
    l2.rows = rows;
    l2.has_shared = (Ys != nullptr && shape->has_shared) ? 1 : 0;
    e = launch_grouped_linear_bf16(l2, stream);
  }
  return e;
}

// Everything after the recompute, on the activations in the workspace.
hipError_t backward_from_saved(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                               const void* Wg, const moe_expert_weights* weights,
                               const int32_t* expert_ids, const float* gate_weights, const void* dY,
                               const moe_grads* grads, void* ws, hipStream_t stream) {
  const Layout L = make_layout(*shape);
  const BwdLayout B = make_bwd_layout(*shape);
  BackwardArgs b{};
  b.T = shape->tokens;
  b.h = shape->hidden;
  b.E = shape->experts;
  b.k = shape->topk;
  b.f = shape->inter;
  b.has_shared = shape->has_shared;
  b.route = opts != nullptr;
  if (opts) {
    b.score_fn = opts->score_fn;
    b.renorm = opts->renorm;
    b.alpha = opts->alpha;
    b.hash = (opts->token_ids && opts->tid2eid) ? 1 : 0;
    b.beta = opts->expert_bias;
  }
  b.X = X;
  b.Wg = Wg;
  b.W1 = weights->W1;
  b.W2 = weights->W2;
  b.Ws1 = weights->Ws1;
  b.Ws2 = weights->Ws2;
  b.ids = expert_ids;
  b.G = gate_weights;
  b.dY = dY;
  b.offsets = at<int32_t>(ws, L.offsets);
  b.dst_row = at<int32_t>(ws, L.dst_row);
  b.Xp = at<void>(ws, L.Xp);
  b.grow = at<float>(ws, B.grow);
  b.H1 = at<void>(ws, B.H1);
  b.Aact = at<void>(ws, B.Aact);
  b.dGp = at<float>(ws, B.dGp);
  b.dYp = at<void>(ws, B.dYp);
  b.dH1 = at<void>(ws, B.dH1);
  b.dXp = at<void>(ws, B.dXp);
  b.dXr = at<void>(ws, B.dXr);
  b.keys = at<float>(ws, B.keys);
  b.dG = grads->dG ? grads->dG : at<float>(ws, B.dG);
  b.dl32 = at<float>(ws, B.dl32);
  b.dl16 = at<void>(ws, B.dl16);
  b.tile_off = at<int32_t>(ws, L.tile_off);
  b.tile_b = at<int32_t>(ws, B.tile_b);
  b.colsum = at<float>(ws, B.colsum);
  b.dX = grads->dX;
  b.dWg = opts ? grads->dWg : nullptr;
  b.dgate_bias = opts ? grads->dgate_bias : nullptr;
  b.dW1 = grads->dW1;
  b.dW2 = grads->dW2;
  b.dWs1 = grads->dWs1;
  b.dWs2 = grads->dWs2;
  return launch_backward(b, stream);
}

}  // namespace

int moe_backward(const moe_shape* shape, const moe_route_opts* opts, const void* X, const void* Wg,
                 const moe_expert_weights* weights, const int32_t* expert_ids,
                 const float* gate_weights, const void* dY, const moe_grads* grads,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_backward(shape, opts, X, Wg, weights, expert_ids, gate_weights, dY, grads,
                                workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  const Layout L = make_layout(*shape);
  hipError_t e = launch_clear_flag(at<int32_t>(workspace, L.flag), stream);
  if (e == hipSuccess)
    e = recompute(shape, opts, X, Wg, weights, expert_ids, gate_weights, nullptr, nullptr, false,
                  nullptr, workspace, stream);
  if (e == hipSuccess)
    e = backward_from_saved(shape, opts, X, Wg, weights, expert_ids, gate_weights, dY, grads,
                            workspace, stream);
  return hip_status(e);
}

int moe_forward_train(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                      const void* Wg, const moe_expert_weights* weights, int32_t* expert_ids,
                      float* gate_weights, void* Y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->precision != MOE_PREC_BF16) return MOE_ERR_UNSUPPORTED;
  if (shape->hidden % 256 != 0 || shape->inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((st = check_weights(shape, weights)) != MOE_OK) return st;
  if (!X || !expert_ids || !gate_weights || !Y) return MOE_ERR_INVALID_ARG;
  if (!aligned16({X, Wg, Y})) return MOE_ERR_INVALID_ARG;
  if (opts) {
    if ((st = check_route_opts(opts)) != MOE_OK) return st;
    if (!Wg) return MOE_ERR_INVALID_ARG;
    if (shape->experts % 64 != 0) return MOE_ERR_UNSUPPORTED;
  }
  if (!workspace || !aligned(workspace, kAlign)) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < make_bwd_layout(*shape).total) return MOE_ERR_WORKSPACE;
  const Layout L = make_layout(*shape);
  void* ws = workspace;
  hipError_t e = launch_clear_flag(at<int32_t>(ws, L.flag), stream);
  if (e == hipSuccess)
    e = recompute(shape, opts, X, Wg, weights, expert_ids, gate_weights,
                  opts ? expert_ids : nullptr, opts ? gate_weights : nullptr, true,
                  shape->has_shared ? at<void>(ws, L.Ys) : nullptr, ws, stream);
  if (e == hipSuccess) {
    CombineArgs c{};
    c.T = shape->tokens;
    c.h = shape->hidden;
    c.k = shape->topk;
    c.precision = shape->precision;
    c.Yp = at<void>(ws, L.Yp);
    c.dst_row = at<int32_t>(ws, L.dst_row);
    c.G = gate_weights;
    c.Ys = shape->has_shared ? at<void>(ws, L.Ys) : nullptr;
    c.Y = Y;
    e = launch_combine(c, stream);
  }
  return hip_status(e);
}

int moe_backward_saved(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                       const void* Wg, const moe_expert_weights* weights,
                       const int32_t* expert_ids, const float* gate_weights, const void* dY,
                       const moe_grads* grads, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  const int st = check_backward(shape, opts, X, Wg, weights, expert_ids, gate_weights, dY, grads,
                                workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  return hip_status(backward_from_saved(shape, opts, X, Wg, weights, expert_ids, gate_weights, dY,
                                        grads, workspace, stream));
}

int moe_check_device_error(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < kAlign)
    return MOE_ERR_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
  int32_t flag = 0;
  if (hipMemcpy(&flag, workspace, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  if (flag != 0) {
    const int32_t zero = 0;
    if (hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_ERR_DEVICE_DATA;
  }
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime or launch error";
    case MOE_ERR_DEVICE_DATA: return "device data out of contract (expert or token id)";
    case MOE_ERR_SCRATCH: return "problem larger than the static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
