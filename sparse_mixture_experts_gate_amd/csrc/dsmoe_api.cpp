// C ABI of the DeepSeekMoE layer: argument validation (host only, before any
// launch), workspace carving and launch sequencing on the caller's stream.
// The library never allocates, frees or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include <hip/hip_runtime.h>

#include "dsmoe.h"
#include "internal.h"

using namespace dsmoe;

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_prof[6] = {};
thread_local bool g_prof_on = false;

hipError_t prof_record(int i, hipStream_t s) {
  return g_prof_on ? hipEventRecord(g_prof[i], s) : hipSuccess;
}

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                     \
  do {                                          \
    hipError_t _e = (expr);                     \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

moe_status validate_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)d->T);
  if (d->d <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "d = %d <= 0", d->d);
  if (d->n_experts < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "n_experts = %d < 1", d->n_experts);
  if (d->n_experts > 512)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts = %d > 512", d->n_experts);
  if (d->top_k < 1 || d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "top_k = %d outside 1..n_experts", d->top_k);
  if (d->top_k > 64) return fail(MOE_ERR_UNSUPPORTED, "top_k = %d > 64", d->top_k);
  if (d->n_groups < 1 || d->n_experts % d->n_groups != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "n_groups = %d must divide n_experts = %d",
                d->n_groups, d->n_experts);
  if (d->n_groups > 64) return fail(MOE_ERR_UNSUPPORTED, "n_groups = %d > 64", d->n_groups);
  if (d->topk_groups < 1 || d->topk_groups > d->n_groups)
    return fail(MOE_ERR_INVALID_ARGUMENT, "topk_groups = %d outside 1..n_groups",
                d->topk_groups);
  const int gs = d->n_experts / d->n_groups;
  if (d->topk_groups * gs < d->top_k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "topk_groups * group size = %d < top_k = %d",
                d->topk_groups * gs, d->top_k);
  if (d->n_groups > 1 && (d->group_topn < 1 || d->group_topn > gs || d->group_topn > 8))
    return fail(MOE_ERR_INVALID_ARGUMENT, "group_topn = %d outside 1..min(group size, 8)",
                d->group_topn);
  if (d->inter < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "inter = %d < 1", d->inter);
  if (d->shared_inter < 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared_inter = %d < 0", d->shared_inter);
  if (!(d->near_tie_eps >= 0.0f) || !std::isfinite(d->near_tie_eps))
    return fail(MOE_ERR_INVALID_ARGUMENT, "near_tie_eps must be finite and >= 0");
  const bool f32 = d->act_dtype == MOE_DT_F32 && d->w_dtype == MOE_DT_F32;
  const bool bf16 = d->act_dtype == MOE_DT_BF16 && d->w_dtype == MOE_DT_BF16;
  const bool fp8 = d->act_dtype == MOE_DT_BF16 && d->w_dtype == MOE_DT_FP8_E4M3;
  if (!(f32 || bf16 || fp8))
    return fail(MOE_ERR_UNSUPPORTED, "dtype pair act=%d w=%d not supported", d->act_dtype,
                d->w_dtype);
  if (d->out_dtype != MOE_DT_F32 && d->out_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "out_dtype = %d: y is fp32 or bf16", d->out_dtype);
  const int mult = fp8 ? 128 : 64;
  if (d->d % mult || d->inter % mult || d->shared_inter % mult)
    return fail(MOE_ERR_UNSUPPORTED, "d, inter, shared_inter must be multiples of %d", mult);
  if (d->T * static_cast<int64_t>(d->top_k) + d->T >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*(K+1) must be < 2^31");
  // the permutation reads topk_idx through a 32-bit byte range
  if (d->T * static_cast<int64_t>(d->top_k) * 4 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*K*4 must be < 2^31 bytes");
  // the GEMMs address the gathered rows of x and each expert's weights with
  // 32-bit byte offsets (H is addressed per tile, from a 64-bit base)
  const int64_t lim = (int64_t(1) << 31) - 1;
  const int64_t s_act = d->act_dtype == MOE_DT_F32 ? 4 : 2;
  const int64_t s_w = d->w_dtype == MOE_DT_F32 ? 4 : d->w_dtype == MOE_DT_BF16 ? 2 : 1;
  const int64_t ldh = std::max(d->inter, d->shared_inter);
  if (d->T * d->d * s_act > lim)
    return fail(MOE_ERR_UNSUPPORTED, "T*d*sizeof(act) must be < 2^31 bytes");
  // H's scales (FP8) are addressed as one range
  if (s_w == 1 && (d->T * d->top_k + d->T) * (ldh / 128) * 4 > lim)
    return fail(MOE_ERR_UNSUPPORTED, "T*(K+1)*max(I,Is)/128*4 must be < 2^31 bytes");
  if (int64_t(2) * ldh * d->d * s_w > lim)
    return fail(MOE_ERR_UNSUPPORTED, "one expert's weights must be < 2^31 bytes");
  if (int64_t(d->n_experts) * 3 * d->d * 2 > lim)
    return fail(MOE_ERR_UNSUPPORTED, "E*3*d*2 must be < 2^31 bytes");
  return MOE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

int io_bytes(const moe_layer_desc* d) { return d->act_dtype == MOE_DT_F32 ? 4 : 2; }
int h_bytes(const moe_layer_desc* d) {
  return d->w_dtype == MOE_DT_F32 ? 4 : d->w_dtype == MOE_DT_BF16 ? 2 : 1;
}

struct GateLayout {
  int splits;
  size_t partial, wsplit, ntie, bytes;
};

GateLayout gate_layout(const moe_layer_desc* d) {
  GateLayout L{};
  const int E = d->n_experts;
  L.splits = router_splits(d->T, d->d, E, d->act_dtype);
  Carver c;
  L.partial = c.take(sizeof(float) * size_t(L.splits) * size_t(d->T) * E);
  L.wsplit = c.take(d->act_dtype == MOE_DT_BF16 ? size_t(E) * 3 * d->d * 2 : 0);
  L.ntie = c.take(sizeof(int32_t));
  L.bytes = c.off;
  return L;
}

struct FfnLayout {
  GemmTiling tiling;
  int ldh;
  size_t tiles1, tiles2, xq, xs, xsT, H, Hs, bytes;
};

FfnLayout ffn_layout(const moe_layer_desc* d) {
  FfnLayout L{};
  const int64_t T = d->T, TK = d->T * d->top_k;
  const int E = d->n_experts;
  L.tiling = choose_tiling(T, d->top_k, E, d->w_dtype);
  L.ldh = std::max(d->inter, d->shared_inter);
  Carver c;
  L.tiles1 = c.take(sizeof(int32_t) * (E + 2));
  L.tiles2 = c.take(sizeof(int32_t) * (E + 2));
  const bool fp8 = d->w_dtype == MOE_DT_FP8_E4M3;
  L.xq = c.take(fp8 ? size_t(T) * d->d : 0);
  L.xs = c.take(fp8 ? sizeof(float) * size_t(T) * (d->d / 128) : 0);
  const int64_t hrows = TK + (d->shared_inter > 0 ? T : 0);
  L.xsT = c.take(fp8 ? sizeof(float) * size_t(hrows) * (d->d / 128) : 0);
  L.Hs = c.take(fp8 ? sizeof(float) * size_t(hrows) * (L.ldh / 128) : 0);
  L.H = c.take(size_t(hrows) * L.ldh * h_bytes(d));
  L.bytes = c.off;
  return L;
}

struct FwdLayout {
  GateLayout gate;
  FfnLayout ffn;
  size_t gate_base, ffn_base, offsets, perm, inv, yperm, yshared, bytes;
};

FwdLayout fwd_layout(const moe_layer_desc* d) {
  FwdLayout L{};
  L.gate = gate_layout(d);
  L.ffn = ffn_layout(d);
  const int64_t T = d->T, TK = d->T * d->top_k;
  Carver c;
  L.gate_base = c.take(L.gate.bytes);
  L.ffn_base = c.take(L.ffn.bytes);
  L.offsets = c.take(sizeof(int32_t) * (d->n_experts + 1));
  L.perm = c.take(sizeof(int32_t) * size_t(TK));
  L.inv = c.take(sizeof(int32_t) * size_t(TK));
  L.yperm = c.take(size_t(TK) * d->d * io_bytes(d));
  L.yshared = c.take(d->shared_inter > 0 ? size_t(T) * d->d * io_bytes(d) : 0);
  L.bytes = c.off;
  return L;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> req) {
  for (auto& p : req) {
    if (!p.first) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", p.second);
    if (misaligned(p.first)) return fail(MOE_ERR_MISALIGNED, "%s is not 16-byte aligned", p.second);
  }
  return MOE_OK;
}

moe_status check_opt(std::initializer_list<std::pair<const void*, const char*>> opt) {
  for (auto& p : opt)
    if (p.first && misaligned(p.first))
      return fail(MOE_ERR_MISALIGNED, "%s is not 16-byte aligned", p.second);
  return MOE_OK;
}

moe_status check_weights(const moe_layer_desc* d, const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  moe_status st = check_ptrs({{w->w13, "w13"}, {w->w2, "w2"}});
  if (st) return st;
  if (d->shared_inter > 0) {
    st = check_ptrs({{w->ws13, "ws13"}, {w->ws2, "ws2"}});
    if (st) return st;
  }
  if (d->w_dtype == MOE_DT_FP8_E4M3) {
    st = check_ptrs({{w->w13_scale, "w13_scale"}, {w->w2_scale, "w2_scale"}});
    if (st) return st;
    if (d->shared_inter > 0) {
      st = check_ptrs({{w->ws13_scale, "ws13_scale"}, {w->ws2_scale, "ws2_scale"}});
      if (st) return st;
    }
  }
  return MOE_OK;
}

// T == 0: the only outputs are the per-expert counts (all zero) and the
// near-tie count (zero); T-sized pointers may be NULL.
moe_status zero_counts(const moe_layer_desc* d, int32_t* counts, int32_t* near_tie,
                       hipStream_t s) {
  moe_status st = check_ptrs({{counts, "counts"}});
  if (st) return st;
  st = check_opt({{near_tie, "near_tie"}});
  if (st) return st;
  HIP_TRY(launch_fill_i32(counts, d->n_experts, 0, s), "zero counts");
  if (near_tie) HIP_TRY(launch_fill_i32(near_tie, 1, 0, s), "zero near_tie");
  return MOE_OK;
}

RouteParams route_params(const moe_layer_desc* d) {
  RouteParams p;
  p.T = d->T;
  p.E = d->n_experts;
  p.K = d->top_k;
  p.G = d->n_groups;
  p.M = d->n_groups > 1 ? d->topk_groups : 1;
  p.topn = d->n_groups > 1 ? d->group_topn : 1;
  p.eps = d->near_tie_eps;
  return p;
}

PlanParams plan_params(const moe_layer_desc* d, const GemmTiling& t) {
  PlanParams p;
  p.T = d->T;
  p.E = d->n_experts;
  p.K = d->top_k;
  p.d = d->d;
  p.I = d->inter;
  p.Is = d->shared_inter;
  p.bm1 = t.bm1;
  p.bnh1 = t.bnh1;
  p.bm2 = t.bm2;
  p.bn2 = t.bn2;
  return p;
}

// Router + routing on a validated call; ws points at a GateLayout region.
moe_status run_gate(const moe_layer_desc* d, const void* x, const float* w_router,
                    const float* bias, float* logits, int32_t* idx, float* gate, int32_t* counts,
                    int32_t* near_tie, void* ws, const GateLayout& L, hipStream_t s) {
  int32_t* ntie = near_tie ? near_tie : at<int32_t>(ws, L.ntie);
  float* partial = at<float>(ws, L.partial);
  if (d->T > 0 && d->T <= kSmallRouterT && d->act_dtype == MOE_DT_BF16) {
    // one launch: logits from the fp32 weights, counts and near_tie cleared
    HIP_TRY(launch_router_small(x, w_router, d->T, d->d, d->n_experts, partial, counts, ntie, s),
            "router (small batch)");
    HIP_TRY(launch_route(partial, 1, logits, bias, route_params(d), idx, gate, counts, ntie, s),
            "route");
    return MOE_OK;
  }
  HIP_TRY(launch_fill_i32(counts, d->n_experts, 0, s), "zero counts");
  HIP_TRY(launch_fill_i32(ntie, 1, 0, s), "zero near_tie");
  if (d->T == 0) return MOE_OK;
  if (d->act_dtype == MOE_DT_F32)
    HIP_TRY(launch_router_f32(static_cast<const float*>(x), w_router, d->T, d->d, d->n_experts,
                              partial, s),
            "router (fp32)");
  else
    HIP_TRY(launch_router_logits_bf16(x, w_router, d->T, d->d, d->n_experts, L.splits,
                                      at<uint16_t>(ws, L.wsplit), partial, s),
            "router (bf16)");
  int splits = L.splits;
  if (splits >= 8) {  // small T: many partials, summed by a wide kernel first
    HIP_TRY(launch_sum_partials(partial, splits, d->T * d->n_experts, s), "router partial sums");
    splits = 1;
  }
  HIP_TRY(launch_route(partial, splits, logits, bias, route_params(d), idx, gate, counts, ntie, s),
          "route");
  return MOE_OK;
}

// Expert FFNs on a validated call; ws points at an FfnLayout region. With
// planned == true the tile tables were already written (by the forward's
// single planning launch).
moe_status run_ffn(const moe_layer_desc* d, const moe_weights* w, const void* x,
                   const int32_t* perm, const void* x_perm, const float* x_perm_scale,
                   const int32_t* offsets, void* y_perm, void* y_shared, void* ws,
                   const FfnLayout& L, bool profile, bool planned, hipStream_t s,
                   void* h_out = nullptr, void* gu_out = nullptr) {
  if (d->T == 0) return MOE_OK;
  int32_t* tiles1 = at<int32_t>(ws, L.tiles1);
  int32_t* tiles2 = at<int32_t>(ws, L.tiles2);
  FfnArgs a{};
  a.offsets = offsets;
  a.tiles1 = tiles1;
  a.tiles2 = tiles2;
  a.T = d->T;
  a.TK = d->T * d->top_k;
  a.E = d->n_experts;
  a.d = d->d;
  a.I = d->inter;
  a.Is = d->shared_inter;
  a.ldh = L.ldh;
  a.perm = x_perm ? nullptr : perm;
  a.xperm = x_perm;
  a.xperm_scale = x_perm_scale;
  a.w13 = w->w13;
  a.ws13 = w->ws13;
  a.w13_scale = w->w13_scale;
  a.ws13_scale = w->ws13_scale;
  a.w2 = w->w2;
  a.ws2 = w->ws2;
  a.w2_scale = w->w2_scale;
  a.ws2_scale = w->ws2_scale;
  // training: bf16 weights keep H itself, FP8 weights its E4M3 codes in the
  // workspace and a bf16 copy in h_out
  const bool fp8w = d->w_dtype == MOE_DT_FP8_E4M3;
  a.H = (h_out && !fp8w) ? h_out : at<void>(ws, L.H);
  a.h16 = fp8w ? h_out : nullptr;
  a.H_scale = at<float>(ws, L.Hs);
  a.xsT = at<float>(ws, L.xsT);
  a.gu = gu_out;
  a.yperm = y_perm;
  a.yshared = y_shared;
  if (!planned)
    HIP_TRY(launch_plan(nullptr, offsets, nullptr, tiles1, tiles2, plan_params(d, L.tiling), s),
            "plan");
  if (d->w_dtype == MOE_DT_FP8_E4M3) {
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    float* xs = at<float>(ws, L.xs);
    HIP_TRY(launch_quant_rows(x, MOE_DT_BF16, nullptr, d->T, d->d, xq, xs, s), "quantize x");
    a.x = xq;
    a.x_scale = xs;
  } else {
    a.x = x;
  }
  hipEvent_t mid = nullptr;
  if (profile) {
    HIP_TRY(prof_record(2, s), "profile event");
    mid = g_prof_on ? g_prof[3] : nullptr;
  }
  if (d->w_dtype == MOE_DT_FP8_E4M3)
    HIP_TRY(launch_ffn_fp8(a, L.tiling, s, mid), "expert ffn (fp8)");
  else if (d->w_dtype == MOE_DT_BF16)
    HIP_TRY(launch_ffn_bf16(a, L.tiling, s, mid), "expert ffn (bf16)");
  else
    HIP_TRY(launch_ffn_f32(a, s, mid), "expert ffn (fp32)");
  if (profile) HIP_TRY(prof_record(4, s), "profile event");
  return MOE_OK;
}

// ---- training ---------------------------------------------------------------

moe_status validate_train(const moe_layer_desc* d) {
  moe_status st = validate_desc(d);
  if (st) return st;
  if (d->act_dtype != MOE_DT_BF16 ||
      (d->w_dtype != MOE_DT_BF16 && d->w_dtype != MOE_DT_FP8_E4M3))
    return fail(MOE_ERR_UNSUPPORTED,
                "training supports bf16 activations with bf16 or FP8 weights only");
  // 32-bit byte offsets of the backward's buffers: the input-gradient GEMMs
  // address their row operands per tile from a 64-bit base; the
  // weight-gradient GEMMs address one group's rows (an expert's segment, or
  // all T rows for the shared expert) of x, dY, H and [da | db] as one range
  const int64_t lim = (int64_t(1) << 31) - 1;
  const int64_t ldh = std::max(d->inter, d->shared_inter);
  if (d->T * std::max<int64_t>(d->d, 2 * ldh) * 2 > lim)
    return fail(MOE_ERR_UNSUPPORTED,
                "T*max(d, 2*max(I,Is))*2 must be < 2^31 bytes for training");
  // one expert's fp32 weight gradient (the largest, [2 max(I,Is), d]) is
  // written through a buffer resource whose byte size must stay below 2^31,
  // so that the out-of-range offset of masked epilogue entries lies past it
  if (2 * ldh * d->d * 4 > lim)
    return fail(MOE_ERR_UNSUPPORTED, "2*max(I,Is)*d*4 must be < 2^31 bytes for training");
  return MOE_OK;
}

moe_status check_saved(const moe_layer_desc* d, const moe_saved* sv) {
  if (!sv) return fail(MOE_ERR_INVALID_ARGUMENT, "saved is NULL");
  return check_ptrs({{sv->logits, "saved.logits"}, {sv->topk_idx, "saved.topk_idx"},
                     {sv->topk_gate, "saved.topk_gate"}, {sv->counts, "saved.counts"},
                     {sv->offsets, "saved.offsets"}, {sv->perm, "saved.perm"},
                     {sv->inv, "saved.inv"}, {sv->h, "saved.h"}, {sv->gu, "saved.gu"},
                     {sv->y_perm, "saved.y_perm"}});
}

struct BwdLayout {
  int ldh;
  size_t tiles_h, tiles_d, dyp, du, du_perm, dg, dap, das, xperm, bytes;
};

BwdLayout bwd_layout(const moe_layer_desc* d) {
  BwdLayout L{};
  const int64_t T = d->T, TK = d->T * d->top_k;
  const int E = d->n_experts;
  L.ldh = std::max(d->inter, d->shared_inter);
  const int64_t hrows = TK + (d->shared_inter > 0 ? T : 0);
  Carver c;
  L.tiles_h = c.take(sizeof(int32_t) * (E + 2));
  L.tiles_d = c.take(sizeof(int32_t) * (E + 2));
  L.dyp = c.take(size_t(TK) * d->d * 2);
  L.du = c.take(sizeof(float) * size_t(TK));
  L.du_perm = c.take(sizeof(float) * size_t(TK));
  L.dg = c.take(size_t(hrows) * 2 * L.ldh * 2);
  L.dap = c.take(size_t(TK) * d->d * 2);
  L.das = c.take(d->shared_inter > 0 ? size_t(T) * d->d * 2 : 0);
  L.xperm = c.take(size_t(TK) * d->d * 2);
  L.bytes = c.off;
  return L;
}

// Workspace of the FP8 backward. The transposed 128x1-tile operands of the
// weight-gradient GEMMs hold, per routed expert, its tokens padded to a
// multiple of 128 (at most TK + 128 E in all), then the shared rows.
struct Bwd8Layout {
  int ldh;
  int64_t rblocks, sblocks;  // upper bounds of the 128-row blocks: routed, shared
  size_t tiles_h, tiles_d, qtiles, dyp, du, du_perm, dyq, dys, dysq, dyss, dg, dgq, dgs, dap,
      das, qt_dy, qs_dy, qt_h, qs_h, qt_dg, qs_dg, qt_x, qs_x, bytes;
};

Bwd8Layout bwd8_layout(const moe_layer_desc* d) {
  Bwd8Layout L{};
  const int64_t T = d->T, TK = d->T * d->top_k;
  const int E = d->n_experts, D = d->d, I = d->inter, Is = d->shared_inter;
  L.ldh = std::max(I, Is);
  const int64_t hrows = TK + (Is > 0 ? T : 0);
  L.rblocks = (TK + 127) / 128 + E;
  L.sblocks = Is > 0 ? (T + 127) / 128 : 0;
  auto qt = [&](int64_t cr, int64_t cs) { return size_t(cr * 128 * L.rblocks + cs * 128 * L.sblocks); };
  auto qs = [&](int64_t cr, int64_t cs) { return sizeof(float) * size_t(cr * L.rblocks + cs * L.sblocks); };
  Carver c;
  L.tiles_h = c.take(sizeof(int32_t) * (E + 2));
  L.tiles_d = c.take(sizeof(int32_t) * (E + 2));
  L.qtiles = c.take(sizeof(int32_t) * (E + 2));
  L.dyp = c.take(size_t(TK) * D * 2);
  L.du = c.take(sizeof(float) * size_t(TK));
  L.du_perm = c.take(sizeof(float) * size_t(TK));
  L.dyq = c.take(size_t(TK) * D);
  L.dys = c.take(sizeof(float) * size_t(TK) * (D / 128));
  L.dysq = c.take(Is > 0 ? size_t(T) * D : 0);
  L.dyss = c.take(Is > 0 ? sizeof(float) * size_t(T) * (D / 128) : 0);
  L.dg = c.take(size_t(hrows) * 2 * L.ldh * 2);
  L.dgq = c.take(size_t(hrows) * 2 * L.ldh);
  L.dgs = c.take(sizeof(float) * size_t(hrows) * (2 * L.ldh / 128));
  L.dap = c.take(size_t(TK) * D * 2);
  L.das = c.take(Is > 0 ? size_t(T) * D * 2 : 0);
  L.qt_dy = c.take(qt(D, D));
  L.qs_dy = c.take(qs(D, D));
  L.qt_h = c.take(qt(I, Is));
  L.qs_h = c.take(qs(I, Is));
  L.qt_dg = c.take(qt(2 * int64_t(I), 2 * int64_t(Is)));
  L.qs_dg = c.take(qs(2 * int64_t(I), 2 * int64_t(Is)));
  L.qt_x = c.take(qt(D, D));
  L.qs_x = c.take(qs(D, D));
  L.bytes = c.off;
  return L;
}

moe_status zero_grads(const moe_layer_desc* desc, const moe_grads* g, hipStream_t stream) {
  const int E = desc->n_experts, d = desc->d, I = desc->inter, Is = desc->shared_inter;
  HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dw13), int64_t(E) * 2 * I * d, 0, stream),
          "zero dw13");
  HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dw2), int64_t(E) * d * I, 0, stream),
          "zero dw2");
  HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dw_router), int64_t(E) * d, 0, stream),
          "zero dw_router");
  if (Is > 0) {
    HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dws13), int64_t(2) * Is * d, 0, stream),
            "zero dws13");
    HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dws2), int64_t(d) * Is, 0, stream),
            "zero dws2");
  }
  return MOE_OK;
}

// ---- sequence-level balance loss ---------------------------------------------

int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

moe_status validate_seq_balance(const moe_layer_desc* d, int32_t seq_len) {
  moe_status st = validate_desc(d);
  if (st) return st;
  if (d->act_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the balance loss supports bf16 activations only");
  if (seq_len < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "seq_len must be >= 1 (got %d)", seq_len);
  if (d->T % seq_len != 0)
    return fail(MOE_ERR_INVALID_ARGUMENT, "seq_len %d does not divide T = %lld", seq_len,
                static_cast<long long>(d->T));
  // 32-bit byte offsets of the two products' operands and outputs
  const int64_t lim = (int64_t(1) << 31) - 1;
  const int64_t T = d->T, E = d->n_experts;
  if (T * d->d * 4 > lim) return fail(MOE_ERR_UNSUPPORTED, "T*d*4 must be < 2^31 bytes");
  if (T * round8(E) * 2 > lim || E * round8(T) * 2 > lim)
    return fail(MOE_ERR_UNSUPPORTED, "T*E*2 must be < 2^31 bytes");
  return MOE_OK;
}

struct SeqBalLayout {
  int64_t n_seq, chunks, ldE, ldT;
  int groups, group_step;  // token groups of the split router weight gradient
  size_t part_p, part_c, f, du16, duT16, wr16, goff, gpart, bytes;
};

SeqBalLayout seqbal_layout(const moe_layer_desc* d, int32_t seq_len) {
  SeqBalLayout L{};
  const int64_t T = d->T, E = d->n_experts;
  L.n_seq = T / seq_len;
  L.chunks = L.n_seq * ((seq_len + kBalanceChunk - 1) / kBalanceChunk);
  L.ldE = round8(E);
  L.ldT = round8(T);
  // dW_r = du^T x has few output tiles (E x d over 128 x 256): its
  // contraction over the tokens is split into up to 16 groups of at least 64
  // tokens, so that about 512 tiles run, and the partial products are added
  // in group order. A function of the descriptor only.
  const int64_t tiles = ((E + 127) / 128) * ((d->d + 255) / 256);
  int64_t g = std::min<int64_t>({16, (512 + tiles - 1) / tiles, (T + 63) / 64});
  g = std::max<int64_t>(g, 1);
  L.group_step = static_cast<int>(((T + g - 1) / g + 63) / 64 * 64);
  L.groups = T > 0 ? static_cast<int>((T + L.group_step - 1) / L.group_step) : 1;
  Carver c;
  L.part_p = c.take(sizeof(float) * size_t(L.chunks * E));
  L.part_c = c.take(sizeof(int32_t) * size_t(L.chunks * E));
  L.f = c.take(sizeof(float) * size_t(L.n_seq * E));
  L.du16 = c.take(size_t(T) * L.ldE * 2);
  L.duT16 = c.take(size_t(E) * L.ldT * 2);
  L.wr16 = c.take(size_t(E) * d->d * 2);
  L.goff = c.take(sizeof(int32_t) * size_t(L.groups + 1));
  L.gpart = c.take(L.groups > 1 ? sizeof(float) * size_t(L.groups) * E * d->d : 0);
  L.bytes = c.off;
  return L;
}

moe_status check_forward_ptrs(const void* x, const float* w_router, const float* bias, void* y,
                              int32_t* topk_idx, float* topk_gate, int32_t* counts,
                              int32_t* near_tie, float* logits) {
  moe_status st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {bias, "bias"}, {y, "y"},
                              {topk_idx, "topk_idx"}, {topk_gate, "topk_gate"},
                              {counts, "counts"}});
  if (st) return st;
  return check_opt({{near_tie, "near_tie"}, {logits, "logits"}});
}

moe_status run_forward(const moe_layer_desc* desc, const void* x, const float* w_router,
                       const float* bias, const moe_weights* w, void* y, int32_t* topk_idx,
                       float* topk_gate, int32_t* counts, int32_t* near_tie, float* logits,
                       void* ws, const FwdLayout& L, hipStream_t stream);

// ---- fixed scratch of the allocation-free forward ------------------------------
//
// Workspace of deepseek_moe_forward_noalloc: a file-scope device array, so the
// call allocates nothing. Each GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` only names the array: its
// device address, per GPU, comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is passed on.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_ptr(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return DSMOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

moe_status moe_workspace_size(const moe_layer_desc* desc, size_t* bytes) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = fwd_layout(desc).bytes;
  return MOE_OK;
}

moe_status moe_gate(const moe_layer_desc* desc, const void* x, const float* w_router,
                    const float* bias, float* logits, int32_t* topk_idx, float* topk_gate,
                    int32_t* counts, int32_t* near_tie, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  if (desc->T == 0) return zero_counts(desc, counts, near_tie, stream);
  st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {bias, "bias"}, {topk_idx, "topk_idx"},
                   {topk_gate, "topk_gate"}, {counts, "counts"}, {ws, "ws"}});
  if (st) return st;
  st = check_opt({{logits, "logits"}, {near_tie, "near_tie"}});
  if (st) return st;
  const GateLayout L = gate_layout(desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_gate needs %zu workspace bytes, got %zu",
                L.bytes, ws_bytes);
  return run_gate(desc, x, w_router, bias, logits, topk_idx, topk_gate, counts, near_tie, ws, L,
                  stream);
}

moe_status moe_route_from_logits(const moe_layer_desc* desc, const float* logits,
                                 const float* bias, int32_t* topk_idx, float* topk_gate,
                                 int32_t* counts, int32_t* near_tie, hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  if (desc->T == 0) return zero_counts(desc, counts, near_tie, stream);
  st = check_ptrs({{logits, "logits"}, {bias, "bias"}, {topk_idx, "topk_idx"},
                   {topk_gate, "topk_gate"}, {counts, "counts"}, {near_tie, "near_tie"}});
  if (st) return st;
  HIP_TRY(launch_fill_i32(counts, desc->n_experts, 0, stream), "zero counts");
  HIP_TRY(launch_fill_i32(near_tie, 1, 0, stream), "zero near_tie");
  if (desc->T == 0) return MOE_OK;
  HIP_TRY(launch_route(logits, 1, nullptr, bias, route_params(desc), topk_idx, topk_gate, counts,
                       near_tie, stream),
          "route");
  return MOE_OK;
}

moe_status moe_permute(const moe_layer_desc* desc, const int32_t* topk_idx,
                       const int32_t* counts, const void* x, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* x_perm, float* x_perm_scale, hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  if (desc->T == 0) {
    st = check_ptrs({{offsets, "offsets"}});
    if (st) return st;
    HIP_TRY(launch_fill_i32(offsets, desc->n_experts + 1, 0, stream), "zero offsets");
    return MOE_OK;
  }
  st = check_ptrs({{topk_idx, "topk_idx"}, {counts, "counts"}, {offsets, "offsets"},
                   {perm, "perm"}, {inv, "inv"}});
  if (st) return st;
  if (x_perm) {
    st = check_ptrs({{x, "x"}});
    if (st) return st;
    if (desc->w_dtype == MOE_DT_FP8_E4M3) {
      st = check_ptrs({{x_perm_scale, "x_perm_scale"}});
      if (st) return st;
    }
    st = check_opt({{x_perm, "x_perm"}});
    if (st) return st;
  }
  PlanParams pp = plan_params(desc, choose_tiling(desc->T, desc->top_k, desc->n_experts,
                                                  desc->w_dtype));
  HIP_TRY(launch_plan(counts, nullptr, offsets, nullptr, nullptr, pp, stream),
          "offsets");
  if (desc->T == 0) return MOE_OK;
  HIP_TRY(launch_permute(topk_idx, offsets, desc->T, desc->top_k, desc->n_experts, perm, inv,
                         stream),
          "permute");
  if (x_perm) {
    const int64_t TK = desc->T * desc->top_k;
    if (desc->w_dtype == MOE_DT_FP8_E4M3)
      HIP_TRY(launch_quant_rows(x, MOE_DT_BF16, perm, TK, desc->d,
                                static_cast<uint8_t*>(x_perm), x_perm_scale, stream),
              "quantize gathered rows");
    else
      HIP_TRY(launch_gather_rows(x, desc->T, perm, TK, int64_t(desc->d) * io_bytes(desc), x_perm,
                                 stream),
              "gather rows");
  }
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_weights* w, const void* x,
                          const int32_t* perm, const void* x_perm, const float* x_perm_scale,
                          const int32_t* offsets, void* y_perm, void* y_shared, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  st = check_weights(desc, w);
  if (st) return st;
  if (desc->T == 0) return MOE_OK;
  st = check_ptrs({{x, "x"}, {offsets, "offsets"}, {y_perm, "y_perm"}, {ws, "ws"}});
  if (st) return st;
  if (!x_perm) {
    st = check_ptrs({{perm, "perm"}});
    if (st) return st;
  } else if (desc->w_dtype == MOE_DT_FP8_E4M3) {
    st = check_ptrs({{x_perm, "x_perm"}, {x_perm_scale, "x_perm_scale"}});
    if (st) return st;
  } else {
    st = check_ptrs({{x_perm, "x_perm"}});
    if (st) return st;
  }
  if (x_perm) {
    const int64_t s = desc->w_dtype == MOE_DT_FP8_E4M3 ? 1 : io_bytes(desc);
    if (desc->T * desc->top_k * desc->d * s > (int64_t(1) << 31) - 1)
      return fail(MOE_ERR_UNSUPPORTED, "T*K*d*sizeof(x_perm) must be < 2^31 bytes");
  }
  if (desc->shared_inter > 0) {
    st = check_ptrs({{y_shared, "y_shared"}});
    if (st) return st;
  }
  const FfnLayout L = ffn_layout(desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_expert_ffn needs %zu workspace bytes, got %zu",
                L.bytes, ws_bytes);
  return run_ffn(desc, w, x, perm, x_perm, x_perm_scale, offsets, y_perm, y_shared, ws, L, false,
                 false, stream);
}

moe_status moe_combine(const moe_layer_desc* desc, const void* y_perm, const int32_t* inv,
                       const float* topk_gate, const void* y_shared, void* y,
                       hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  if (desc->T == 0) return MOE_OK;
  st = check_ptrs({{y_perm, "y_perm"}, {inv, "inv"}, {topk_gate, "topk_gate"}, {y, "y"}});
  if (st) return st;
  st = check_opt({{y_shared, "y_shared"}});
  if (st) return st;
  HIP_TRY(launch_combine(y_perm, inv, topk_gate, desc->shared_inter > 0 ? y_shared : nullptr, y,
                         desc->T, desc->top_k, desc->d, desc->act_dtype, desc->out_dtype, stream),
          "combine");
  return MOE_OK;
}

moe_status moe_bias_update(const moe_layer_desc* desc, const int32_t* counts, float gamma,
                           float* bias, hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  st = check_ptrs({{counts, "counts"}, {bias, "bias"}});
  if (st) return st;
  if (!std::isfinite(gamma)) return fail(MOE_ERR_INVALID_ARGUMENT, "gamma must be finite");
  HIP_TRY(launch_bias_update(counts, gamma, bias, desc->n_experts, desc->T, desc->top_k, stream),
          "bias update");
  return MOE_OK;
}

moe_status deepseek_moe_forward(const moe_layer_desc* desc, const void* x,
                                const float* w_router, const float* bias, const moe_weights* w,
                                void* y, int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                int32_t* near_tie, float* logits, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  st = check_weights(desc, w);
  if (st) return st;
  if (desc->T == 0) return zero_counts(desc, counts, near_tie, stream);
  st = check_forward_ptrs(x, w_router, bias, y, topk_idx, topk_gate, counts, near_tie, logits);
  if (st) return st;
  st = check_ptrs({{ws, "ws"}});
  if (st) return st;
  const FwdLayout L = fwd_layout(desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "deepseek_moe_forward needs %zu workspace bytes, got %zu", L.bytes, ws_bytes);
  return run_forward(desc, x, w_router, bias, w, y, topk_idx, topk_gate, counts, near_tie, logits,
                     ws, L, stream);
}

moe_status deepseek_moe_forward_noalloc(const moe_layer_desc* desc, const void* x,
                                        const float* w_router, const float* bias,
                                        const moe_weights* w, void* y, int32_t* topk_idx,
                                        float* topk_gate, int32_t* counts, int32_t* near_tie,
                                        float* logits, hipStream_t stream) {
  moe_status st = validate_desc(desc);
  if (st) return st;
  st = check_weights(desc, w);
  if (st) return st;
  if (desc->T == 0) return zero_counts(desc, counts, near_tie, stream);
  st = check_forward_ptrs(x, w_router, bias, y, topk_idx, topk_gate, counts, near_tie, logits);
  if (st) return st;
  const FwdLayout L = fwd_layout(desc);
  if (L.bytes > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "deepseek_moe_forward_noalloc: this call needs %zu workspace bytes, the fixed "
                "scratch holds %zu (use deepseek_moe_forward with a caller workspace)",
                L.bytes, kScratchBytes);
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st) return st;
  return run_forward(desc, x, w_router, bias, w, y, topk_idx, topk_gate, counts, near_tie, logits,
                     ws, L, stream);
}

}  // extern "C"

namespace {

// The forward on a validated call (T > 0) with workspace ws of L.bytes.
moe_status run_forward(const moe_layer_desc* desc, const void* x, const float* w_router,
                       const float* bias, const moe_weights* w, void* y, int32_t* topk_idx,
                       float* topk_gate, int32_t* counts, int32_t* near_tie, float* logits,
                       void* ws, const FwdLayout& L, hipStream_t stream) {
  moe_status st;
  void* gws = at<void>(ws, L.gate_base);
  void* fws = at<void>(ws, L.ffn_base);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);
  void* yperm = at<void>(ws, L.yperm);
  void* yshared = desc->shared_inter > 0 ? at<void>(ws, L.yshared) : nullptr;
  HIP_TRY(prof_record(0, stream), "profile event");
  st = run_gate(desc, x, w_router, bias, logits, topk_idx, topk_gate, counts, near_tie, gws,
                L.gate, stream);
  if (st) return st;
  HIP_TRY(prof_record(1, stream), "profile event");
  HIP_TRY(launch_plan(counts, nullptr, offsets, at<int32_t>(fws, L.ffn.tiles1),
                      at<int32_t>(fws, L.ffn.tiles2), plan_params(desc, L.ffn.tiling), stream),
          "plan");
  HIP_TRY(launch_permute(topk_idx, offsets, desc->T, desc->top_k, desc->n_experts, perm, inv,
                         stream),
          "permute");
  st = run_ffn(desc, w, x, perm, nullptr, nullptr, offsets, yperm, yshared, fws, L.ffn, true,
               true, stream);
  if (st) return st;
  HIP_TRY(launch_combine(yperm, inv, topk_gate, yshared, y, desc->T, desc->top_k, desc->d,
                         desc->act_dtype, desc->out_dtype, stream),
          "combine");
  HIP_TRY(prof_record(5, stream), "profile event");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_profile_events(const hipEvent_t* events, int32_t n_events) {
  if (!events || n_events == 0) {
    g_prof_on = false;
    return MOE_OK;
  }
  if (n_events < 6) return fail(MOE_ERR_INVALID_ARGUMENT, "need 6 events, got %d", n_events);
  for (int i = 0; i < 6; ++i) {
    if (!events[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "event %d is NULL", i);
    g_prof[i] = events[i];
  }
  g_prof_on = true;
  return MOE_OK;
}

moe_status moe_quantize_fp8_blocks(const void* src, int32_t src_dtype, int64_t n_mats,
                                   int32_t rows, int32_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream) {
  if (src_dtype != MOE_DT_F32 && src_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "src_dtype %d not supported", src_dtype);
  if (n_mats < 0 || rows < 0 || cols < 0 || rows % 128 || cols % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "rows and cols must be non-negative multiples of 128");
  if (n_mats * (rows / 128) * int64_t(cols / 128) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "too many blocks");
  moe_status st = check_ptrs({{src, "src"}, {q, "q"}, {scale, "scale"}});
  if (st) return st;
  HIP_TRY(launch_quant_blocks(src, src_dtype, n_mats, rows, cols, q, scale, stream),
          "quantize blocks");
  return MOE_OK;
}

moe_status moe_quantize_fp8_rows(const void* src, int32_t src_dtype, int64_t n, int32_t cols,
                                 uint8_t* q, float* scale, hipStream_t stream) {
  if (src_dtype != MOE_DT_F32 && src_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "src_dtype %d not supported", src_dtype);
  if (n < 0 || cols < 0 || cols % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cols must be a non-negative multiple of 128");
  if ((n * (cols / 128) + 3) / 4 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "too many tiles");
  moe_status st = check_ptrs({{src, "src"}, {q, "q"}, {scale, "scale"}});
  if (st) return st;
  HIP_TRY(launch_quant_rows(src, src_dtype, nullptr, n, cols, q, scale, stream), "quantize rows");
  return MOE_OK;
}

moe_status moe_forward_train(const moe_layer_desc* desc, const void* x, const float* w_router,
                             const float* bias, const moe_weights* w, void* y,
                             const moe_saved* sv, int32_t* near_tie, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  moe_status st = validate_train(desc);
  if (st) return st;
  st = check_weights(desc, w);
  if (st) return st;
  if (!sv) return fail(MOE_ERR_INVALID_ARGUMENT, "saved is NULL");
  if (desc->T == 0) {
    st = check_ptrs({{sv->counts, "saved.counts"}, {sv->offsets, "saved.offsets"}});
    if (st) return st;
    st = zero_counts(desc, sv->counts, near_tie, stream);
    if (st) return st;
    HIP_TRY(launch_fill_i32(sv->offsets, desc->n_experts + 1, 0, stream), "zero offsets");
    return MOE_OK;
  }
  st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {bias, "bias"}, {y, "y"}, {ws, "ws"}});
  if (st) return st;
  st = check_saved(desc, sv);
  if (st) return st;
  st = check_opt({{near_tie, "near_tie"}});
  if (st) return st;
  const FwdLayout L = fwd_layout(desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_forward_train needs %zu workspace bytes, got %zu",
                L.bytes, ws_bytes);
  void* gws = at<void>(ws, L.gate_base);
  void* fws = at<void>(ws, L.ffn_base);
  void* yshared = desc->shared_inter > 0 ? at<void>(ws, L.yshared) : nullptr;
  st = run_gate(desc, x, w_router, bias, sv->logits, sv->topk_idx, sv->topk_gate, sv->counts,
                near_tie, gws, L.gate, stream);
  if (st) return st;
  HIP_TRY(launch_plan(sv->counts, nullptr, sv->offsets, at<int32_t>(fws, L.ffn.tiles1),
                      at<int32_t>(fws, L.ffn.tiles2), plan_params(desc, L.ffn.tiling), stream),
          "plan");
  HIP_TRY(launch_permute(sv->topk_idx, sv->offsets, desc->T, desc->top_k, desc->n_experts,
                         sv->perm, sv->inv, stream),
          "permute");
  st = run_ffn(desc, w, x, sv->perm, nullptr, nullptr, sv->offsets, sv->y_perm, yshared, fws,
               L.ffn, false, true, stream, sv->h, sv->gu);
  if (st) return st;
  HIP_TRY(launch_combine(sv->y_perm, sv->inv, sv->topk_gate, yshared, y, desc->T, desc->top_k,
                         desc->d, desc->act_dtype, desc->out_dtype, stream),
          "combine");
  return MOE_OK;
}

moe_status moe_backward_workspace_size(const moe_layer_desc* desc, size_t* bytes) {
  moe_status st = validate_train(desc);
  if (st) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = desc->w_dtype == MOE_DT_FP8_E4M3 ? bwd8_layout(desc).bytes : bwd_layout(desc).bytes;
  return MOE_OK;
}

moe_status moe_backward(const moe_layer_desc* desc, const void* x, const float* w_router,
                        const moe_weights* w, const moe_saved* sv, const void* dy, void* dx,
                        const moe_grads* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate_train(desc);
  if (st) return st;
  if (desc->w_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_backward takes bf16 weights; FP8 weights go through moe_backward_fp8");
  const int64_t T = desc->T, TK = T * desc->top_k;
  const int E = desc->n_experts, d = desc->d, I = desc->inter, Is = desc->shared_inter;
  const int K = desc->top_k;
  const bool shared = Is > 0;
  if (!g) return fail(MOE_ERR_INVALID_ARGUMENT, "grads is NULL");
  st = check_ptrs({{g->dw13, "dw13"}, {g->dw2, "dw2"}, {g->dw_router, "dw_router"}});
  if (st) return st;
  if (shared) {
    st = check_ptrs({{g->dws13, "dws13"}, {g->dws2, "dws2"}});
    if (st) return st;
  }
  if (T == 0) {
    // no token: every weight gradient is zero
    HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dw13), int64_t(E) * 2 * I * d, 0, stream),
            "zero dw13");
    HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dw2), int64_t(E) * d * I, 0, stream),
            "zero dw2");
    HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dw_router), int64_t(E) * d, 0, stream),
            "zero dw_router");
    if (shared) {
      HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dws13), int64_t(2) * Is * d, 0, stream),
              "zero dws13");
      HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(g->dws2), int64_t(d) * Is, 0, stream),
              "zero dws2");
    }
    return MOE_OK;
  }
  st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {dy, "dy"}, {dx, "dx"}, {ws, "ws"}});
  if (st) return st;
  st = check_weights(desc, w);
  if (st) return st;
  st = check_saved(desc, sv);
  if (st) return st;
  const BwdLayout L = bwd_layout(desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_backward needs %zu workspace bytes, got %zu",
                L.bytes, ws_bytes);
  int32_t* tiles_h = at<int32_t>(ws, L.tiles_h);
  int32_t* tiles_d = at<int32_t>(ws, L.tiles_d);
  void* dyp = at<void>(ws, L.dyp);
  float* du = at<float>(ws, L.du);
  float* du_perm = at<float>(ws, L.du_perm);
  void* dgb = at<void>(ws, L.dg);
  void* dap = at<void>(ws, L.dap);
  void* das = shared ? at<void>(ws, L.das) : nullptr;
  void* xperm = at<void>(ws, L.xperm);
  const int ldh = L.ldh;

  // tile tables: 128-row tiles over 256-column tiles of Ig (dgrad2) and d (dgrad1)
  PlanParams pp{};
  pp.T = T;
  pp.E = E;
  pp.K = K;
  pp.d = d;
  pp.I = I;
  pp.Is = Is;
  pp.bm1 = 128;
  pp.bnh1 = 256;
  pp.bm2 = 128;
  pp.bn2 = 256;
  HIP_TRY(launch_plan(nullptr, sv->offsets, nullptr, tiles_h, tiles_d, pp, stream), "plan");
  HIP_TRY(launch_bwd_gate(dy, sv->y_perm, sv->topk_idx, sv->inv, sv->topk_gate, sv->logits, T, K,
                          E, d, dyp, du, du_perm, stream),
          "gate gradients");
  BwdArgs b{};
  b.offsets = sv->offsets;
  b.tiles = tiles_h;
  b.T = T;
  b.TK = TK;
  b.E = E;
  b.d = d;
  b.I = I;
  b.Is = Is;
  b.ldh = ldh;
  b.dyp = dyp;
  b.dy = dy;
  b.w2 = w->w2;
  b.ws2 = w->ws2;
  b.w13 = w->w13;
  b.ws13 = w->ws13;
  b.gu = sv->gu;
  b.dg = dgb;
  b.dap = dap;
  b.das = das;
  HIP_TRY(launch_dgrad2_bf16(b, stream), "dgrad of the down projection");
  b.tiles = tiles_d;
  HIP_TRY(launch_dgrad1_bf16(b, stream), "dgrad of the gate/up projection");
  HIP_TRY(launch_bwd_combine(dap, das, sv->inv, sv->topk_idx, du, w_router, T, K, d, dx, stream),
          "input gradient");
  HIP_TRY(launch_router_wgrad(x, sv->perm, sv->offsets, du_perm, E, d, g->dw_router, stream),
          "router weight gradient");
  // weight gradients: contractions over each expert's rows; A_e of the
  // gate/up projection is x gathered into the routed order
  HIP_TRY(launch_gather_rows(x, T, sv->perm, TK, int64_t(d) * 2, xperm, stream), "gather x");
  const uint16_t* dg16 = static_cast<const uint16_t*>(dgb);
  const uint16_t* h16 = static_cast<const uint16_t*>(sv->h);
  WgradArgs w1{};
  w1.offsets = sv->offsets;
  w1.E = E;
  w1.T = T;
  w1.shared = shared;
  w1.a = dg16;
  w1.a_s = dg16 + TK * 2 * ldh;
  w1.lda = w1.lda_s = 2 * int64_t(ldh);
  w1.b = xperm;
  w1.b_s = x;
  w1.ldb = w1.ldb_s = d;
  w1.M = 2 * I;
  w1.N = d;
  w1.Ms = 2 * Is;
  w1.Ns = d;
  w1.out = g->dw13;
  w1.out_s = g->dws13;
  HIP_TRY(launch_wgrad_bf16(w1, stream), "weight gradient of the gate/up projection");
  WgradArgs w2{};
  w2.offsets = sv->offsets;
  w2.E = E;
  w2.T = T;
  w2.shared = shared;
  w2.a = dyp;
  w2.a_s = dy;
  w2.lda = w2.lda_s = d;
  w2.b = h16;
  w2.b_s = h16 + TK * ldh;
  w2.ldb = w2.ldb_s = ldh;
  w2.M = d;
  w2.N = I;
  w2.Ms = d;
  w2.Ns = Is;
  w2.out = g->dw2;
  w2.out_s = g->dws2;
  HIP_TRY(launch_wgrad_bf16(w2, stream), "weight gradient of the down projection");
  return MOE_OK;
}

moe_status moe_transpose_fp8_blocks(const uint8_t* q, const float* scale, int64_t n_mats,
                                    int32_t rows, int32_t cols, uint8_t* qt, float* scale_t,
                                    hipStream_t stream) {
  if (n_mats < 0 || rows < 0 || cols < 0 || rows % 128 || cols % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "rows and cols must be non-negative multiples of 128");
  if (n_mats * (rows / 64) * int64_t(cols / 64) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "too many blocks");
  moe_status st = check_ptrs({{q, "q"}, {scale, "scale"}, {qt, "qt"}, {scale_t, "scale_t"}});
  if (st) return st;
  HIP_TRY(launch_transpose_fp8(q, scale, n_mats, rows, cols, qt, scale_t, stream),
          "transpose FP8 blocks");
  return MOE_OK;
}

moe_status moe_backward_fp8(const moe_layer_desc* desc, const void* x, const float* w_router,
                            const moe_weights* w, const moe_weights* wt, const moe_saved* sv,
                            const void* dy, void* dx, const moe_grads* g, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate_train(desc);
  if (st) return st;
  if (desc->w_dtype != MOE_DT_FP8_E4M3)
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward_fp8 takes FP8 weights (w_dtype E4M3)");
  const int64_t T = desc->T, TK = T * desc->top_k;
  const int E = desc->n_experts, d = desc->d, I = desc->inter, Is = desc->shared_inter;
  const int K = desc->top_k;
  const bool shared = Is > 0;
  if (!g) return fail(MOE_ERR_INVALID_ARGUMENT, "grads is NULL");
  st = check_ptrs({{g->dw13, "dw13"}, {g->dw2, "dw2"}, {g->dw_router, "dw_router"}});
  if (st) return st;
  if (shared) {
    st = check_ptrs({{g->dws13, "dws13"}, {g->dws2, "dws2"}});
    if (st) return st;
  }
  if (T == 0) return zero_grads(desc, g, stream);
  st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {dy, "dy"}, {dx, "dx"}, {ws, "ws"}});
  if (st) return st;
  st = check_weights(desc, w);
  if (st) return st;
  if (!wt) return fail(MOE_ERR_INVALID_ARGUMENT, "transposed weights are NULL");
  st = check_ptrs({{wt->w13, "wt.w13"}, {wt->w2, "wt.w2"}, {wt->w13_scale, "wt.w13_scale"},
                   {wt->w2_scale, "wt.w2_scale"}});
  if (st) return st;
  if (shared) {
    st = check_ptrs({{wt->ws13, "wt.ws13"}, {wt->ws2, "wt.ws2"}, {wt->ws13_scale, "wt.ws13_scale"},
                     {wt->ws2_scale, "wt.ws2_scale"}});
    if (st) return st;
  }
  st = check_saved(desc, sv);
  if (st) return st;
  const Bwd8Layout L = bwd8_layout(desc);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_backward_fp8 needs %zu workspace bytes, got %zu",
                L.bytes, ws_bytes);
  const int ldh = L.ldh;
  int32_t* tiles_h = at<int32_t>(ws, L.tiles_h);
  int32_t* tiles_d = at<int32_t>(ws, L.tiles_d);
  int32_t* qtiles = at<int32_t>(ws, L.qtiles);
  void* dyp = at<void>(ws, L.dyp);
  float* du = at<float>(ws, L.du);
  float* du_perm = at<float>(ws, L.du_perm);

  // tile tables: 128 x 256 tiles over (rows, Ig) and (rows, d); 128-row
  // blocks per group for the weight-gradient operands
  PlanParams pp{};
  pp.T = T;
  pp.E = E;
  pp.K = K;
  pp.d = d;
  pp.I = I;
  pp.Is = Is;
  pp.bm1 = 128;
  pp.bnh1 = 256;
  pp.bm2 = 128;
  pp.bn2 = 256;
  HIP_TRY(launch_plan(nullptr, sv->offsets, nullptr, tiles_h, tiles_d, pp, stream), "plan");
  pp.bnh1 = 1 << 30;
  HIP_TRY(launch_plan(nullptr, sv->offsets, nullptr, qtiles, nullptr, pp, stream), "plan blocks");
  HIP_TRY(launch_bwd_gate(dy, sv->y_perm, sv->topk_idx, sv->inv, sv->topk_gate, sv->logits, T, K,
                          E, d, dyp, du, du_perm, stream),
          "gate gradients");
  // E5M2 gradients in 1x128 tiles along d for the down projection's input gradient
  BwdFp8Args b{};
  b.offsets = sv->offsets;
  b.tiles_h = tiles_h;
  b.tiles_d = tiles_d;
  b.T = T;
  b.TK = TK;
  b.E = E;
  b.d = d;
  b.I = I;
  b.Is = Is;
  b.ldh = ldh;
  b.dyq = at<uint8_t>(ws, L.dyq);
  b.dys = at<float>(ws, L.dys);
  b.dysq = shared ? at<uint8_t>(ws, L.dysq) : nullptr;
  b.dyss = shared ? at<float>(ws, L.dyss) : nullptr;
  HIP_TRY(launch_quant_rows(dyp, MOE_DT_BF16, nullptr, TK, d, at<uint8_t>(ws, L.dyq),
                            at<float>(ws, L.dys), stream, 1, true),
          "quantize gated output gradients");
  if (shared)
    HIP_TRY(launch_quant_rows(dy, MOE_DT_BF16, nullptr, T, d, at<uint8_t>(ws, L.dysq),
                              at<float>(ws, L.dyss), stream, 1, true),
            "quantize output gradient");
  b.w2t = static_cast<const uint8_t*>(wt->w2);
  b.w2t_scale = wt->w2_scale;
  b.ws2t = static_cast<const uint8_t*>(wt->ws2);
  b.ws2t_scale = wt->ws2_scale;
  b.w13t = static_cast<const uint8_t*>(wt->w13);
  b.w13t_scale = wt->w13_scale;
  b.ws13t = static_cast<const uint8_t*>(wt->ws13);
  b.ws13t_scale = wt->ws13_scale;
  b.gu = static_cast<const uint16_t*>(sv->gu);
  b.dg = at<uint16_t>(ws, L.dg);
  b.dgq = at<uint8_t>(ws, L.dgq);
  b.dgs = at<float>(ws, L.dgs);
  b.dap = at<uint16_t>(ws, L.dap);
  b.das = shared ? at<uint16_t>(ws, L.das) : nullptr;
  HIP_TRY(launch_dgrad2_fp8(b, stream), "FP8 input gradient of the down projection");
  HIP_TRY(launch_dgrad1_fp8(b, stream), "FP8 input gradient of the gate/up projection");
  HIP_TRY(launch_bwd_combine(b.dap, b.das, sv->inv, sv->topk_idx, du, w_router, T, K, d, dx, stream),
          "input gradient");
  HIP_TRY(launch_router_wgrad(x, sv->perm, sv->offsets, du_perm, E, d, g->dw_router, stream),
          "router weight gradient");
  // weight-gradient operands: 128x1 tiles down each expert's token segment,
  // written transposed (channels x tokens)
  const int64_t max_blocks = L.rblocks + L.sblocks;
  auto qcols = [&](const void* src, const int32_t* perm, int64_t ld, const void* src_s,
                   int64_t ld_s, int C, int Cs, size_t qoff, size_t soff, int fmt) {
    QuantColsArgs q{};
    q.qtiles = qtiles;
    q.offsets = sv->offsets;
    q.E = E;
    q.shared = shared;
    q.T = T;
    q.src = static_cast<const uint16_t*>(src);
    q.perm = perm;
    q.ld = ld;
    q.src_s = static_cast<const uint16_t*>(src_s);
    q.ld_s = ld_s;
    q.C = C;
    q.Cs = Cs;
    q.q = at<uint8_t>(ws, qoff);
    q.scale = at<float>(ws, soff);
    return launch_quant_cols(q, max_blocks, fmt, stream);
  };
  const uint16_t* h16 = static_cast<const uint16_t*>(sv->h);
  HIP_TRY(qcols(dyp, nullptr, d, dy, d, d, d, L.qt_dy, L.qs_dy, 1), "quantize dY (128x1)");
  HIP_TRY(qcols(h16, nullptr, ldh, h16 + TK * ldh, ldh, I, Is, L.qt_h, L.qs_h, 0),
          "quantize H (128x1)");
  HIP_TRY(qcols(b.dg, nullptr, 2 * ldh, b.dg + TK * 2 * ldh, 2 * ldh, 2 * I, 2 * Is, L.qt_dg,
                L.qs_dg, 1),
          "quantize [da | db] (128x1)");
  HIP_TRY(qcols(x, sv->perm, d, x, d, d, d, L.qt_x, L.qs_x, 0), "quantize x (128x1)");
  WgradFp8Args w2{};
  w2.qtiles = qtiles;
  w2.E = E;
  w2.shared = shared;
  w2.a = at<uint8_t>(ws, L.qt_dy);
  w2.as = at<float>(ws, L.qs_dy);
  w2.b = at<uint8_t>(ws, L.qt_h);
  w2.bs = at<float>(ws, L.qs_h);
  w2.M = d;
  w2.N = I;
  w2.Ms = d;
  w2.Ns = Is;
  w2.out = g->dw2;
  w2.out_s = g->dws2;
  HIP_TRY(launch_wgrad_fp8(w2, 1, 0, stream), "FP8 weight gradient of the down projection");
  WgradFp8Args w1{};
  w1.qtiles = qtiles;
  w1.E = E;
  w1.shared = shared;
  w1.a = at<uint8_t>(ws, L.qt_dg);
  w1.as = at<float>(ws, L.qs_dg);
  w1.b = at<uint8_t>(ws, L.qt_x);
  w1.bs = at<float>(ws, L.qs_x);
  w1.M = 2 * I;
  w1.N = d;
  w1.Ms = 2 * Is;
  w1.Ns = d;
  w1.out = g->dw13;
  w1.out_s = g->dws13;
  HIP_TRY(launch_wgrad_fp8(w1, 1, 0, stream), "FP8 weight gradient of the gate/up projection");
  return MOE_OK;
}

moe_status moe_seq_balance_workspace_size(const moe_layer_desc* desc, int32_t seq_len,
                                          size_t* bytes) {
  moe_status st = validate_seq_balance(desc, seq_len);
  if (st) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = seqbal_layout(desc, seq_len).bytes;
  return MOE_OK;
}

moe_status moe_seq_balance_loss(const moe_layer_desc* desc, int32_t seq_len, float alpha,
                                const void* x, const float* w_router, const float* logits,
                                const int32_t* topk_idx, float* loss, float* dlogits, float* dx,
                                float* dw_router, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate_seq_balance(desc, seq_len);
  if (st) return st;
  if (!std::isfinite(alpha)) return fail(MOE_ERR_INVALID_ARGUMENT, "alpha must be finite");
  st = check_ptrs({{dw_router, "dw_router"}});
  if (st) return st;
  const int64_t T = desc->T;
  const int E = desc->n_experts, d = desc->d;
  if (T == 0) {
    HIP_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(dw_router), int64_t(E) * d, 0, stream),
            "zero dw_router");
    return MOE_OK;
  }
  st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {logits, "logits"}, {topk_idx, "topk_idx"},
                   {loss, "loss"}, {dx, "dx"}, {ws, "ws"}});
  if (st) return st;
  st = check_opt({{dlogits, "dlogits"}});
  if (st) return st;
  const SeqBalLayout L = seqbal_layout(desc, seq_len);
  if (ws_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "moe_seq_balance_loss needs %zu workspace bytes, got %zu", L.bytes, ws_bytes);
  uint16_t* du16 = at<uint16_t>(ws, L.du16);
  uint16_t* duT16 = at<uint16_t>(ws, L.duT16);
  uint16_t* wr16 = at<uint16_t>(ws, L.wr16);
  int32_t* part_c = at<int32_t>(ws, L.part_c);
  HIP_TRY(launch_seq_balance(logits, topk_idx, T, E, desc->top_k, seq_len, alpha,
                             at<float>(ws, L.part_p), part_c, at<float>(ws, L.f), loss, dlogits,
                             du16, static_cast<int>(L.ldE), duT16, L.ldT, stream),
          "balance loss");
  HIP_TRY(launch_to_bf16(w_router, int64_t(E) * d, wr16, stream), "router weights to bf16");
  // dW_r = du^T x: contraction over the T tokens (rows of du and x), split
  // into token groups whose partial products are then added in group order
  int32_t* goff = at<int32_t>(ws, L.goff);
  HIP_TRY(launch_token_groups(goff, L.groups, L.group_step, T, stream), "token groups");
  WgradArgs a{};
  a.offsets = goff;
  a.E = L.groups;
  a.T = T;
  a.shared = false;
  a.a = du16;
  a.lda = L.ldE;
  a.b = x;
  a.ldb = d;
  a.M = E;
  a.N = d;
  a.out = L.groups > 1 ? at<float>(ws, L.gpart) : dw_router;
  HIP_TRY(launch_wgrad_bf16(a, stream), "balance loss: router weight gradient");
  if (L.groups > 1)
    HIP_TRY(launch_sum_groups(at<float>(ws, L.gpart), L.groups, int64_t(E) * d, dw_router, stream),
            "balance loss: router weight gradient groups");
  // dx = du W_r = (du^T)^T W_r: contraction over the E experts (rows of du^T
  // and W_r)
  WgradArgs b{};
  b.offsets = goff;  // no routed groups: only its first entry is read
  b.E = 0;
  b.T = E;
  b.shared = true;
  b.a_s = duT16;
  b.lda_s = L.ldT;
  b.b_s = wr16;
  b.ldb_s = d;
  b.Ms = static_cast<int>(T);
  b.Ns = d;
  b.out_s = dx;
  HIP_TRY(launch_wgrad_bf16(b, stream), "balance loss: input gradient");
  return MOE_OK;
}

}  // extern "C"
