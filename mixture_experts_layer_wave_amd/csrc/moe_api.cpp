// moe_api.cpp: the C ABI of include/moe.h. Validates every argument on the host, then
// enqueues the gfx950 kernels on the caller's stream. Allocates nothing.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

// Size/enum validation shared by every entry point.
int check_desc(const moe_desc* d) {
  if (!d) return MOE_E_INVAL;
  if (d->N < 1 || d->D < 1 || d->F < 1 || d->E < 1 || d->k < 1 || d->k > d->E) return MOE_E_INVAL;
  if (d->dtype != MOE_DT_F32 && d->dtype != MOE_DT_BF16) return MOE_E_INVAL;
  if (d->routing_mode != MOE_ROUTE_SOFTMAX_TOPK && d->routing_mode != MOE_ROUTE_TOPK_SOFTMAX) return MOE_E_INVAL;
  if (d->second_choice < MOE_SECOND_TOPK || d->second_choice > MOE_SECOND_NOISY_ALL) return MOE_E_INVAL;
  if (d->capacity_priority != MOE_PRIO_SLOT_MAJOR && d->capacity_priority != MOE_PRIO_TOKEN_MAJOR) return MOE_E_INVAL;
  if (d->capacity_formula != MOE_CAPF_TOKENS_K && d->capacity_formula != MOE_CAPF_TOKENS) return MOE_E_INVAL;
  if (d->activation < MOE_ACT_SILU || d->activation > MOE_ACT_GELU_TANH) return MOE_E_INVAL;
  if (d->capacity_mode != MOE_CAP_NONE && d->capacity_mode != MOE_CAP_PADDED) return MOE_E_INVAL;
  if (d->capacity_mode == MOE_CAP_PADDED && (!(d->capacity_factor > 0.0) || d->min_capacity < 0)) return MOE_E_INVAL;
  if (d->E > kMaxE || d->k > kMaxK) return MOE_E_UNSUPPORTED;
  if (d->D % 128 != 0 || d->F % 128 != 0) return MOE_E_UNSUPPORTED;
  if (d->D > (1 << 20) || d->F > (1 << 20)) return MOE_E_UNSUPPORTED;
  if (d->N * (int64_t)d->k > INT32_MAX) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

int capacity_of(const moe_desc* d, int64_t* C) {
  if (d->capacity_mode == MOE_CAP_NONE) { *C = d->N; return MOE_OK; }
  const double c = d->capacity_formula == MOE_CAPF_TOKENS
                       ? ceil(((double)d->N / (double)d->E) * d->capacity_factor)
                       : ceil(((d->capacity_factor * (double)d->N) * (double)d->k) / (double)d->E);
  if (!(c < 4.0e18)) return MOE_E_UNSUPPORTED;
  int64_t ci = (int64_t)c;
  if (ci < d->min_capacity) ci = d->min_capacity;
  *C = ci;
  return MOE_OK;
}

int rows_of(const moe_desc* d, int64_t* rows) {
  int64_t C;
  int st = capacity_of(d, &C);
  if (st) return st;
  const int64_t r = d->capacity_mode == MOE_CAP_PADDED ? C * d->E : d->N * d->k;
  if (r > INT32_MAX) return MOE_E_UNSUPPORTED;
  *rows = r;
  return MOE_OK;
}

size_t esize(const moe_desc* d) { return d->dtype == MOE_DT_BF16 ? 2 : 4; }

moe_ws_layout layout_of(const moe_desc* d, int64_t rows) {
  moe_ws_layout L;
  const ScratchLayout s = scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16);
  const size_t nk = (size_t)d->N * d->k;
  size_t o = 0;
  L.scratch = o; o = align_up(o + s.total, 256);
  L.topk_idx = o; o = align_up(o + 4 * nk, 256);
  L.topk_gate = o; o = align_up(o + 4 * nk, 256);
  L.load = o; o = align_up(o + 4 * (size_t)d->E, 256);
  L.counts = o; o = align_up(o + 4 * (size_t)d->E, 256);
  L.offsets = o; o = align_up(o + 4 * ((size_t)d->E + 1), 256);
  L.row_of = o; o = align_up(o + 4 * nk, 256);
  L.dropped = o; o = align_up(o + nk, 256);
  L.gate_eff = o; o = align_up(o + 4 * nk, 256);
  L.token_of_row = o; o = align_up(o + 4 * (size_t)rows, 256);
  L.x_perm = o; o = align_up(o + esize(d) * (size_t)rows * d->D, 256);
  L.h = o; o = align_up(o + esize(d) * (size_t)rows * d->F, 256);
  L.y_perm = o; o = align_up(o + esize(d) * (size_t)rows * d->D, 256);
  L.total = o;
  return L;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off); }

// ---- step bodies (arguments already validated) ----------------------------------------

RouterArgs router_args(const moe_desc* d, const void* x, const float* w_r, const float* bias, const float* noise,
                       const float* logits_in, float* logits_out, float* probs_out, int32_t* idx, float* gate,
                       void* scratch) {
  RouterArgs a{};
  a.x = x; a.w_r = w_r; a.bias = bias;
  a.noise = d->second_choice != MOE_SECOND_TOPK ? noise : nullptr;
  a.logits_in = logits_in; a.logits_out = logits_out; a.probs_out = probs_out;
  a.topk_idx = idx; a.topk_gate = gate;
  if (scratch) {
    const ScratchLayout s = scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16);
    a.psum = at<float>(scratch, s.psum);
    a.psum_magic = at<uint32_t>(scratch, s.header + 64);
    if (d->dtype == MOE_DT_BF16) a.rpart = at<float>(scratch, s.rpart);
  }
  a.N = d->N; a.D = (int)d->D; a.E = d->E; a.k = d->k;
  a.mode = d->routing_mode; a.noisy = d->second_choice;
  return a;
}

int do_route(const moe_desc* d, const void* x, const float* w_r, const float* bias, const float* noise,
             const float* logits_in, float* logits_out, float* probs_out, int32_t* idx, float* gate,
             void* scratch, hipStream_t st) {
  const RouterArgs a = router_args(d, x, w_r, bias, noise, logits_in, logits_out, probs_out, idx, gate, scratch);
  return status_of(launch_router(a, d->dtype == MOE_DT_BF16, st));
}

// Router of the forward pass followed by its dispatch. A batch of at most kDispatchTokens
// tokens with bf16 x (E <= 16, buffer of at most kSmallRows rows) takes two launches: the
// split-K logit kernel, then one kernel that finishes the routing and dispatches; or, for
// at most kTokRouterTokens tokens, the token-parallel router, then the one-launch dispatch.
int do_dispatch(const moe_desc* d, const void* x, const int32_t* idx, const float* gate, int32_t* load,
                int32_t* counts, int32_t* offsets, int32_t* row_of, uint8_t* dropped, float* gate_eff,
                int32_t* token_of_row, void* x_perm, void* scratch, hipStream_t st,
                const RouterArgs* route = nullptr, bool gather = true);

int do_route_dispatch(const moe_desc* d, const void* x, const float* w_r, const float* bias, const float* noise,
                      int32_t* idx, float* gate, int32_t* load, int32_t* counts, int32_t* offsets, int32_t* row_of,
                      uint8_t* dropped, float* gate_eff, int32_t* token_of_row, void* x_perm, void* scratch,
                      hipStream_t st, bool gather = true) {
  int64_t rows;
  int rc = rows_of(d, &rows);
  if (rc) return rc;
  const RouterArgs ra = router_args(d, x, w_r, bias, noise, nullptr, nullptr, nullptr, idx, gate, scratch);
  // (Batches the router takes token-parallel need one router launch already: then the
  // router and the one-launch dispatch.)
  const bool fused = d->dtype == MOE_DT_BF16 && d->N <= kDispatchTokens && rows <= kSmallRows && d->E <= 16 &&
                     d->D % kRouterChunk == 0 && ra.rpart != nullptr && !router_token_parallel(d->N, d->E);
  if (!fused) {
    rc = status_of(launch_router(ra, d->dtype == MOE_DT_BF16, st));
    if (rc) return rc;
    return do_dispatch(d, x, idx, gate, load, counts, offsets, row_of, dropped, gate_eff, token_of_row, x_perm,
                       scratch, st, nullptr, gather);
  }
  rc = status_of(launch_router_split(ra, st));
  if (rc) return rc;
  return do_dispatch(d, x, idx, gate, load, counts, offsets, row_of, dropped, gate_eff, token_of_row, x_perm, scratch,
                     st, &ra);
}

int do_dispatch(const moe_desc* d, const void* x, const int32_t* idx, const float* gate, int32_t* load,
                int32_t* counts, int32_t* offsets, int32_t* row_of, uint8_t* dropped, float* gate_eff,
                int32_t* token_of_row, void* x_perm, void* scratch, hipStream_t st, const RouterArgs* route,
                bool gather) {
  int64_t C, rows;
  int rc = capacity_of(d, &C);
  if (rc) return rc;
  rc = rows_of(d, &rows);
  if (rc) return rc;
  const ScratchLayout s = scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16);
  DispatchArgs a{};
  a.topk_idx = idx; a.topk_gate = gate;
  a.blockcnt = at<int32_t>(scratch, s.blockcnt);
  a.base = at<int32_t>(scratch, s.base);
  a.tokdrop = at<int32_t>(scratch, s.tokdrop);
  a.load_copy = at<int32_t>(scratch, s.load);
  a.load = load; a.counts = counts; a.offsets = offsets; a.row_of = row_of; a.dropped = dropped;
  a.gate_eff = gate_eff; a.token_of_row = token_of_row;
  a.N = d->N; a.E = d->E; a.k = d->k; a.nblk = s.nblk_d;
  a.token_major = d->capacity_priority == MOE_PRIO_TOKEN_MAJOR;
  const bool padded = d->capacity_mode == MOE_CAP_PADDED;
  a.C = padded ? C : -1;
  a.padded = padded;
  GatherArgs g{};
  g.x = x; g.token_of_row = token_of_row; g.counts = counts; g.x_perm = x_perm;
  g.rows = rows; g.N = d->N; g.D = (int)d->D; g.elem_bytes = (int)esize(d);
  g.C = padded ? C : -1; g.padded = padded;
  if (route != nullptr) return status_of(launch_route_dispatch_small(*route, a, g, st));
  if (d->N <= kDispatchTokens && rows <= kSmallRows) return status_of(launch_dispatch_small(a, g, st));
  hipError_t e = launch_dispatch(a, st);
  if (e != hipSuccess) return MOE_E_HIP;
  return gather ? status_of(launch_gather(g, st)) : MOE_OK;
}

// Column scales of int8 expert weights (all null: weights in the layer dtype).
struct Scales {
  const float* s1;
  const float* s2;
  const float* s3;
};

FfnArgs ffn_args(const moe_desc* d, int64_t C, int64_t rows, const void* x_perm, const int32_t* offsets,
                 const int32_t* counts, const void* w1, const void* w2, const void* w3, void* h, void* y_perm,
                 void* scratch, Scales sc, const int32_t* x_row_token = nullptr) {
  FfnArgs a{};
  a.x_row_token = x_row_token;
  a.s1 = sc.s1; a.s2 = sc.s2; a.s3 = sc.s3;
  if (d->dtype == MOE_DT_BF16) a.partial = at<float>(scratch, scratch_layout(d->N, d->D, d->E, d->k, true).partial);
  a.x_perm = x_perm; a.offsets = offsets; a.counts = counts; a.w1 = w1; a.w2 = w2; a.w3 = w3;
  a.h = h; a.y_perm = y_perm; a.rows = rows;
  a.max_rows_per_expert = d->capacity_mode == MOE_CAP_PADDED ? (C < d->N ? C : d->N) : d->N;
  a.D = (int)d->D; a.F = (int)d->F; a.E = d->E; a.act = d->activation;
  return a;
}

// which: 1 = up only, 2 = down only, 3 = both
// x_row_token non-null: x_perm is x and the up-projection gathers its rows from it.
int do_ffn(const moe_desc* d, const void* x_perm, const int32_t* offsets, const int32_t* counts, const void* w1,
           const void* w2, const void* w3, void* h, void* y_perm, void* scratch, int which, hipStream_t st,
           Scales sc = Scales{nullptr, nullptr, nullptr}, const int32_t* x_row_token = nullptr) {
  int64_t C, rows;
  int rc = capacity_of(d, &C);
  if (rc) return rc;
  rc = rows_of(d, &rows);
  if (rc) return rc;
  const FfnArgs a = ffn_args(d, C, rows, x_perm, offsets, counts, w1, w2, w3, h, y_perm, scratch, sc, x_row_token);
  const bool bf = d->dtype == MOE_DT_BF16;
  if (which & 1) {
    if (launch_expert_up(a, bf, st) != hipSuccess) return MOE_E_HIP;
  }
  if (which & 2) {
    if (launch_expert_down(a, bf, st) != hipSuccess) return MOE_E_HIP;
  }
  return MOE_OK;
}

int do_combine(const moe_desc* d, const void* y_perm, const int32_t* row_of, const float* gate_eff, void* y,
               hipStream_t st) {
  CombineArgs a{};
  a.y_perm = y_perm; a.row_of = row_of; a.gate_eff = gate_eff; a.y = y;
  int64_t rows;
  int rc = rows_of(d, &rows);
  if (rc) return rc;
  a.N = d->N; a.rows = rows; a.D = (int)d->D; a.k = d->k;
  return status_of(launch_combine(a, d->dtype == MOE_DT_BF16, st));
}

#define REQUIRE(p) do { if (!(p) || !aligned16(p)) return MOE_E_INVAL; } while (0)
#define OPTIONAL(p) do { if ((p) && !aligned16(p)) return MOE_E_INVAL; } while (0)

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_INVAL: return "MOE_E_INVAL: invalid argument";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED: valid but not supported by these kernels";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace or scratch missing or too small";
    case MOE_E_HIP: return "MOE_E_HIP: HIP runtime error";
    default: return "unknown moe status";
  }
}

int moe_capacity(const moe_desc* d, int64_t* capacity) {
  if (!d || !capacity) return MOE_E_INVAL;
  if (d->N < 1 || d->E < 1 || d->k < 1 || d->k > d->E) return MOE_E_INVAL;
  if (d->capacity_mode == MOE_CAP_PADDED && (!(d->capacity_factor > 0.0) || d->min_capacity < 0)) return MOE_E_INVAL;
  return capacity_of(d, capacity);
}

int moe_rows(const moe_desc* d, int64_t* rows) {
  if (!rows) return MOE_E_INVAL;
  int rc = check_desc(d);
  if (rc) return rc;
  return rows_of(d, rows);
}

int moe_scratch_size(const moe_desc* d, size_t* bytes) {
  if (!bytes) return MOE_E_INVAL;
  int rc = check_desc(d);
  if (rc) return rc;
  *bytes = scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total;
  return MOE_OK;
}

int moe_workspace_layout(const moe_desc* d, moe_ws_layout* layout) {
  if (!layout) return MOE_E_INVAL;
  int rc = check_desc(d);
  if (rc) return rc;
  int64_t rows;
  rc = rows_of(d, &rows);
  if (rc) return rc;
  *layout = layout_of(d, rows);
  return MOE_OK;
}

int moe_workspace_size(const moe_desc* d, size_t* bytes) {
  if (!bytes) return MOE_E_INVAL;
  moe_ws_layout L;
  int rc = moe_workspace_layout(d, &L);
  if (rc) return rc;
  *bytes = L.total;
  return MOE_OK;
}

int moe_route(const moe_desc* d, const void* x, const float* w_r, const float* logit_bias, const float* noise,
              const float* logits_in, float* logits_out, float* probs_out, int32_t* topk_idx, float* topk_gate,
              void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!logits_in) { REQUIRE(x); REQUIRE(w_r); OPTIONAL(logit_bias); } else { REQUIRE(logits_in); }
  if (d->second_choice != MOE_SECOND_TOPK) REQUIRE(noise);
  OPTIONAL(logits_out); OPTIONAL(probs_out);
  REQUIRE(topk_idx); REQUIRE(topk_gate);
  if (scratch) {
    OPTIONAL(scratch);
    if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total) return MOE_E_WORKSPACE;
  }
  return do_route(d, x, w_r, logit_bias, noise, logits_in, logits_out, probs_out, topk_idx, topk_gate, scratch,
                  (hipStream_t)stream);
}

int moe_dispatch(const moe_desc* d, const void* x, const int32_t* topk_idx, const float* topk_gate, int32_t* load,
                 int32_t* counts, int32_t* offsets, int32_t* row_of, uint8_t* dropped, float* gate_eff,
                 int32_t* token_of_row, void* x_perm, void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  int64_t rows;
  rc = rows_of(d, &rows);
  if (rc) return rc;
  REQUIRE(x); REQUIRE(topk_idx); REQUIRE(topk_gate); REQUIRE(load); REQUIRE(counts); REQUIRE(offsets);
  REQUIRE(row_of); REQUIRE(dropped); REQUIRE(gate_eff); REQUIRE(token_of_row); REQUIRE(x_perm);
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total) return MOE_E_WORKSPACE;
  return do_dispatch(d, x, topk_idx, topk_gate, load, counts, offsets, row_of, dropped, gate_eff, token_of_row,
                     x_perm, scratch, (hipStream_t)stream);
}

int moe_expert_ffn(const moe_desc* d, const void* x_perm, const int32_t* offsets, const int32_t* counts,
                   const void* w1, const void* w2, const void* w3, void* h, void* y_perm, void* scratch,
                   size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  REQUIRE(x_perm); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w1); REQUIRE(w2); REQUIRE(w3); REQUIRE(h);
  REQUIRE(y_perm);
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total) return MOE_E_WORKSPACE;
  return do_ffn(d, x_perm, offsets, counts, w1, w2, w3, h, y_perm, scratch, 3, (hipStream_t)stream);
}

int moe_expert_up(const moe_desc* d, const void* x_perm, const int32_t* offsets, const int32_t* counts,
                  const void* w1, const void* w2, void* h, void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  REQUIRE(x_perm); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w1); REQUIRE(w2); REQUIRE(h);
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total) return MOE_E_WORKSPACE;
  return do_ffn(d, x_perm, offsets, counts, w1, w2, nullptr, h, nullptr, scratch, 1, (hipStream_t)stream);
}

int moe_expert_up_gathered(const moe_desc* d, const void* x, const int32_t* token_of_row, const int32_t* offsets,
                           const int32_t* counts, const void* w1, const void* w2, void* h, void* scratch,
                           size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  REQUIRE(x); REQUIRE(token_of_row); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w1); REQUIRE(w2); REQUIRE(h);
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total) return MOE_E_WORKSPACE;
  int64_t C, rows;
  if ((rc = capacity_of(d, &C)) != MOE_OK || (rc = rows_of(d, &rows)) != MOE_OK) return rc;
  const bool bf = d->dtype == MOE_DT_BF16;
  if (!bf || !expert_up_gathers(ffn_args(d, C, rows, x, offsets, counts, w1, w2, nullptr, h, nullptr, scratch,
                                         Scales{nullptr, nullptr, nullptr}), bf))
    return MOE_E_UNSUPPORTED;
  return do_ffn(d, x, offsets, counts, w1, w2, nullptr, h, nullptr, scratch, 1, (hipStream_t)stream,
                Scales{nullptr, nullptr, nullptr}, token_of_row);
}

int moe_expert_down(const moe_desc* d, const void* h, const int32_t* offsets, const int32_t* counts,
                    const void* w3, void* y_perm, void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  REQUIRE(h); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w3); REQUIRE(y_perm);
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16).total) return MOE_E_WORKSPACE;
  return do_ffn(d, nullptr, offsets, counts, nullptr, nullptr, w3, const_cast<void*>(h), y_perm, scratch, 2,
                (hipStream_t)stream);
}

int moe_combine(const moe_desc* d, const void* y_perm, const int32_t* row_of, const float* gate_eff, void* y,
                void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  REQUIRE(y_perm); REQUIRE(row_of); REQUIRE(gate_eff); REQUIRE(y);
  return do_combine(d, y_perm, row_of, gate_eff, y, (hipStream_t)stream);
}

// Checks shared by the int8-weight entry points: bf16 activations, scales present.
static int check_q8(const moe_desc* d, const void* sa, const void* sb) {
  if (d->dtype != MOE_DT_BF16) return MOE_E_UNSUPPORTED;
  if (!sa || !aligned16(sa) || (sb != nullptr && !aligned16(sb))) return MOE_E_INVAL;
  return MOE_OK;
}

static int forward_impl(const moe_desc* d, const void* x, const float* w_r, const float* logit_bias,
                        const float* noise, const void* w1, const void* w2, const void* w3, void* y, void* workspace,
                        size_t workspace_bytes, void* stream, Scales sc);

int moe_forward(const moe_desc* d, const void* x, const float* w_r, const float* logit_bias, const float* noise,
                const void* w1, const void* w2, const void* w3, void* y, void* workspace, size_t workspace_bytes,
                void* stream) {
  return forward_impl(d, x, w_r, logit_bias, noise, w1, w2, w3, y, workspace, workspace_bytes, stream,
                      Scales{nullptr, nullptr, nullptr});
}

int moe_forward_q8(const moe_desc* d, const void* x, const float* w_r, const float* logit_bias, const float* noise,
                   const int8_t* w1, const float* s1, const int8_t* w2, const float* s2, const int8_t* w3,
                   const float* s3, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_q8(d, s1, s2)) != MOE_OK || (rc = check_q8(d, s3, nullptr)) != MOE_OK) return rc;
  return forward_impl(d, x, w_r, logit_bias, noise, w1, w2, w3, y, workspace, workspace_bytes, stream,
                      Scales{s1, s2, s3});
}

}  // extern "C"

// ---- the forward without a caller workspace ---------------------------------------------
// moe_forward_noalloc runs moe_forward with its workspace in one file-scope device array
// per GPU (allocated with the library's code object on that GPU, held until the process
// ends). Its host-side name is not a device address: the address is taken once per
// device, with that device current, by hipGetSymbolAddress and kept in g_noalloc_ws;
// kernels only ever receive that address.
namespace noalloc {
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WORKSPACE_BYTES];
}  // namespace noalloc

namespace {
constexpr int kNoallocDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ws[kNoallocDevices];  // per device; guarded by g_noalloc_mu

// Device address of the static workspace on device `dev` (the current device), or null
// if the runtime call fails.
void* noalloc_workspace(int dev) {
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ws[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_noalloc_ws[dev] = p;
  }
  return g_noalloc_ws[dev];
}
}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_desc* d, const void* x, const float* w_r, const float* logit_bias,
                        const float* noise, const void* w1, const void* w2, const void* w3, void* y, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  int64_t rows;
  rc = rows_of(d, &rows);
  if (rc) return rc;
  if (layout_of(d, rows).total > (size_t)MOE_NOALLOC_WORKSPACE_BYTES) return MOE_E_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
  if (dev < 0 || dev >= kNoallocDevices) return MOE_E_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sd) != hipSuccess) return MOE_E_HIP;
    if (sd != dev) return MOE_E_INVAL;  // the stream must belong to the current device
  }
  void* ws = noalloc_workspace(dev);
  if (ws == nullptr) return MOE_E_HIP;
  return forward_impl(d, x, w_r, logit_bias, noise, w1, w2, w3, y, ws, (size_t)MOE_NOALLOC_WORKSPACE_BYTES, stream,
                      Scales{nullptr, nullptr, nullptr});
}

int moe_expert_up_q8(const moe_desc* d, const void* x_perm, const int32_t* offsets, const int32_t* counts,
                     const int8_t* w1, const float* s1, const int8_t* w2, const float* s2, void* h, void* scratch,
                     size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_q8(d, s1, s2)) != MOE_OK) return rc;
  REQUIRE(x_perm); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w1); REQUIRE(w2); REQUIRE(h);
  if (!s2) return MOE_E_INVAL;
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, true).total) return MOE_E_WORKSPACE;
  return do_ffn(d, x_perm, offsets, counts, w1, w2, nullptr, h, nullptr, scratch, 1, (hipStream_t)stream,
                Scales{s1, s2, nullptr});
}

int moe_expert_down_q8(const moe_desc* d, const void* h, const int32_t* offsets, const int32_t* counts,
                       const int8_t* w3, const float* s3, void* y_perm, void* scratch, size_t scratch_bytes,
                       void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_q8(d, s3, nullptr)) != MOE_OK) return rc;
  REQUIRE(h); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w3); REQUIRE(y_perm);
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, true).total) return MOE_E_WORKSPACE;
  return do_ffn(d, nullptr, offsets, counts, nullptr, nullptr, w3, const_cast<void*>(h), y_perm, scratch, 2,
                (hipStream_t)stream, Scales{nullptr, nullptr, s3});
}

int moe_expert_ffn_q8(const moe_desc* d, const void* x_perm, const int32_t* offsets, const int32_t* counts,
                      const int8_t* w1, const float* s1, const int8_t* w2, const float* s2, const int8_t* w3,
                      const float* s3, void* h, void* y_perm, void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_q8(d, s1, s2)) != MOE_OK || (rc = check_q8(d, s3, nullptr)) != MOE_OK) return rc;
  REQUIRE(x_perm); REQUIRE(offsets); REQUIRE(counts); REQUIRE(w1); REQUIRE(w2); REQUIRE(w3); REQUIRE(h);
  REQUIRE(y_perm);
  if (!s2) return MOE_E_INVAL;
  if (!scratch || !aligned16(scratch)) return MOE_E_WORKSPACE;
  if (scratch_bytes < scratch_layout(d->N, d->D, d->E, d->k, true).total) return MOE_E_WORKSPACE;
  return do_ffn(d, x_perm, offsets, counts, w1, w2, w3, h, y_perm, scratch, 3, (hipStream_t)stream,
                Scales{s1, s2, s3});
}

static int forward_impl(const moe_desc* d, const void* x, const float* w_r, const float* logit_bias,
                        const float* noise, const void* w1, const void* w2, const void* w3, void* y, void* workspace,
                        size_t workspace_bytes, void* stream, Scales sc) {
  int rc = check_desc(d);
  if (rc) return rc;
  REQUIRE(x); REQUIRE(w_r); OPTIONAL(logit_bias); REQUIRE(w1); REQUIRE(w2); REQUIRE(w3); REQUIRE(y);
  if (d->second_choice != MOE_SECOND_TOPK) REQUIRE(noise);
  int64_t rows;
  rc = rows_of(d, &rows);
  if (rc) return rc;
  if (!workspace || !aligned16(workspace)) return MOE_E_WORKSPACE;
  const moe_ws_layout L = layout_of(d, rows);
  if (workspace_bytes < L.total) return MOE_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  // Beyond the single-launch dispatch of small batches, the up-projection reads the token
  // rows of x directly (through token_of_row) when it can, and x_perm is not materialised.
  int64_t C;
  rc = capacity_of(d, &C);
  if (rc) return rc;
  const bool small = d->N <= kDispatchTokens && rows <= kSmallRows;
  const bool gathered = !small && expert_up_gathers(ffn_args(d, C, rows, x, nullptr, nullptr, w1, w2, w3, nullptr,
                                                             nullptr, at<void>(ws, L.scratch), sc),
                                                    d->dtype == MOE_DT_BF16);
  rc = do_route_dispatch(d, x, w_r, logit_bias, noise, at<int32_t>(ws, L.topk_idx), at<float>(ws, L.topk_gate),
                         at<int32_t>(ws, L.load), at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                         at<int32_t>(ws, L.row_of), at<uint8_t>(ws, L.dropped), at<float>(ws, L.gate_eff),
                         at<int32_t>(ws, L.token_of_row), at<void>(ws, L.x_perm), at<void>(ws, L.scratch), st,
                         !gathered);
  if (rc) return rc;
  rc = do_ffn(d, gathered ? x : at<void>(ws, L.x_perm), at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.counts), w1,
              w2, w3, at<void>(ws, L.h), at<void>(ws, L.y_perm), at<void>(ws, L.scratch), 3, st, sc,
              gathered ? at<int32_t>(ws, L.token_of_row) : nullptr);
  if (rc) return rc;
  return do_combine(d, at<void>(ws, L.y_perm), at<int32_t>(ws, L.row_of), at<float>(ws, L.gate_eff), y, st);
}

int moe_read_stats(const moe_desc* d, const void* scratch, size_t scratch_bytes, moe_stats* out, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!out) return MOE_E_INVAL;
  const ScratchLayout s = scratch_layout(d->N, d->D, d->E, d->k, d->dtype == MOE_DT_BF16);
  if (!scratch || !aligned16(scratch) || scratch_bytes < s.total) return MOE_E_WORKSPACE;
  int64_t C;
  rc = capacity_of(d, &C);
  if (rc) return rc;
  void* sc = const_cast<void*>(scratch);
  StatsArgs a{};
  a.psum = at<float>(sc, s.psum);
  a.psum_magic = at<uint32_t>(sc, s.header + 64);
  a.probs = d->dtype == MOE_DT_BF16 ? at<float>(sc, s.rpart) : nullptr;
  a.load = at<int32_t>(sc, s.load);
  a.tokdrop = at<int32_t>(sc, s.tokdrop);
  a.out = at<void>(sc, s.header);
  a.N = d->N; a.C = d->capacity_mode == MOE_CAP_PADDED ? C : -1;
  a.E = d->E; a.k = d->k; a.nblk_r = s.nblk_r; a.nblk_d = s.nblk_d;
  hipStream_t st = (hipStream_t)stream;
  if (launch_stats(a, st) != hipSuccess) return MOE_E_HIP;
  if (hipMemcpyAsync(out, at<void>(sc, s.header), sizeof(moe_stats), hipMemcpyDeviceToHost, st) != hipSuccess)
    return MOE_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

}  // extern "C"
