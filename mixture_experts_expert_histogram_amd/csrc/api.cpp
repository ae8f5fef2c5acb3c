// C ABI of the routed MoE expert computation: argument checks, workspace
// layout and the launch sequence of the forward and backward passes.
#include "../../include/moe.h"
#include "moe_internal.h"

#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

struct Dims {
  int64_t T, H, I, E, K, S;
  size_t esz;       // bytes per activation / weight element
  size_t gsz;       // bytes per weight-gradient element
  int nblk;         // routing chunks
  int nparts;       // dTopkW partials per slot
};

// Workspace carving.  The routing block comes first in both workspaces.
struct Layout {
  size_t status, counts, offsets, tile_prefix, expert_order, blk_hist, blk_bad;
  size_t sorted_slot, inv_pos, tok_of_pos, w_of_pos, route_end;
  // forward
  size_t f_a, f_y, f_end;
  // backward
  size_t b_xp, b_dyp, b_z, b_dz, b_aw, b_part, b_dx, b_end;
};

Layout make_layout(const Dims& d) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  L.status = take(4 * sizeof(int32_t));
  L.counts = take(d.E * sizeof(int32_t));
  L.offsets = take((d.E + 1) * sizeof(int32_t));
  L.tile_prefix = take(N_TILE_TABLES * (d.E + 1) * sizeof(int32_t));
  L.expert_order = take(d.E * sizeof(int32_t));
  L.blk_hist = take((size_t)d.nblk * d.E * sizeof(int32_t));
  L.blk_bad = take((size_t)d.nblk * sizeof(int32_t));
  L.sorted_slot = take(d.S * sizeof(int32_t));
  L.inv_pos = take(d.S * sizeof(int32_t));
  L.tok_of_pos = take(d.S * sizeof(int32_t));
  L.w_of_pos = take(d.S * sizeof(float));
  L.route_end = o;
  // hidden / d_out rows gathered into expert order
  const size_t perm_rows = (size_t)d.S * d.H * d.esz;
  L.f_a = take((size_t)d.S * d.I * d.esz);
  L.f_y = take((size_t)d.S * d.H * sizeof(float));
  L.f_end = o;
  o = L.route_end;
  L.b_xp = take(perm_rows);
  L.b_dyp = take(perm_rows);
  L.b_z = take((size_t)d.S * 2 * d.I * sizeof(float));
  L.b_dz = take((size_t)d.S * 2 * d.I * d.esz);
  L.b_aw = take((size_t)d.S * d.I * d.esz);
  L.b_part = take((size_t)d.S * d.nparts * sizeof(float));
  L.b_dx = take((size_t)d.S * d.H * sizeof(float));
  L.b_end = o;
  return L;
}

RouteState route_state(void* ws, const Layout& L, const Dims& d) {
  char* b = (char*)ws;
  RouteState rs;
  rs.status = (int32_t*)(b + L.status);
  rs.counts = (int32_t*)(b + L.counts);
  rs.offsets = (int32_t*)(b + L.offsets);
  rs.tile_prefix = (int32_t*)(b + L.tile_prefix);
  rs.expert_order = (int32_t*)(b + L.expert_order);
  rs.blk_hist = (int32_t*)(b + L.blk_hist);
  rs.blk_bad = (int32_t*)(b + L.blk_bad);
  rs.sorted_slot = (int32_t*)(b + L.sorted_slot);
  rs.inv_pos = (int32_t*)(b + L.inv_pos);
  rs.tok_of_pos = (int32_t*)(b + L.tok_of_pos);
  rs.w_of_pos = (float*)(b + L.w_of_pos);
  rs.nblk = d.nblk;
  rs.big_min = 0x7fffffff;   // no large-tile experts unless the GEMM problem allows them
  rs.small_bm = 128;
  return rs;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Bytes of the optional `saved` buffer: Z fp32 [S,2I] in expert-sorted order.
size_t saved_size(const Dims& d) { return (size_t)d.S * 2 * d.I * sizeof(float); }

// Shape and enum checks shared by every entry point.
moe_status_t check_desc(const moe_desc_t* desc, Dims* d) {
  if (!desc) return MOE_ERR_INVALID_ARG;
  if (desc->T < 0 || desc->K < 1 || desc->E < 1 || desc->H < 1 || desc->I < 1) return MOE_ERR_INVALID_ARG;
  if (desc->dtype != MOE_BF16 && desc->dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (desc->act != MOE_SWIGLU && desc->act != MOE_CLAMPED_GLU) return MOE_ERR_INVALID_ARG;
  if (desc->gu_layout != MOE_GU_CONCAT && desc->gu_layout != MOE_GU_INTERLEAVED) return MOE_ERR_INVALID_ARG;
  if (desc->grad_dtype != MOE_BF16 && desc->grad_dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (desc->act == MOE_CLAMPED_GLU && !(desc->clamp_limit > 0.f)) return MOE_ERR_INVALID_ARG;
  if (desc->H % 8 != 0 || desc->I % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (desc->E > MAX_E || desc->K > 64) return MOE_ERR_UNSUPPORTED;
  const int64_t S = desc->T * desc->K;
  if (S >= (int64_t(1) << 31) || desc->H >= (int64_t(1) << 30) || desc->I >= (int64_t(1) << 29))
    return MOE_ERR_UNSUPPORTED;
  if (S * 2 * desc->I >= (int64_t(1) << 40) || S * desc->H >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  d->T = desc->T; d->H = desc->H; d->I = desc->I; d->E = desc->E; d->K = desc->K; d->S = S;
  d->esz = desc->dtype == MOE_BF16 ? 2 : 4;
  d->gsz = desc->grad_dtype == MOE_BF16 ? 2 : 4;
  d->nblk = (int)((S + ROUTE_CHUNK - 1) / ROUTE_CHUNK);
  if (d->nblk < 1) d->nblk = 1;
  d->nparts = down_dgrad_nparts((int)desc->I);
  return MOE_OK;
}

GemmProblem problem(const moe_desc_t* desc, const Dims& d, const RouteState* rs) {
  GemmProblem pb;
  pb.dtype = desc->dtype == MOE_BF16 ? 0 : 1;
  pb.gdtype = desc->grad_dtype == MOE_BF16 ? 0 : 1;
  pb.act = desc->act == MOE_CLAMPED_GLU ? 1 : 0;
  pb.layout = desc->gu_layout == MOE_GU_INTERLEAVED ? 1 : 0;
  pb.limit = desc->clamp_limit;
  pb.alpha = desc->glu_alpha;
  pb.T = (int)d.T; pb.H = (int)d.H; pb.I = (int)d.I; pb.E = (int)d.E; pb.K = (int)d.K; pb.S = (int)d.S;
  pb.rs = rs;
  return pb;
}

#define HIP_TRY(x)                       \
  do {                                   \
    if ((x) != hipSuccess) {             \
      (void)hipGetLastError();           \
      return MOE_ERR_HIP;                \
    }                                    \
  } while (0)

// ------------------------------------------------------------------ timing
struct TimingPool {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> ev;        // pairs
  std::vector<std::string> names;    // one per used pair
  int used = 0;
};
TimingPool& pool() {
  static TimingPool p;
  return p;
}

}  // namespace

namespace moe {
int timing_begin(const char* name, hipStream_t stream) {
  TimingPool& p = pool();
  if (!p.enabled) return -1;
  std::lock_guard<std::mutex> g(p.mu);
  if (p.used * 2 + 1 >= (int)p.ev.size()) return -1;
  const int slot = p.used++;
  p.names[slot] = name;
  if (hipEventRecord(p.ev[2 * slot], stream) != hipSuccess) return -1;
  return slot;
}
void timing_end(int slot, hipStream_t stream) {
  if (slot < 0) return;
  TimingPool& p = pool();
  (void)hipEventRecord(p.ev[2 * slot + 1], stream);
}
}  // namespace moe

extern "C" {

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_BAD_EXPERT_ID: return "MOE_ERR_BAD_EXPERT_ID";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status_t moe_route_workspace_size(const moe_desc_t* desc, size_t* route_ws) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (!route_ws) return MOE_ERR_INVALID_ARG;
  *route_ws = make_layout(d).route_end;
  return MOE_OK;
}

moe_status_t moe_workspace_size(const moe_desc_t* desc, size_t* fwd_ws, size_t* bwd_ws, size_t* saved_bytes) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  const Layout L = make_layout(d);
  if (fwd_ws) *fwd_ws = L.f_end;
  if (bwd_ws) *bwd_ws = L.b_end;
  if (saved_bytes) *saved_bytes = saved_size(d);
  return MOE_OK;
}

moe_status_t moe_route(const moe_desc_t* desc, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_slot, int32_t* inv_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (!ws || (d.S > 0 && !topk_ids)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(d);
  if (ws_bytes < L.route_end) return MOE_ERR_WORKSPACE;
  RouteState rs = route_state(ws, L, d);
  HIP_TRY(launch_route(topk_ids, nullptr, (int)d.S, (int)d.K, (int)d.E, rs, stream));
  if (counts) HIP_TRY(hipMemcpyAsync(counts, rs.counts, d.E * 4, hipMemcpyDeviceToDevice, stream));
  if (offsets) HIP_TRY(hipMemcpyAsync(offsets, rs.offsets, (d.E + 1) * 4, hipMemcpyDeviceToDevice, stream));
  if (sorted_slot && d.S)
    HIP_TRY(hipMemcpyAsync(sorted_slot, rs.sorted_slot, d.S * 4, hipMemcpyDeviceToDevice, stream));
  if (inv_pos && d.S) HIP_TRY(hipMemcpyAsync(inv_pos, rs.inv_pos, d.S * 4, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

moe_status_t moe_router(const moe_desc_t* desc, const float* logits, int32_t* topk_ids, float* topk_weights,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* inv_pos, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (d.K > d.E || !ws) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {logits, topk_ids, topk_weights, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(d);
  if (ws_bytes < L.route_end) return MOE_ERR_WORKSPACE;
  RouteState rs = route_state(ws, L, d);
  if (d.T == 0) {
    HIP_TRY(launch_fill_zero((char*)ws + L.status, 4 * sizeof(int32_t), stream));
  } else {
    HIP_TRY(launch_route_logits(logits, (int)d.T, (int)d.K, (int)d.E, topk_ids, topk_weights, rs, stream));
  }
  if (counts) {
    if (d.T == 0) HIP_TRY(launch_fill_zero(counts, d.E * 4, stream));
    else HIP_TRY(hipMemcpyAsync(counts, rs.counts, d.E * 4, hipMemcpyDeviceToDevice, stream));
  }
  if (offsets) {
    if (d.T == 0) HIP_TRY(launch_fill_zero(offsets, (d.E + 1) * 4, stream));
    else HIP_TRY(hipMemcpyAsync(offsets, rs.offsets, (d.E + 1) * 4, hipMemcpyDeviceToDevice, stream));
  }
  if (sorted_slot && d.S)
    HIP_TRY(hipMemcpyAsync(sorted_slot, rs.sorted_slot, d.S * 4, hipMemcpyDeviceToDevice, stream));
  if (inv_pos && d.S) HIP_TRY(hipMemcpyAsync(inv_pos, rs.inv_pos, d.S * 4, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

moe_status_t moe_router_bwd(const moe_desc_t* desc, const int32_t* topk_ids, const float* topk_weights,
                            const float* d_topk_weights, float* d_logits, hipStream_t stream) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (d.T > 0 && (!topk_ids || !topk_weights || !d_topk_weights || !d_logits)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {topk_ids, topk_weights, d_topk_weights, d_logits};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  HIP_TRY(launch_router_bwd(topk_ids, topk_weights, d_topk_weights, (int)d.T, (int)d.E, (int)d.K, d_logits,
                            stream));
  return MOE_OK;
}

static moe_status_t fwd_impl(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                             const float* topk_weights, const float* logits, int32_t* ids_out, float* w_out,
                             const void* w_gate_up, const void* w_up, const void* w_down, void* out, void* saved,
                             size_t saved_bytes, void* ws, size_t ws_bytes, hipStream_t stream);

moe_status_t moe_fwd(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                     const float* topk_weights, const void* w_gate_up, const void* w_down, void* out, void* saved,
                     size_t saved_bytes, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (desc && desc->T > 0 && (!topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  return fwd_impl(desc, hidden, topk_ids, topk_weights, nullptr, nullptr, nullptr, w_gate_up, nullptr, w_down, out,
                  saved, saved_bytes, ws, ws_bytes, stream);
}

moe_status_t moe_fwd_sep(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                         const float* topk_weights, const void* w_gate, const void* w_up, const void* w_down,
                         void* out, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (desc && desc->T > 0 && (!topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  if (!w_up) return MOE_ERR_INVALID_ARG;
  return fwd_impl(desc, hidden, topk_ids, topk_weights, nullptr, nullptr, nullptr, w_gate, w_up, w_down, out, saved,
                  saved_bytes, ws, ws_bytes, stream);
}

moe_status_t moe_fwd_logits(const moe_desc_t* desc, const void* hidden, const float* logits,
                            const void* w_gate_up, const void* w_down, void* out, int32_t* topk_ids,
                            float* topk_weights, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (desc && desc->T > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  if (desc && desc->K > desc->E) return MOE_ERR_INVALID_ARG;
  return fwd_impl(desc, hidden, topk_ids, topk_weights, logits, topk_ids, topk_weights, w_gate_up, nullptr, w_down,
                  out, saved, saved_bytes, ws, ws_bytes, stream);
}

// Forward from given ids and weights (logits == NULL) or from router logits
// (ids_out / w_out receive the router's choice); w_up != NULL: w_gate_up is
// the gate tensor [E,I,H] and w_up the up tensor.
static moe_status_t fwd_impl(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                             const float* topk_weights, const float* logits, int32_t* ids_out, float* w_out,
                             const void* w_gate_up, const void* w_up, const void* w_down, void* out, void* saved,
                             size_t saved_bytes, void* ws, size_t ws_bytes, hipStream_t stream) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (!w_gate_up || !w_down || !ws) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!hidden || !topk_ids || !topk_weights || !out)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {hidden, topk_ids, topk_weights, logits, w_gate_up, w_up, w_down, out, saved, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(d);
  if (ws_bytes < L.f_end) return MOE_ERR_WORKSPACE;
  if (saved && saved_bytes < saved_size(d)) return MOE_ERR_WORKSPACE;
  if (d.T == 0) {   // nothing to route: clear the status word so it reports this call
    HIP_TRY(launch_fill_zero((char*)ws + L.status, 4 * sizeof(int32_t), stream));
    return MOE_OK;
  }
  RouteState rs = route_state(ws, L, d);
  GemmProblem pb = problem(desc, d, &rs);
  if (w_up) {
    pb.w_up = w_up;
    pb.layout = 0;   // Z columns: gate then up
  }
  rs.big_min = large_tile_min_slots(pb);
  rs.small_bm = small_tile_rows(pb);
  char* b = (char*)ws;
  void* a = b + L.f_a;
  float* yp = (float*)(b + L.f_y);
  if (logits)
    HIP_TRY(launch_route_logits(logits, (int)d.T, (int)d.K, (int)d.E, ids_out, w_out, rs, stream));
  else
    HIP_TRY(launch_route(topk_ids, topk_weights, (int)d.S, (int)d.K, (int)d.E, rs, stream));
  HIP_TRY(launch_gate_up(pb, hidden, w_gate_up, a, saved, stream));
  HIP_TRY(launch_down(pb, a, w_down, yp, stream));
  HIP_TRY(launch_combine(pb.dtype, yp, rs.inv_pos, (int)d.T, (int)d.K, (int)d.H, out, stream));
  return MOE_OK;
}

// Backward; w_up != NULL: w_gate_up / d_w_gate_up are the gate tensors
// [E,I,H] and w_up / d_w_up the up tensors.
static moe_status_t bwd_impl(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                             const float* topk_weights, const void* w_gate_up, const void* w_up, const void* w_down,
                             const void* d_out, const void* saved, size_t saved_bytes, void* d_hidden,
                             float* d_topk_weights, void* d_w_gate_up, void* d_w_up, void* d_w_down, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (!w_gate_up || !w_down || !d_w_gate_up || !d_w_down || !ws) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!hidden || !topk_ids || !topk_weights || !d_out || !d_hidden || !d_topk_weights))
    return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {hidden, topk_ids, topk_weights, w_gate_up, w_up, w_down, d_out, saved,
                        d_hidden, d_topk_weights, d_w_gate_up, d_w_up, d_w_down, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(d);
  if (ws_bytes < L.b_end) return MOE_ERR_WORKSPACE;
  if (saved && saved_bytes < saved_size(d)) return MOE_ERR_WORKSPACE;
  if (d.T == 0) {   // no slots: zero weight gradients, and a status word that reports this call
    HIP_TRY(launch_fill_zero((char*)ws + L.status, 4 * sizeof(int32_t), stream));
    if (w_up) {
      HIP_TRY(launch_fill_zero(d_w_gate_up, (size_t)d.E * d.I * d.H * d.gsz, stream));
      HIP_TRY(launch_fill_zero(d_w_up, (size_t)d.E * d.I * d.H * d.gsz, stream));
    } else {
      HIP_TRY(launch_fill_zero(d_w_gate_up, (size_t)d.E * 2 * d.I * d.H * d.gsz, stream));
    }
    HIP_TRY(launch_fill_zero(d_w_down, (size_t)d.E * d.H * d.I * d.gsz, stream));
    return MOE_OK;
  }
  RouteState rs = route_state(ws, L, d);
  GemmProblem pb = problem(desc, d, &rs);
  if (w_up) {
    pb.w_up = w_up;
    pb.dw_up = d_w_up;
    pb.layout = 0;   // Z and dZ columns: gate then up
  }
  rs.big_min = large_tile_min_slots(pb);
  rs.small_bm = small_tile_rows(pb);
  char* b = (char*)ws;
  void* z = b + L.b_z;
  void* dz = b + L.b_dz;
  void* aw = b + L.b_aw;
  float* part = (float*)(b + L.b_part);
  float* dx = (float*)(b + L.b_dx);
  HIP_TRY(launch_route(topk_ids, topk_weights, (int)d.S, (int)d.K, (int)d.E, rs, stream));
  const void* zsrc = saved;
  int nparts = 0;
  void* xp = b + L.b_xp;
  void* dyp = b + L.b_dyp;
  HIP_TRY(launch_gather_rows(hidden, rs.tok_of_pos, (int)d.S, d.H * d.esz, xp, stream));
  HIP_TRY(launch_gather_rows(d_out, rs.tok_of_pos, (int)d.S, d.H * d.esz, dyp, stream));
  if (!zsrc) {
    HIP_TRY(launch_gate_up(pb, hidden, w_gate_up, nullptr, z, stream));
    zsrc = z;
  }
  HIP_TRY(launch_down_dgrad(pb, dyp, w_down, zsrc, dz, aw, part, &nparts, stream));
  HIP_TRY(launch_topkw_reduce(part, nparts, rs.inv_pos, (int)d.S, d_topk_weights, stream));
  HIP_TRY(launch_gate_up_dgrad(pb, dz, w_gate_up, dx, stream));
  HIP_TRY(launch_combine(pb.dtype, dx, rs.inv_pos, (int)d.T, (int)d.K, (int)d.H, d_hidden, stream));
  HIP_TRY(launch_wgrad_down(pb, dyp, aw, d_w_down, stream));
  HIP_TRY(launch_wgrad_gate_up(pb, dz, xp, d_w_gate_up, stream));
  return MOE_OK;
}

moe_status_t moe_bwd(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                     const float* topk_weights, const void* w_gate_up, const void* w_down, const void* d_out,
                     const void* saved, size_t saved_bytes, void* d_hidden, float* d_topk_weights,
                     void* d_w_gate_up, void* d_w_down, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(desc, hidden, topk_ids, topk_weights, w_gate_up, nullptr, w_down, d_out, saved, saved_bytes,
                  d_hidden, d_topk_weights, d_w_gate_up, nullptr, d_w_down, ws, ws_bytes, stream);
}

moe_status_t moe_bwd_sep(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                         const float* topk_weights, const void* w_gate, const void* w_up, const void* w_down,
                         const void* d_out, const void* saved, size_t saved_bytes, void* d_hidden,
                         float* d_topk_weights, void* d_w_gate, void* d_w_up, void* d_w_down, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (!w_up || !d_w_up) return MOE_ERR_INVALID_ARG;
  return bwd_impl(desc, hidden, topk_ids, topk_weights, w_gate, w_up, w_down, d_out, saved, saved_bytes, d_hidden,
                  d_topk_weights, d_w_gate, d_w_up, d_w_down, ws, ws_bytes, stream);
}

// ------------------------------------------------------------ no-allocation forward
// The workspace of moe_fwd_noalloc: one array per GPU, part of the library's
// code object, held until the process ends.  Host code never uses the name
// `scratch` as an address (on the host it is only a stand-in for the symbol);
// the device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and is what the kernels receive.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];

// Device address of the current device's scratch array, or null on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace

moe_status_t moe_fwd_noalloc(const moe_desc_t* desc, const void* hidden, const int32_t* topk_ids,
                             const float* topk_weights, const void* w_gate_up, const void* w_down, void* out,
                             void* saved, size_t saved_bytes, int32_t* bad_ids, hipStream_t stream) {
  Dims d;
  moe_status_t st = check_desc(desc, &d);
  if (st != MOE_OK) return st;
  if (d.T > 0 && (!topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  if (bad_ids && !aligned16(bad_ids)) return MOE_ERR_INVALID_ARG;
  // beyond the scratch array: rejected before any device call
  if (make_layout(d).f_end > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  st = fwd_impl(desc, hidden, topk_ids, topk_weights, nullptr, nullptr, nullptr, w_gate_up, nullptr, w_down, out,
                saved, saved_bytes, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
  if (st != MOE_OK || !bad_ids) return st;
  HIP_TRY(launch_copy_i32((const int32_t*)ws, bad_ids, 1, stream));   // the routing status word
  return MOE_OK;
}

moe_status_t moe_check_device_status(const void* ws, hipStream_t stream) {
  if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  int32_t bad = 0;
  HIP_TRY(hipMemcpyAsync(&bad, ws, sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  return bad ? MOE_ERR_BAD_EXPERT_ID : MOE_OK;
}

moe_status_t moe_timing_enable(int32_t max_launches) {
  if (max_launches < 1) return MOE_ERR_INVALID_ARG;
  TimingPool& p = pool();
  std::lock_guard<std::mutex> g(p.mu);
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.assign(2 * (size_t)max_launches, nullptr);
  p.names.assign(max_launches, std::string());
  for (auto& e : p.ev) HIP_TRY(hipEventCreate(&e));
  p.used = 0;
  p.enabled = true;
  return MOE_OK;
}

moe_status_t moe_timing_disable(void) {
  TimingPool& p = pool();
  std::lock_guard<std::mutex> g(p.mu);
  p.enabled = false;
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.names.clear();
  p.used = 0;
  return MOE_OK;
}

moe_status_t moe_timing_read(moe_kernel_time_t* out, int32_t max_entries, int32_t* n_entries) {
  if (!n_entries || (max_entries > 0 && !out)) return MOE_ERR_INVALID_ARG;
  TimingPool& p = pool();
  std::lock_guard<std::mutex> g(p.mu);
  std::vector<moe_kernel_time_t> acc;
  for (int i = 0; i < p.used; ++i) {
    HIP_TRY(hipEventSynchronize(p.ev[2 * i + 1]));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]));
    size_t j = 0;
    for (; j < acc.size(); ++j)
      if (p.names[i] == acc[j].name) break;
    if (j == acc.size()) {
      moe_kernel_time_t t;
      memset(&t, 0, sizeof(t));
      strncpy(t.name, p.names[i].c_str(), sizeof(t.name) - 1);
      acc.push_back(t);
    }
    acc[j].launches += 1;
    acc[j].total_ms += ms;
  }
  p.used = 0;
  *n_entries = (int32_t)acc.size();
  for (int i = 0; i < (int)acc.size() && i < max_entries; ++i) out[i] = acc[i];
  return MOE_OK;
}

}  // extern "C"
