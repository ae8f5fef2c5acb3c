// Internal declarations shared by the HIP translation units of the MoE library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

// Routing kernels process the slots in chunks of ROUTE_CHUNK per workgroup.
constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_CHUNK = 512;
constexpr int MAX_E = 1024;
// Tile prefix tables the routing scan writes, one per (M-tile height, set of
// experts): tables 0-4 cover every expert with 32, 64, 128, 256 and 192-row
// tiles; table 5 covers the large-tile experts (large_tile_expert) in
// 256-row tiles, tables 6 and 7 the others in 128 and 192-row tiles.
constexpr int N_TILE_TABLES = 8;
constexpr int TILE_BIG256 = 5, TILE_SMALL128 = 6, TILE_SMALL192 = 7;
__host__ __device__ constexpr int tile_bm(int j) {
  return j < 4 ? 32 << j : j == 4 ? 192 : j == TILE_BIG256 ? 256 : j == TILE_SMALL128 ? 128 : 192;
}
// 0: every expert, 1: the large-tile experts, 2: the others
__host__ __device__ constexpr int tile_set(int j) { return j < 5 ? 0 : j == TILE_BIG256 ? 1 : 2; }

// Whether an expert of c slots runs on the large-tile engine's 256-row tiles:
// from big_min slots on, and below that when its 256-row tiles hold no more
// rows than the small_bm-row tiles of the other engine would (with 128-row
// tiles 129-256 and 385-511 slots, with 192-row tiles 193-256 and 385-511):
// the same rows on the faster engine.  big_min = INT_MAX: none.
__host__ __device__ constexpr bool large_tile_expert(int c, int big_min, int small_bm) {
  return c >= big_min ||
         (big_min != 0x7fffffff && c > 0 && (c + 255) / 256 * 256 <= (c + small_bm - 1) / small_bm * small_bm);
}

// Device views of the routing state that lives in the workspace.
struct RouteState {
  int32_t* status;        // [4]  status[0] = number of slots with a bad id
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* tile_prefix;   // [N_TILE_TABLES][E+1]
  int32_t* expert_order;  // [E] experts by descending count (ties: lower id)
  int32_t* blk_hist;      // [nblk][E] (histogram, then per-block base)
  int32_t* blk_bad;       // [nblk]
  int32_t* sorted_slot;   // [S]
  int32_t* inv_pos;       // [S]
  int32_t* tok_of_pos;    // [S] token of the slot at each position
  float* w_of_pos;        // [S] routing weight of the slot at each position
  int nblk;
  int big_min;            // experts with at least this many slots use the large-tile engine
  int small_bm;           // M-tile rows of the other engine (128 or 192), for large_tile_expert
};

// Host side: optional timing events around each kernel launch (api.cpp).
int timing_begin(const char* name, hipStream_t stream);   // slot, or -1 when not timing
void timing_end(int slot, hipStream_t stream);

template <class F>
inline hipError_t run_kernel(const char* name, hipStream_t stream, F&& launch) {
  int slot = timing_begin(name, stream);
  launch();
  hipError_t e = hipGetLastError();
  timing_end(slot, stream);
  return e;
}

// ---- routing / combine / reduce (route.hip)
hipError_t launch_route(const int32_t* ids, const float* w, int S, int K, int E,
                        const RouteState& rs, hipStream_t stream);
// router: top-K of logits [T,E] and their softmax -> ids, w [T,K]; then as launch_route
hipError_t launch_route_logits(const float* logits, int T, int K, int E, int32_t* ids, float* w,
                               const RouteState& rs, hipStream_t stream);
// d_logits [T,E] from the routing-weight gradient through the softmax over the chosen K
hipError_t launch_router_bwd(const int32_t* ids, const float* w, const float* dw, int T, int E, int K,
                             float* d_logits, hipStream_t stream);
// out[t] = sum_k Yp[inv_pos[t*K+k]] from fp32 rows, stored in dtype
hipError_t launch_combine(int dtype, const float* Yp, const int32_t* inv_pos, int T, int K, int H,
                          void* out, hipStream_t stream);
hipError_t launch_topkw_reduce(const float* partials, int nparts, const int32_t* inv_pos, int S,
                               float* dw, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t stream);

// ---- grouped GEMMs (gemm.hip)
struct GemmProblem {
  int dtype;             // activations / weights: 0 bf16, 1 fp32
  int gdtype;            // weight gradients: 0 bf16, 1 fp32
  int act;               // 0 swiglu, 1 clamped
  int layout;            // 0 concat, 1 interleaved
  float limit, alpha;
  int T, H, I, E, K, S;
  const RouteState* rs;
  // separate gate and up weights: the launches' w_gate_up / d_w_gate_up
  // arguments are then the gate tensors [E,I,H] and these the up tensors
  // (layout is then the concatenated one for Z and dZ); null when fused
  const void* w_up = nullptr;
  void* dw_up = nullptr;
  // experts a token-row launch covers: 0 all, 1 the large-tile experts
  // (large_tile_expert), 2 the others
  int tile_set = 0;
};
// Per-slot buffers are indexed by the expert-sorted position p.
// forward gate_up projection + GLU: writes a [S,I] (dtype, if a_out) and Z fp32 [S,2I] (if z_out)
hipError_t launch_gate_up(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                          hipStream_t stream);
// forward down projection with routing weight: Yp fp32 [S,H]
hipError_t launch_down(const GemmProblem& pb, const void* a, const void* Wd, void* Yp, hipStream_t stream);
// backward: r = dYp.Wd (d_out rows gathered into expert order), GLU backward (Z fp32)
//   -> dZ [S,2I], aw = w*a [S,I], partials fp32 [S, nparts]
hipError_t launch_down_dgrad(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z,
                             void* dZ, void* aw, float* partials, int* nparts, hipStream_t stream);
int down_dgrad_nparts(int I);
// backward: dXp = dZ . Wgu, fp32 [S,H]
hipError_t launch_gate_up_dgrad(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp,
                                hipStream_t stream);
// backward weight gradients (dYp, Xp: d_out / hidden rows gathered into expert order)
hipError_t launch_wgrad_down(const GemmProblem& pb, const void* dY, const void* aw, void* dWd,
                             hipStream_t stream);
hipError_t launch_wgrad_gate_up(const GemmProblem& pb, const void* dZ, const void* X, void* dWgu,
                                hipStream_t stream);

// Experts with at least this many slots take the large-tile engine in every
// token-row GEMM of the problem (INT_MAX: none); set in the routing state
// before routing.
int large_tile_min_slots(const GemmProblem& pb);
// M-tile rows of the small-tile engine for the other experts (128 or 192).
int small_tile_rows(const GemmProblem& pb);

// rows dst[p] = src[tok_of_pos[p]] of width `row_bytes` (a multiple of 16)
hipError_t launch_gather_rows(const void* src, const int32_t* tok_of_pos, int S, size_t row_bytes, void* dst,
                              hipStream_t stream);

}  // namespace moe
