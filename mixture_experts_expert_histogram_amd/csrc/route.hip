// Routing permutation (expert histogram, prefix scan, stable counting sort),
// the deterministic per-token combine, and the routing-weight gradient reduce.
//
// The pages ("Sparse expert dispatch and combine", "MoE training token repeat
// and expert computation", descriptions) select each expert's tokens by masked
// indexing and scatter the weighted expert outputs back with index_add_.
// Here the selection is one stable counting sort of the T*K slots by expert
// id, and the scatter is replaced by a gather: every token sums its own K
// expert rows in fp32, in k order, so no two threads ever write one element
// and no float atomics are used.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Pass 1: per-chunk expert histogram.  Integer LDS atomics are exact, so the
// counts do not depend on their order.
__global__ __launch_bounds__(ROUTE_THREADS) void route_hist_kernel(
    const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ blk_hist,
    int32_t* __restrict__ blk_bad) {
  __shared__ int hist[MAX_E];
  __shared__ int bad;
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) hist[e] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int base = blockIdx.x * ROUTE_CHUNK;
  int my_bad = 0;
  for (int i = threadIdx.x; i < ROUTE_CHUNK; i += ROUTE_THREADS) {
    const int s = base + i;
    if (s < S) {
      const int e = ids[s];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
      else ++my_bad;
    }
  }
  if (my_bad) atomicAdd(&bad, my_bad);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) blk_hist[(size_t)blockIdx.x * E + e] = hist[e];
  if (threadIdx.x == 0) blk_bad[blockIdx.x] = bad;
}

// Exclusive scan over one value per thread of a 1024-thread block.
__device__ int block_exclusive_scan_1024(int v, int* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    int add = (t >= d) ? sh[t - d] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  int incl = sh[t];
  __syncthreads();
  return incl - v;
}

// Pass 2 (one workgroup): counts, offsets, per-chunk bases, M-tile tables,
// the bad-id flag, and the experts ordered by descending count.
__global__ __launch_bounds__(1024) void route_scan_kernel(int nblk, int E, int big_min, int small_bm,
                                                          int32_t* __restrict__ blk_hist,
                                                          int32_t* __restrict__ blk_bad,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_prefix,
                                                          int32_t* __restrict__ expert_order,
                                                          int32_t* __restrict__ status) {
  __shared__ int sh[1024];
  __shared__ int cnt[MAX_E];
  __shared__ int part[1024];   // [slice][expert]: per-slice sums, then their bases
  __shared__ int base[MAX_E];
  const int e = threadIdx.x;
  // The chunks are cut into `slices` contiguous ranges; thread t sums expert
  // t % E over range t / E, so all 1024 threads read the histogram at once.
  const int slices = max(1, min(1024 / E, nblk));
  const int per = (nblk + slices - 1) / slices;
  const int te = threadIdx.x % E, ts = threadIdx.x / E;
  const bool slice_thread = threadIdx.x < slices * E;
  const int b0 = ts * per, b1 = min(nblk, b0 + per);
  // The chunk loops load 16 entries before using any, so a thread waits for
  // one round trip per 16 chunks rather than per chunk (the sums are integer,
  // so the grouping changes nothing).
  constexpr int U = 16;
  if (slice_thread) {
    int sum = 0;
    int b = b0;
    for (; b + U <= b1; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = blk_hist[(size_t)(b + u) * E + te];
#pragma unroll
      for (int u = 0; u < U; ++u) sum += v[u];
    }
    for (; b < b1; ++b) sum += blk_hist[(size_t)b * E + te];
    part[threadIdx.x] = sum;
  }
  __syncthreads();
  int c = 0;
  if (e < E)
    for (int q = 0; q < slices; ++q) {   // exclusive scan of the expert's slice sums
      const int v = part[q * E + e];
      part[q * E + e] = c;
      c += v;
    }
  const int off = block_exclusive_scan_1024(c, sh);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    cnt[e] = c;
    base[e] = off;
    if (e == E - 1) offsets[E] = off + c;
  }
  __syncthreads();
  if (slice_thread) {   // per-chunk bases of the expert's slots, chunk by chunk
    int run = base[te] + part[threadIdx.x];
    int b = b0;
    for (; b + U <= b1; b += U) {
      int h[U];
#pragma unroll
      for (int u = 0; u < U; ++u) h[u] = blk_hist[(size_t)(b + u) * E + te];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        blk_hist[(size_t)(b + u) * E + te] = run;
        run += h[u];
      }
    }
    for (; b < b1; ++b) {
      const int h = blk_hist[(size_t)b * E + te];
      blk_hist[(size_t)b * E + te] = run;
      run += h;
    }
  }
  for (int j = 0; j < N_TILE_TABLES; ++j) {
    const int bm = tile_bm(j), set = tile_set(j);
    const bool in = set == 0 || (set == 1) == large_tile_expert(c, big_min, small_bm);
    const int nt = (e < E && in) ? (c + bm - 1) / bm : 0;
    const int p = block_exclusive_scan_1024(nt, sh);
    if (e < E) tile_prefix[j * (E + 1) + e] = p;
    if (e == E - 1) tile_prefix[j * (E + 1) + E] = p + nt;
  }
  __syncthreads();
  if (e < E) {
    int r = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const int c2 = cnt[e2];
      r += (c2 > c) || (c2 == c && e2 < e);
    }
    expert_order[r] = e;
  }
  // Slots with an id outside [0,E) go after every valid slot, chunk by chunk
  // in slot order, so positions [offsets[E], S) hold them and every position
  // names a real slot and token: blk_bad becomes each chunk's first position
  // (an exclusive scan over the chunks, 1024 at a time by the whole block).
  const int valid = base[E - 1] + cnt[E - 1];
  int run = valid;
  for (int c0 = 0; c0 < nblk; c0 += 1024) {
    const int b = c0 + threadIdx.x;
    const int h = b < nblk ? blk_bad[b] : 0;
    const int ex = block_exclusive_scan_1024(h, sh);
    const int tot = sh[1023];   // inclusive total of this group of chunks
    __syncthreads();            // read before the next group's scan writes sh
    if (b < nblk) blk_bad[b] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) status[0] = run - valid;
}

// Pass 3: stable scatter.  A chunk is walked in rounds of 256 consecutive
// slots; inside a wavefront, lanes holding the same expert id are grouped
// with ballots, and a lane's rank is the number of lower lanes in its group.
// Waves of one round are ordered by wave index, rounds by round index, chunks
// by the bases from pass 2 — so every expert receives its slots in
// ascending slot order.  Slots with a bad id are grouped the same way under
// the key E and fill the positions after the valid ones (inv_pos -1, routing
// weight 0, their own token), so every position in [0, S) is written once.
__global__ __launch_bounds__(ROUTE_THREADS) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int S, int K, int E,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ blk_bad_base,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ inv_pos, int32_t* __restrict__ tok_of_pos,
    float* __restrict__ w_of_pos) {
  constexpr int NW = ROUTE_THREADS / 64;
  __shared__ int running[MAX_E + 1];
  __shared__ int wcnt[NW][MAX_E + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e <= E; e += ROUTE_THREADS) {
    running[e] = e < E ? blk_base[(size_t)blockIdx.x * E + e] : blk_bad_base[blockIdx.x];
#pragma unroll
    for (int v = 0; v < NW; ++v) wcnt[v][e] = 0;
  }
  __syncthreads();
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < ROUTE_CHUNK / ROUTE_THREADS; ++r) {
    const int s = blockIdx.x * ROUTE_CHUNK + r * ROUTE_THREADS + tid;
    int e = -1;   // grouping key: the expert id, E for a bad id, -1 past the end
    if (s < S) {
      e = ids[s];
      if ((unsigned)e >= (unsigned)E) e = E;
    }
    uint64_t peers = 0;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {                       // wave-uniform loop over distinct keys
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int le = __shfl(e, leader);
      const uint64_t m = __ballot(e == le);
      if (e == le) peers = m;
      todo &= ~m;
    }
    const int rank = __popcll(peers & lower);
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int pos = running[e] + rank;
      for (int v = 0; v < wave; ++v) pos += wcnt[v][e];
      sorted_slot[pos] = s;
      tok_of_pos[pos] = s / K;
      const bool ok = e < E;
      inv_pos[s] = ok ? pos : -1;
      w_of_pos[pos] = (ok && w) ? w[s] : 0.f;
    }
    __syncthreads();
    for (int e2 = tid; e2 <= E; e2 += ROUTE_THREADS) {
      int add = 0;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        add += wcnt[v][e2];
        wcnt[v][e2] = 0;
      }
      running[e2] += add;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Router: for each token the K largest of its E logits (descending; equal
// logits in ascending expert id) and, as its routing weights, the softmax of
// those K logits, which is the softmax over all E logits renormalised over
// the K chosen.  One wavefront per token, spread over the whole chip: a lane
// holds logits lane, lane+64, ...; each of K rounds takes the wave-wide best
// (value, then lower id) of the logits not yet taken.  The histogram, scan
// and scatter then run on the ids as for given ids.  (Counting the histogram
// in this kernel instead ties each chunk's tokens to one workgroup, so with
// 2048-slot chunks a 4096-token batch ran on 8 CUs, ~150 us of dependent
// cross-lane reductions; spread out it is a few microseconds.)  A token whose
// remaining logits are all NaN gets id -1 in the slots left, which the
// histogram reports as a bad id.
namespace {
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}
}  // namespace

constexpr int LOGIT_SLOTS = MAX_E / 64;   // logits per lane

__global__ __launch_bounds__(256) void route_logits_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                           int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nj = (E + 63) >> 6;
  const float* row = logits + (long)t * E;
  float v[LOGIT_SLOTS];
  unsigned taken = 0;   // bit j: logit lane + 64 j is chosen or does not exist
#pragma unroll
  for (int j = 0; j < LOGIT_SLOTS; ++j) {
    const int e = lane + 64 * j;
    const bool ok = j < nj && e < E;
    v[j] = ok ? row[e] : 0.f;
    if (!ok) taken |= 1u << j;
  }
  float top_z = 0.f, mx = 0.f, denom = 0.f;
  int top_i = -1;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < LOGIT_SLOTS; ++j)
      if (!(taken >> j & 1u) && better(v[j], lane + 64 * j, bv, bi)) { bv = v[j]; bi = lane + 64 * j; }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d);
      const int oi = __shfl_xor(bi, d);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const bool found = bi < E;
    if (found && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (k == 0) mx = bv;
    // fp32 softmax of the chosen logits, summed in k order; lane k keeps round k
    const float z = found ? expf(bv - mx) : 0.f;
    denom += z;
    if (lane == k) { top_z = z; top_i = found ? bi : -1; }
  }
  if (lane < K) {
    const long s = (long)t * K + lane;
    ids[s] = top_i;
    w[s] = top_i >= 0 ? top_z / denom : 0.f;
  }
}

// d_logits[t, ids[t,k]] = w_k (g_k - sum_j w_j g_j), zero elsewhere: the
// derivative of the softmax over the K chosen logits (the choice itself is
// piecewise constant).  One wavefront per token, each lane owning logits
// lane, lane+64, ...; repeated ids of a token add their terms.
__global__ __launch_bounds__(256) void router_bwd_kernel(const int32_t* __restrict__ ids,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ dw, int T, int E, int K,
                                                         float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int32_t* ti = ids + (long)t * K;
  const float* tw = w + (long)t * K;
  const float* tg = dw + (long)t * K;
  float dot = 0.f;
  for (int k = 0; k < K; ++k) dot += tw[k] * tg[k];
  for (int e = lane; e < E; e += 64) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k)
      if (ti[k] == e) acc += tw[k] * (tg[k] - dot);
    d_logits[(long)t * E + e] = acc;
  }
}

hipError_t launch_router_bwd(const int32_t* ids, const float* w, const float* dw, int T, int E, int K,
                             float* d_logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  return run_kernel("router_bwd", stream, [&] {
    router_bwd_kernel<<<(T + 3) / 4, 256, 0, stream>>>(ids, w, dw, T, E, K, d_logits);
  });
}

hipError_t launch_route(const int32_t* ids, const float* w, int S, int K, int E, const RouteState& rs,
                        hipStream_t stream) {
  const int nblk = rs.nblk;
  hipError_t err = run_kernel("route_hist", stream, [&] {
    route_hist_kernel<<<nblk, ROUTE_THREADS, 0, stream>>>(ids, S, E, rs.blk_hist, rs.blk_bad);
  });
  if (err != hipSuccess) return err;
  err = run_kernel("route_scan", stream, [&] {
    route_scan_kernel<<<1, 1024, 0, stream>>>(nblk, E, rs.big_min, rs.small_bm, rs.blk_hist, rs.blk_bad, rs.counts,
                                              rs.offsets,
                                              rs.tile_prefix, rs.expert_order, rs.status);
  });
  if (err != hipSuccess) return err;
  return run_kernel("route_scatter", stream, [&] {
    route_scatter_kernel<<<nblk, ROUTE_THREADS, 0, stream>>>(ids, w, S, K, E, rs.blk_hist, rs.blk_bad,
                                                             rs.sorted_slot, rs.inv_pos, rs.tok_of_pos,
                                                             rs.w_of_pos);
  });
}

hipError_t launch_route_logits(const float* logits, int T, int K, int E, int32_t* ids, float* w,
                               const RouteState& rs, hipStream_t stream) {
  hipError_t err = run_kernel("route_logits", stream, [&] {
    route_logits_kernel<<<(T + 3) / 4, 256, 0, stream>>>(logits, T, E, K, ids, w);
  });
  if (err != hipSuccess) return err;
  return launch_route(ids, w, T * K, K, E, rs, stream);
}

// ---------------------------------------------------------------------------
// Combine: out[t] = sum_{k<K} Yp[inv_pos[t*K+k]] over fp32 rows, summed in k
// order, one rounding to the storage type.  One thread owns 16 bytes of one
// output row.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values rounded to bf16 (nearest, ties to even), low half first.
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Yp,
                                                      const int32_t* __restrict__ inv_pos, int T, int K,
                                                      int H, int chunks, void* __restrict__ out) {
  constexpr int V = OUT_BF16 ? 8 : 4;      // output elements per thread (16 bytes)
  const long total = (long)T * chunks;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (long)gridDim.x * blockDim.x) {
    const int t = (int)(idx / chunks);
    const int c = (int)(idx - (long)t * chunks);
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int p = inv_pos[(long)t * K + k];
      if (p < 0) continue;
      const float4* row = (const float4*)(Yp + (long)p * H + (long)c * V);
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const float4 v = row[q];
        acc[4 * q + 0] += v.x; acc[4 * q + 1] += v.y; acc[4 * q + 2] += v.z; acc[4 * q + 3] += v.w;
      }
    }
    uint4 o;
    if (OUT_BF16) {
      o.x = pack_bf16(acc[0], acc[1]);
      o.y = pack_bf16(acc[2], acc[3]);
      o.z = pack_bf16(acc[4 % V], acc[5 % V]);
      o.w = pack_bf16(acc[6 % V], acc[7 % V]);
    } else {
      o.x = __float_as_uint(acc[0]); o.y = __float_as_uint(acc[1]);
      o.z = __float_as_uint(acc[2 % V]); o.w = __float_as_uint(acc[3 % V]);
    }
    ((uint4*)out)[idx] = o;
  }
}

hipError_t launch_combine(int dtype, const float* Yp, const int32_t* inv_pos, int T, int K, int H, void* out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int chunks = dtype == 0 ? H / 8 : H / 4;
  const long total = (long)T * chunks;
  const long blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  return run_kernel("combine", stream, [&] {
    if (dtype == 0)
      combine_kernel<true><<<grid, 256, 0, stream>>>(Yp, inv_pos, T, K, H, chunks, out);
    else
      combine_kernel<false><<<grid, 256, 0, stream>>>(Yp, inv_pos, T, K, H, chunks, out);
  });
}

// ---------------------------------------------------------------------------
// dTopkW[s] = sum over column tiles of the partial <r, a> dot products, in
// tile order (deterministic).
__global__ __launch_bounds__(256) void topkw_reduce_kernel(const float* __restrict__ partials, int nparts,
                                                           const int32_t* __restrict__ inv_pos, int S,
                                                           float* __restrict__ dw) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int p = inv_pos[s];
  float a = 0.f;
  if (p >= 0) {
    // 8 partials loaded before they are added, in the same order
    const float* row = partials + (long)p * nparts;
    int j = 0;
    for (; j + 8 <= nparts; j += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = row[j + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) a += v[u];
    }
    for (; j < nparts; ++j) a += row[j];
  }
  dw[s] = a;
}

hipError_t launch_topkw_reduce(const float* partials, int nparts, const int32_t* inv_pos, int S, float* dw,
                               hipStream_t stream) {
  if (S == 0) return hipSuccess;
  return run_kernel("topkw_reduce", stream, [&] {
    topkw_reduce_kernel<<<(S + 255) / 256, 256, 0, stream>>>(partials, nparts, inv_pos, S, dw);
  });
}

// ---------------------------------------------------------------------------
// Gather token rows into expert-sorted order: dst[p] = src[tok_of_pos[p]].
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ src,
                                                          const int32_t* __restrict__ tok, int S, int chunks,
                                                          uint4* __restrict__ dst) {
  const long total = (long)S * chunks;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (long)gridDim.x * blockDim.x) {
    const int p = (int)(idx / chunks);
    const int c = (int)(idx - (long)p * chunks);
    const uint4 v = src[(long)tok[p] * chunks + c];   // token rows are read K times: the copies stream past L2
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)(dst + idx));
  }
}

hipError_t launch_gather_rows(const void* src, const int32_t* tok_of_pos, int S, size_t row_bytes, void* dst,
                              hipStream_t stream) {
  if (S == 0) return hipSuccess;
  const int chunks = (int)(row_bytes / 16);
  const long total = (long)S * chunks;
  const long blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  return run_kernel("gather_rows", stream, [&] {
    gather_rows_kernel<<<grid, 256, 0, stream>>>((const uint4*)src, tok_of_pos, S, chunks, (uint4*)dst);
  });
}

// ---------------------------------------------------------------------------
// Zero fill with vector stores (used instead of a memset so the calls stay
// capturable as plain kernel nodes).
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ p, long n16, uint8_t* __restrict__ tail,
                                                        int ntail) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (long)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// dst[i] = src[i] for n int32 values (a kernel, so the copy is a plain
// kernel node under graph capture).
__global__ __launch_bounds__(64) void copy_i32_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst,
                                                      int n) {
  for (int i = threadIdx.x; i < n; i += 64) dst[i] = src[i];
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  return run_kernel("copy_i32", stream, [&] { copy_i32_kernel<<<1, 64, 0, stream>>>(src, dst, n); });
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const long n16 = (long)(bytes / 16);
  const int ntail = (int)(bytes % 16);
  long g = (n16 + 255) / 256;
  const int grid = (int)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
  return run_kernel("fill_zero", stream, [&] {
    fill_zero_kernel<<<grid, 256, 0, stream>>>((uint4*)p, n16, (uint8_t*)p + n16 * 16, ntail);
  });
}

}  // namespace moe
