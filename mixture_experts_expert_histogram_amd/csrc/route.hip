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
__global__ __launch_bounds__(1024) void route_scan_kernel(int nblk, int E, int32_t* __restrict__ blk_hist,
                                                          const int32_t* __restrict__ blk_bad,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_prefix,
                                                          int32_t* __restrict__ expert_order,
                                                          int32_t* __restrict__ status) {
  __shared__ int sh[1024];
  __shared__ int cnt[MAX_E];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int b = 0; b < nblk; ++b) c += blk_hist[(size_t)b * E + e];
  const int off = block_exclusive_scan_1024(c, sh);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    cnt[e] = c;
    int run = off;
    for (int b = 0; b < nblk; ++b) {
      const int h = blk_hist[(size_t)b * E + e];
      blk_hist[(size_t)b * E + e] = run;
      run += h;
    }
    if (e == E - 1) offsets[E] = off + c;
  }
  for (int j = 0; j < N_TILE_BM; ++j) {
    const int bm = tile_bm(j);
    const int nt = (e < E) ? (c + bm - 1) / bm : 0;
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
  if (threadIdx.x == 0) {
    int bad = 0;
    for (int b = 0; b < nblk; ++b) bad += blk_bad[b];
    status[0] = bad;
  }
}

// Pass 3: stable scatter.  A chunk is walked in rounds of 256 consecutive
// slots; inside a wavefront, lanes holding the same expert id are grouped
// with ballots, and a lane's rank is the number of lower lanes in its group.
// Waves of one round are ordered by wave index, rounds by round index, chunks
// by the bases from pass 2 — so every expert receives its slots in
// ascending slot order.
__global__ __launch_bounds__(ROUTE_THREADS) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int S, int K, int E,
    const int32_t* __restrict__ blk_base, int32_t* __restrict__ sorted_slot, int32_t* __restrict__ inv_pos,
    int32_t* __restrict__ tok_of_pos, float* __restrict__ w_of_pos) {
  constexpr int NW = ROUTE_THREADS / 64;
  __shared__ int running[MAX_E];
  __shared__ int wcnt[NW][MAX_E];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += ROUTE_THREADS) {
    running[e] = blk_base[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int v = 0; v < NW; ++v) wcnt[v][e] = 0;
  }
  __syncthreads();
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < ROUTE_CHUNK / ROUTE_THREADS; ++r) {
    const int s = blockIdx.x * ROUTE_CHUNK + r * ROUTE_THREADS + tid;
    int e = -1;
    if (s < S) {
      e = ids[s];
      if ((unsigned)e >= (unsigned)E) {
        inv_pos[s] = -1;
        e = -1;
      }
    }
    uint64_t peers = 0;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {                       // wave-uniform loop over distinct ids
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
      inv_pos[s] = pos;
      tok_of_pos[pos] = s / K;
      w_of_pos[pos] = w ? w[s] : 0.f;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += ROUTE_THREADS) {
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

hipError_t launch_route(const int32_t* ids, const float* w, int S, int K, int E, const RouteState& rs,
                        hipStream_t stream) {
  const int nblk = rs.nblk;
  hipError_t err = run_kernel("route_hist", stream, [&] {
    route_hist_kernel<<<nblk, ROUTE_THREADS, 0, stream>>>(ids, S, E, rs.blk_hist, rs.blk_bad);
  });
  if (err != hipSuccess) return err;
  err = run_kernel("route_scan", stream, [&] {
    route_scan_kernel<<<1, 1024, 0, stream>>>(nblk, E, rs.blk_hist, rs.blk_bad, rs.counts, rs.offsets,
                                              rs.tile_prefix, rs.expert_order, rs.status);
  });
  if (err != hipSuccess) return err;
  return run_kernel("route_scatter", stream, [&] {
    route_scatter_kernel<<<nblk, ROUTE_THREADS, 0, stream>>>(ids, w, S, K, E, rs.blk_hist, rs.sorted_slot,
                                                             rs.inv_pos, rs.tok_of_pos, rs.w_of_pos);
  });
}

// ---------------------------------------------------------------------------
// Combine: out[t] = sum_{k<K} Yp[inv_pos[t*K+k]] over fp32 rows, summed in k
// order, one rounding to the storage type.  One thread owns 16 bytes of one
// output row.
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
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
      o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
      o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
      o.z = f32_to_bf16_bits(acc[4 % V]) | (f32_to_bf16_bits(acc[5 % V]) << 16);
      o.w = f32_to_bf16_bits(acc[6 % V]) | (f32_to_bf16_bits(acc[7 % V]) << 16);
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
  if (p >= 0)
    for (int j = 0; j < nparts; ++j) a += partials[(long)p * nparts + j];
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
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ src,
                                                          const int32_t* __restrict__ tok, int S, int chunks,
                                                          uint4* __restrict__ dst) {
  const long total = (long)S * chunks;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (long)gridDim.x * blockDim.x) {
    const int p = (int)(idx / chunks);
    const int c = (int)(idx - (long)p * chunks);
    dst[idx] = src[(long)tok[p] * chunks + c];
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
