// Shared pieces of the grouped GEMM kernels: vector types, bf16 packing, the
// gated activation and its derivative, the accumulator layout, the kernel
// arguments, token-row tile mapping and the fused epilogues of the
// token-row GEMMs (used by both GEMM engines).
#pragma once
#include <cstddef>
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ helpers
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values rounded to bf16 (nearest, ties to even) and packed, low
// half first: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
template <typename T> __device__ __forceinline__ void store_val(T* p, float v);
template <> __device__ __forceinline__ void store_val<uint16_t>(uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}
template <> __device__ __forceinline__ void store_val<float>(float* p, float v) { *p = v; }

// The logistic function through the hardware reciprocal (v_rcp_f32, about
// 1 ulp) rather than a correctly rounded division: every value it feeds is
// rounded to bf16 or summed in fp32 afterwards.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Gated activation (SwiGLU, ACT = 0, or the clamped GLU of the gpt-oss-shaped
// pages, ACT = 1), with the kind fixed at compile time.
template <int ACT>
__device__ __forceinline__ float glu_fwd_t(float g, float u, float L, float al) {
  if constexpr (ACT == 0) {
    return g * sigmoid_f(g) * u;
  } else {
    const float gc = __builtin_amdgcn_fmed3f(g, -__builtin_inff(), L);   // min(g, L)
    const float uc = __builtin_amdgcn_fmed3f(u, -L, L);
    return (uc + 1.f) * gc * sigmoid_f(al * gc);
  }
}
// Returns a = phi(g,u) and (dg, du) = phi'(g,u) * da.
template <int ACT>
__device__ __forceinline__ float glu_bwd_t(float g, float u, float da, float L, float al, float& dg, float& du) {
  if constexpr (ACT == 0) {
    const float s = sigmoid_f(g);
    const float silu = g * s;
    dg = da * u * s * (1.f + g * (1.f - s));
    du = da * silu;
    return silu * u;
  } else {
    const float gc = __builtin_amdgcn_fmed3f(g, -__builtin_inff(), L);   // min(g, L)
    const float uc = __builtin_amdgcn_fmed3f(u, -L, L);
    const float s = sigmoid_f(al * gc);
    const float q = gc * s;
    dg = (g <= L) ? da * (uc + 1.f) * s * (1.f + al * gc * (1.f - s)) : 0.f;
    du = (uc == u) ? da * q : 0.f;   // u inside [-L, L]
    return (uc + 1.f) * q;
  }
}
// The same with the kind chosen at run time (act = 0 or 1).
__device__ __forceinline__ float glu_fwd(float g, float u, int act, float L, float al) {
  return act == 0 ? glu_fwd_t<0>(g, u, L, al) : glu_fwd_t<1>(g, u, L, al);
}
__device__ __forceinline__ float glu_bwd(float g, float u, float da, int act, float L, float al, float& dg,
                                         float& du) {
  return act == 0 ? glu_bwd_t<0>(g, u, da, L, al, dg, du) : glu_bwd_t<1>(g, u, da, L, al, dg, du);
}

// The MFMA is issued with the B fragment first, so it computes the tile
// transposed: accumulator element (fm, fn, v) of a lane is output row
// wm*WTM + fm*32 + lane%32 and output column wn*WTN + fn*32 + acc_col4 + v%4,
// where acc_col4 = 8*(v/4) + 4*(lane/32).  A lane therefore holds 4
// consecutive columns of one row per register group, and stores are 16 (fp32)
// or 8 (bf16) bytes wide.
__device__ __forceinline__ int acc_col4(int vg, int lane) { return (vg << 3) + ((lane >> 5) << 2); }

template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2(pack_bf16(a, b), pack_bf16(c, d));
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
// interleaved pairs (g0 u0 g1 u1 g2 u2 g3 u3)
template <typename T> __device__ __forceinline__ void store4x2(T* p, const float* g, const float* u);
template <> __device__ __forceinline__ void store4x2<uint16_t>(uint16_t* p, const float* g, const float* u) {
  *(uint4*)p = make_uint4(pack_bf16(g[0], u[0]), pack_bf16(g[1], u[1]), pack_bf16(g[2], u[2]), pack_bf16(g[3], u[3]));
}
template <> __device__ __forceinline__ void store4x2<float>(float* p, const float* g, const float* u) {
  *(float4*)p = make_float4(g[0], u[0], g[1], u[1]);
  *(float4*)(p + 4) = make_float4(g[2], u[2], g[3], u[3]);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// ------------------------------------------------------------------ arguments
struct GArgs {
  const int32_t* offsets;
  const int32_t* tile_prefix;   // for this kernel's BM
  const int32_t* tok_of_pos;
  const float* w_of_pos;
  const int32_t* expert_order;
  const void* A;
  const void* B;
  const void* Z;
  void* out0;
  void* out1;
  float* partials;
  int T, H, I, E, K, S;
  int act, layout;
  float limit, alpha;
  int ntn, ntm, nparts;
  int big;   // weight grads: experts with more positions than this are split over the XCDs
  int small_max;   // weight grads: the tiled kernel takes only experts with more positions (-1: all)
  int hot_min;     // weight grads: experts with more positions go to the long-K kernel (0: none)
  // Gate/up rows of the weights (gu_*) and of their gradients (dgu_*): row j of
  // expert e's gate (up) projection starts gu_es*e + gu_rs*j elements after
  // gu_g (gu_u).  Fused [E,2I,H] concatenated: (W, W + I*H, 2IH, H);
  // interleaved: (W, W + H, 2IH, 2H); separate [E,I,H] tensors: (Wg, Wu, IH, H).
  const void* gu_g;
  const void* gu_u;
  void* dgu_g;
  void* dgu_u;
  long gu_es, gu_rs;
  int gu_sep;   // separate gate and up tensors (Z and dZ columns then concatenated)
};
// GArgs is passed by value as the kernel argument: the host and device passes
// of every source file must lay it out alike (no LDS pointers, which are
// 4 bytes on the device, and 8-byte pointers and longs on both sides).
static_assert(sizeof(void*) == 8 && sizeof(long) == 8, "64-bit pointers and longs on host and device");
static_assert(sizeof(GArgs) == 208 && offsetof(GArgs, T) == 88 && offsetof(GArgs, hot_min) == 148 &&
                  offsetof(GArgs, gu_g) == 152 && offsetof(GArgs, gu_es) == 184 && offsetof(GArgs, gu_sep) == 200,
              "kernel-argument layout");

// Row j of expert e's gate (up = 0) or up (up = 1) projection.
template <typename P>
__device__ __forceinline__ P* gu_row(P* g0, P* u0, long es, long rs, int e, int up, int j) {
  return (up ? u0 : g0) + es * e + rs * j;
}

// Gate/up half and index of column m of Z and dZ [S,2I] (interleaved:
// columns 2j, 2j+1; otherwise gate columns [0,I), up columns [I,2I)).
__device__ __forceinline__ void zcol(int m, int I, int layout, int& up, int& j) {
  up = layout ? (m & 1) : (m >= I);
  j = layout ? (m >> 1) : m - (up ? I : 0);
}

constexpr int kRowTileGroup = 8;

// Token-row tiles: (expert, N-tile, M-tile of BM rows), ordered by expert,
// then by groups of M-tiles, then N-tile, then M-tile, so the M-tiles of one
// expert that share a weight tile are neighbours.  row_tile_of decodes tile t
// of that order (t below the total, tile_prefix[E] * ntn).
template <int BM>
__device__ __forceinline__ void row_tile_of(const GArgs& g, int t, int& e, int& m0, int& rows, int& nt) {
  const int* tp = g.tile_prefix;
  const int ntn = g.ntn;
  const int q = t / ntn;
  int lo = 0, hi = g.E;            // largest e with tp[e] <= q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tp[mid] <= q) lo = mid; else hi = mid - 1;
  }
  e = lo;
  const int nm = tp[e + 1] - tp[e];
  // Inside an expert the M-tiles go in groups of kRowTileGroup; a group's
  // tiles run N-tile by N-tile, M-tile fastest.  The ~64 workgroups an XCD
  // holds at once then cover an 8x8 block of (M, N) tiles, each token-row
  // block and each weight tile read by 8 of them; N-tile-major order over a
  // whole hot expert re-streamed its token rows once per N-tile (Zipf
  // workload gate_up: 32.5 GB fetched per launch, 20.5 GB grouped).  Experts
  // with at most kRowTileGroup M-tiles keep the N-major order.
  const int local = t - tp[e] * ntn;
  const int gsz = kRowTileGroup * ntn;
  const int grp = local / gsz;
  const int rem = local - grp * gsz;
  const int gm = min(kRowTileGroup, nm - grp * kRowTileGroup);
  nt = rem / gm;
  const int mt = grp * kRowTileGroup + (rem - nt * gm);
  m0 = g.offsets[e] + mt * BM;
  rows = min(BM, g.offsets[e + 1] - m0);
}

// The grid of one workgroup per tile is sized for the worst case; the actual
// tile count is read from the routing tables and split into 8 equal
// contiguous ranges, one per XCD (hardware deals workgroup b to XCD b % 8).
// Returns false for a workgroup without a tile.
template <int BM>
__device__ __forceinline__ bool row_tile_at(const GArgs& g, int xcd, int j, int& e, int& m0, int& rows, int& nt) {
  const int total = g.tile_prefix[g.E] * g.ntn;
  const int per = (total + 7) >> 3;
  if (j >= per) return false;
  const int t = xcd * per + j;
  if (t >= total) return false;
  row_tile_of<BM>(g, t, e, m0, rows, nt);
  return true;
}

// The tile of this workgroup in a grid of one workgroup per tile (rounded up):
// workgroup b runs on XCD b % 8 and takes that XCD's (b / 8)-th tile.
template <int BM>
__device__ __forceinline__ bool row_tile(const GArgs& g, int& e, int& m0, int& rows, int& nt) {
  return row_tile_at<BM>(g, blockIdx.x & 7, blockIdx.x >> 3, e, m0, rows, nt);
}

// Weight-gradient tiles: chunks of CH consecutive tiles are dealt
// round-robin to the XCDs (experts longest first), so every XCD gets a
// similar share of long and short experts and a chunk's tiles share operands
// in one L2.  The j-th tile of this workgroup's XCD, or -1 past the end.
template <int CH>
__device__ __forceinline__ int dealt_tile(int j, int total) {
  const int x = blockIdx.x & 7;
  const int t = ((j / CH) * 8 + x) * CH + j % CH;
  return t < total ? t : -1;
}

// ------------------------------------------------------------------ epilogues
// The fused epilogues of the token-row GEMMs, for any tile configuration C
// (C::FM x C::FN fragments of 32 x 32 per wave, wave tile C::WTM x C::WTN).
// The MFMA is issued with the B fragment first, so accumulator element
// (fm, fn, v) of a lane is output row wm*WTM + fm*32 + lane%32 and column
// wn*WTN + fn*32 + acc_col4(v/4, lane) + v%4.

// gate_up: fragments fn = 2p and 2p+1 of a wave hold the gate and up values of
// the same 32 activation columns, (wn*FN/2 + p)*32 + 0..31 after j0.  Writes
// a = phi(g, u) (element type T, if WRITE_A) and Z fp32 [S,2I] (if WRITE_Z).
template <class C, typename T, bool WRITE_A, bool WRITE_Z>
__device__ __forceinline__ void epi_gate_up(const GArgs& g, f32x16 (&acc)[C::FM][C::FN], int m0, int rows, int j0,
                                            int wm, int wn, int lane) {
  static_assert(C::FN % 2 == 0, "gate/up pairing needs an even number of 32-column fragments");
  const int I = g.I, layout = g.layout;
  T* a_out = (T*)g.out0;
  float* z_out = (float*)g.out1;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rl = wm * C::WTM + fm * 32 + (lane & 31);
    if (rl >= rows) continue;
    const size_t p = (size_t)(m0 + rl);
#pragma unroll
    for (int pr = 0; pr < C::FN / 2; ++pr)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      const int j = j0 + (wn * (C::FN / 2) + pr) * 32 + acc_col4(vg, lane);
      if (j >= I) continue;
      float gv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gv[i] = acc[fm][2 * pr][vg * 4 + i];
        uv[i] = acc[fm][2 * pr + 1][vg * 4 + i];
      }
      if (WRITE_A)
        store4<T>(a_out + p * I + j, glu_fwd(gv[0], uv[0], g.act, g.limit, g.alpha),
                  glu_fwd(gv[1], uv[1], g.act, g.limit, g.alpha), glu_fwd(gv[2], uv[2], g.act, g.limit, g.alpha),
                  glu_fwd(gv[3], uv[3], g.act, g.limit, g.alpha));
      if (WRITE_Z) {
        float* zr = z_out + p * 2 * I;
        if (layout) {
          store4x2<float>(zr + 2 * j, gv, uv);
        } else {
          store4<float>(zr + j, gv[0], gv[1], gv[2], gv[3]);
          store4<float>(zr + I + j, uv[0], uv[1], uv[2], uv[3]);
        }
      }
    }
  }
}

// down: Y fp32 [S,H] = routing weight * (a . Wd^T), columns n0 + ...
template <class C>
__device__ __forceinline__ void epi_down(const GArgs& g, f32x16 (&acc)[C::FM][C::FN], int m0, int rows, int n0,
                                         int wm, int wn, int lane) {
  const int H = g.H;
  float* Y = (float*)g.out0;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rl = wm * C::WTM + fm * 32 + (lane & 31);
    if (rl >= rows) continue;
    const size_t p = (size_t)(m0 + rl);
    const float w = g.w_of_pos[p];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int n = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
        if (n < H)
          store4<float>(Y + p * H + n, w * acc[fm][fn][vg * 4], w * acc[fm][fn][vg * 4 + 1],
                        w * acc[fm][fn][vg * 4 + 2], w * acc[fm][fn][vg * 4 + 3]);
      }
  }
}

// down dgrad: r = acc (columns n0 + ... of I); a = phi(Z), partial <r, a> of
// the tile's columns per row (reduced over the WN waves of a row through
// `red`, [WN][BM] floats of LDS no wave still reads, into partials[p][nt]),
// da = w r, dZ = phi'(Z) da (type T), aw = w a (type T).  Per 32-row group,
// all of the lane's Z values are loaded first, from addresses clamped into
// the tile (rows past the tile's end read its last row, columns past I the
// last four), and only the results are predicated: loads issued one register
// group at a time behind the bounds test each waited out the HBM latency
// (0.84 -> 0.78 ms on the gpt-oss layer, 4.60 -> 4.00 ms on the Zipf batch).
template <class C, typename T>
__device__ __forceinline__ void epi_down_dgrad(const GArgs& g, f32x16 (&acc)[C::FM][C::FN], int m0, int rows,
                                               int n0, int nt, int wm, int wn, int lane, float* red) {
  const int I = g.I, layout = g.layout;
  const float* Z = (const float*)g.Z;
  T* dZ = (T*)g.out0;
  T* aw = (T*)g.out1;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rl = wm * C::WTM + fm * 32 + (lane & 31);
    float rs = 0.f;
    const size_t p = (size_t)(m0 + min(rl, rows - 1));
    const float w = g.w_of_pos[p];
    const float* zr = Z + p * 2 * I;
    T* dzr = dZ + p * 2 * I;
    // interleaved rows: (g, u) pairs, za = columns i, i+1, zb = i+2, i+3;
    // concatenated rows: za = gate, zb = up, columns i .. i+3
    float4 za[C::FN][4], zb[C::FN][4];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int i = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
        const int ic = i < I ? i : I - 4;   // I is a multiple of 8
        za[fn][vg] = *(const float4*)(zr + (layout ? 2 * ic : ic));
        zb[fn][vg] = *(const float4*)(zr + (layout ? 2 * ic + 4 : I + ic));
      }
    if (rl < rows) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int i = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
          if (i >= I) continue;
          const float4 z0 = za[fn][vg], z1 = zb[fn][vg];
          float gv[4], uv[4];
          if (layout) {
            gv[0] = z0.x; uv[0] = z0.y; gv[1] = z0.z; uv[1] = z0.w;
            gv[2] = z1.x; uv[2] = z1.y; gv[3] = z1.z; uv[3] = z1.w;
          } else {
            gv[0] = z0.x; gv[1] = z0.y; gv[2] = z0.z; gv[3] = z0.w;
            uv[0] = z1.x; uv[1] = z1.y; uv[2] = z1.z; uv[3] = z1.w;
          }
          float dg[4], du[4], a[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float r = acc[fm][fn][vg * 4 + q];
            a[q] = glu_bwd(gv[q], uv[q], w * r, g.act, g.limit, g.alpha, dg[q], du[q]);
            rs += r * a[q];
          }
          if (layout) {
            store4x2<T>(dzr + 2 * i, dg, du);
          } else {
            store4<T>(dzr + i, dg[0], dg[1], dg[2], dg[3]);
            store4<T>(dzr + I + i, du[0], du[1], du[2], du[3]);
          }
          store4<T>(aw + p * I + i, w * a[0], w * a[1], w * a[2], w * a[3]);
        }
    }
    // this lane and lane^32 hold the two column halves of the same row
    rs += __shfl_xor(rs, 32);
    if (lane < 32) red[wn * C::BM + wm * C::WTM + fm * 32 + lane] = rs;
  }
  __syncthreads();
  // one partial per 128 columns (partials[p][slot], slot = column / 128), the
  // sum of the waves that cover them, in wave order
  constexpr int PPT = C::BN / 128, WPP = C::WN / PPT;
  static_assert(C::BN % 128 == 0 && C::WN % PPT == 0, "waves split evenly over 128-column parts");
  for (int idx = threadIdx.x; idx < rows * PPT; idx += C::NT) {
    const int r = idx / PPT, pp = idx - r * PPT;
    const int slot = nt * PPT + pp;
    if (slot * 128 >= I) continue;
    float s = 0.f;
    for (int q = pp * WPP; q < (pp + 1) * WPP; ++q) s += red[q * C::BM + r];
    g.partials[(size_t)(m0 + r) * g.nparts + slot] = s;
  }
}

// gate_up dgrad: dXp fp32 [S,H], columns n0 + ...
template <class C>
__device__ __forceinline__ void epi_gate_up_dgrad(const GArgs& g, f32x16 (&acc)[C::FM][C::FN], int m0, int rows,
                                                  int n0, int wm, int wn, int lane) {
  const int H = g.H;
  float* dXp = (float*)g.out0;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rl = wm * C::WTM + fm * 32 + (lane & 31);
    if (rl >= rows) continue;
    const size_t p = (size_t)(m0 + rl);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int n = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
        if (n < H)
          store4<float>(dXp + p * H + n, acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1], acc[fm][fn][vg * 4 + 2],
                        acc[fm][fn][vg * 4 + 3]);
      }
  }
}

// ------------------------------------------------------------------ host side
// Large-tile engine (gemm_dma.hip): bf16 operands, H and I multiples of 32;
// each launch covers the large-tile experts (large_tile_expert).
bool dma_enabled(const GemmProblem& pb);
hipError_t dma_gate_up(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                       hipStream_t s);
hipError_t dma_down(const GemmProblem& pb, const void* a, const void* Wd, void* Yp, hipStream_t s);
hipError_t dma_down_dgrad(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ, void* aw,
                          float* partials, int nparts, hipStream_t s);
hipError_t dma_gate_up_dgrad(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp, hipStream_t s);
// The experts of tile set 2 (ps = the problem with tile_set 2) on 128 x 256
// tiles of the same engine, when H and I are multiples of 64.
bool dma_small_enabled(const GemmProblem& pb);
hipError_t dma_gate_up_small(const GemmProblem& ps, const void* X, const void* Wgu, void* a_out, void* z_out,
                             hipStream_t s);
hipError_t dma_down_small(const GemmProblem& ps, const void* a, const void* Wd, void* Yp, hipStream_t s);
hipError_t dma_down_dgrad_small(const GemmProblem& ps, const void* dY, const void* Wd, const void* Z, void* dZ,
                                void* aw, float* partials, int nparts, hipStream_t s);
hipError_t dma_gate_up_dgrad_small(const GemmProblem& ps, const void* dZ, const void* Wgu, void* dXp, hipStream_t s);
// weight gradients (dW[e] = A_e^T B_e) of the experts with more than hot_min positions
bool dma_wgrad_enabled(const GemmProblem& pb);
hipError_t dma_wgrad(const GemmProblem& pb, bool gate_up, const void* A, const void* B, void* dW, int hot_min,
                     hipStream_t s);

// Tile table of a kernel with bm-row tiles over the problem's set of experts.
inline int tile_table(const GemmProblem& pb, int bm) {
  if (pb.tile_set == 1) return TILE_BIG256;   // bm is 256
  if (pb.tile_set == 2) return bm == 192 ? TILE_SMALL192 : TILE_SMALL128;   // bm is 128 or 192
  return bm == 32 ? 0 : bm == 64 ? 1 : bm == 128 ? 2 : bm == 256 ? 3 : 4;
}

inline GArgs base_args(const GemmProblem& pb, int bm) {
  GArgs g = {};
  const RouteState& rs = *pb.rs;
  g.offsets = rs.offsets;
  g.tile_prefix = rs.tile_prefix + tile_table(pb, bm) * (pb.E + 1);
  g.tok_of_pos = rs.tok_of_pos;
  g.w_of_pos = rs.w_of_pos;
  g.expert_order = rs.expert_order;
  g.T = pb.T; g.H = pb.H; g.I = pb.I; g.E = pb.E; g.K = pb.K; g.S = pb.S;
  g.act = pb.act; g.layout = pb.layout; g.limit = pb.limit; g.alpha = pb.alpha;
  return g;
}

// The gate/up row view of a weight-shaped tensor (see GArgs).
inline void gu_view(const GemmProblem& pb, const void* fused_or_gate, const void* up, size_t esz, const void*& g0,
                    const void*& u0) {
  const size_t IH = (size_t)pb.I * pb.H;
  g0 = fused_or_gate;
  if (pb.w_up) u0 = up;
  else u0 = (const char*)fused_or_gate + (pb.layout ? (size_t)pb.H : IH) * esz;
}
inline void set_gu(GArgs& g, const GemmProblem& pb, const void* w, void* dw, size_t dw_esz) {
  const size_t esz = pb.dtype == 0 ? 2 : 4;
  const long IH = (long)pb.I * pb.H;
  g.gu_sep = pb.w_up != nullptr;
  g.gu_es = pb.w_up ? IH : 2 * IH;
  g.gu_rs = (!pb.w_up && pb.layout) ? 2L * pb.H : pb.H;
  if (w) gu_view(pb, w, pb.w_up, esz, g.gu_g, g.gu_u);
  if (dw) {
    const void *dg, *du;
    gu_view(pb, dw, pb.dw_up, dw_esz, dg, du);
    g.dgu_g = (void*)dg;
    g.dgu_u = (void*)du;
  }
}

inline int mtiles_upper(int S, int E, int bm) { return (S + bm - 1) / bm + (E < S ? E : S); }
// Token-row grids: worst-case tile count, rounded up to 8 plus 8 (see row_tile).
inline long row_grid(const GemmProblem& pb, int bm, int ntn) {
  const long t = (long)mtiles_upper(pb.S, pb.E, bm) * ntn;
  return ((t + 7) / 8) * 8 + 8;
}


}  // namespace moe
