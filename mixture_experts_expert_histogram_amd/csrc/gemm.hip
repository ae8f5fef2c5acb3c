// Grouped GEMMs of the routed MoE expert computation on CDNA4 matrix cores.
//
// Forward ("Sparse expert dispatch and combine", "MoE training token repeat
// and expert computation", descriptions): per expert, the gate_up projection
// with the gated activation fused into its epilogue, then the down projection
// with the routing weight fused into its epilogue.
// Backward ("MoE expert parallel execution backward", description): the down
// projection's input gradient with the activation backward and the routing
// weight gradient fused in, the gate_up projection's input gradient, and the
// two weight gradients, which contract over each expert's tokens.
//
// One block computes a BM x BN tile of one expert's product C = A . B^T with
// fp32 accumulation on v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x2f32 for the
// fp32 instantiation).  A and B are staged through LDS, double-buffered, in a
// [row][k] layout whose 16-byte chunks are XOR-swizzled by row so that both
// the stores and the MFMA fragment reads are free of bank conflicts.
// Operands whose rows are contiguous in k are copied with 16-byte loads;
// operands contiguous along m/n (the weights in the backward's input
// gradients, every operand of the weight gradients) are read as 8x8 blocks
// and transposed in registers before their LDS store.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}
template <typename T> __device__ __forceinline__ void store_val(T* p, float v);
template <> __device__ __forceinline__ void store_val<uint16_t>(uint16_t* p, float v) { *p = (uint16_t)bf16_bits(v); }
template <> __device__ __forceinline__ void store_val<float>(float* p, float v) { *p = v; }

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

// Gated activation (SwiGLU, or the clamped GLU of the gpt-oss-shaped pages).
__device__ __forceinline__ float glu_fwd(float g, float u, int act, float L, float al) {
  if (act == 0) return g * sigmoid_f(g) * u;
  const float gc = fminf(g, L);
  const float uc = fminf(fmaxf(u, -L), L);
  return (uc + 1.f) * gc * sigmoid_f(al * gc);
}
// Returns a = phi(g,u) and (dg, du) = phi'(g,u) * da.
__device__ __forceinline__ float glu_bwd(float g, float u, float da, int act, float L, float al, float& dg,
                                         float& du) {
  if (act == 0) {
    const float s = sigmoid_f(g);
    const float silu = g * s;
    dg = da * u * s * (1.f + g * (1.f - s));
    du = da * silu;
    return silu * u;
  }
  const float gc = fminf(g, L);
  const float uc = fminf(fmaxf(u, -L), L);
  const float s = sigmoid_f(al * gc);
  const float q = gc * s;
  dg = (g <= L) ? da * (uc + 1.f) * s * (1.f + al * gc * (1.f - s)) : 0.f;
  du = (u >= -L && u <= L) ? da * q : 0.f;
  return (uc + 1.f) * q;
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
  *(uint2*)p = make_uint2(bf16_bits(a) | (bf16_bits(b) << 16), bf16_bits(c) | (bf16_bits(d) << 16));
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
// interleaved pairs (g0 u0 g1 u1 g2 u2 g3 u3)
template <typename T> __device__ __forceinline__ void store4x2(T* p, const float* g, const float* u);
template <> __device__ __forceinline__ void store4x2<uint16_t>(uint16_t* p, const float* g, const float* u) {
  *(uint4*)p = make_uint4(bf16_bits(g[0]) | (bf16_bits(u[0]) << 16), bf16_bits(g[1]) | (bf16_bits(u[1]) << 16),
                          bf16_bits(g[2]) | (bf16_bits(u[2]) << 16), bf16_bits(g[3]) | (bf16_bits(u[3]) << 16));
}
template <> __device__ __forceinline__ void store4x2<float>(float* p, const float* g, const float* u) {
  *(float4*)p = make_float4(g[0], u[0], g[1], u[1]);
  *(float4*)(p + 4) = make_float4(g[2], u[2], g[3], u[3]);
}

// ------------------------------------------------------------------ config
template <typename T, int BM_, int BN_, int BK_, int WM_, int WN_>
struct Cfg {
  using elem = T;
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int VEC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
  static constexpr int CPR = BK / VEC;                 // chunks per LDS row
  static constexpr int SW = CPR < 8 ? CPR : 8;         // swizzle period
  static constexpr int KSTEP = sizeof(T) == 2 ? 16 : 2;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static constexpr int LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * (int)sizeof(T);
  static_assert((CPR & (CPR - 1)) == 0, "chunks per row must be a power of two");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  __device__ static __forceinline__ int lds_off(int row, int chunk) {
    return row * BK + ((chunk ^ (row & (SW - 1))) * VEC);
  }
};

// K-contiguous operand: tile rows are m (or n), each row a contiguous run of k.
// Every load is issued unconditionally (an out-of-range chunk reads its row's
// first chunk instead) and masked to zero when written to LDS, so the loop
// body has no branches and the compiler can keep later loads in flight.
template <class C, int ROWS, int ROT>
struct RowLoader {
  using T = typename C::elem;
  static constexpr int ITEMS = ROWS * C::CPR;
  static constexpr int NI = (ITEMS + C::NT - 1) / C::NT;
  static constexpr bool ALL_ON = ITEMS % C::NT == 0;
  const T* rowp[NI];
  int koff[NI];
  int loff[NI];
  bool on[NI];
  uint4 reg[2][NI];   // two register sets: k-steps are fetched two steps ahead
  bool okm[2][NI];
  int kdim;

  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rowptr, int kdim_) {
    kdim = kdim_;
    const int t = (threadIdx.x + ROT) % C::NT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = t + i * C::NT;
      on[i] = ALL_ON || q < ITEMS;
      const int qq = on[i] ? q : 0;
      const int row = qq / C::CPR, c = qq % C::CPR;
      rowp[i] = rowptr(row);
      koff[i] = c * C::VEC;
      loff[i] = C::lds_off(row, c);
    }
  }
  template <int SET>
  __device__ __forceinline__ void load(int kt) {
    const int k0 = kt * C::BK;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool ok = k0 + koff[i] < kdim;
      okm[SET][i] = ok;
      reg[SET][i] = *(const uint4*)(rowp[i] + (ok ? k0 + koff[i] : 0));
    }
  }
  template <int SET>
  __device__ __forceinline__ void store(T* lds) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (on[i]) *(uint4*)(lds + loff[i]) = okm[SET][i] ? reg[SET][i] : make_uint4(0, 0, 0, 0);
  }
};

// MN-contiguous operand: memory rows are k, each a contiguous run of m (or n).
// A thread reads a VEC x VEC block (VEC k-rows x VEC columns), transposes it
// in registers, and stores VEC chunks of VEC consecutive k.  Lanes next to
// each other take different k-blocks so the LDS stores spread over banks.
template <class C, int ROWS, int ROT>
struct TransLoader {
  using T = typename C::elem;
  static constexpr int VEC = C::VEC;
  static constexpr int KB = C::BK / VEC;
  static constexpr int ITEMS = KB * (ROWS / VEC);
  static constexpr int NI = (ITEMS + C::NT - 1) / C::NT;
  int kb[NI], cb[NI];
  bool on[NI], mn_ok[NI];
  uint32_t reg[2][NI][VEC][4];   // two register sets (see RowLoader)
  bool okm[2][NI][VEC];
  int kvalid;

  __device__ __forceinline__ void init(int mn_valid, int kvalid_) {
    kvalid = kvalid_;
    const int t = (threadIdx.x + ROT) % C::NT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = t + i * C::NT;
      on[i] = q < ITEMS;
      kb[i] = q % KB;
      cb[i] = q / KB;
      mn_ok[i] = on[i] && cb[i] * VEC < mn_valid;
    }
  }
  // krow(k) -> pointer to element (k, first column of the tile)
  template <int SET, class KRow>
  __device__ __forceinline__ void load(int kt, KRow krow) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        // unconditional load (row 0, column 0 of the tile when out of range;
        // a tile is only loaded when kvalid >= 1), masked in store()
        const int k = kt * C::BK + kb[i] * VEC + j;
        const bool ok = mn_ok[i] && k < kvalid;
        okm[SET][i][j] = ok;
        const uint4 v = *(const uint4*)(krow(ok ? k : 0) + (ok ? cb[i] * VEC : 0));
        reg[SET][i][j][0] = v.x; reg[SET][i][j][1] = v.y; reg[SET][i][j][2] = v.z; reg[SET][i][j][3] = v.w;
      }
    }
  }
  template <int SET>
  __device__ __forceinline__ void store(T* lds) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!on[i]) continue;
#pragma unroll
      for (int j = 0; j < VEC; ++j)
        if (!okm[SET][i][j]) reg[SET][i][j][0] = reg[SET][i][j][1] = reg[SET][i][j][2] = reg[SET][i][j][3] = 0u;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        uint32_t o[4];
        if (sizeof(T) == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t a = reg[SET][i][2 * q][c >> 1], b = reg[SET][i][2 * q + 1][c >> 1];
            o[q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = reg[SET][i][q][c];
        }
        const int row = cb[i] * VEC + c;
        *(uint4*)(lds + C::lds_off(row, kb[i])) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

// MN-contiguous operand kept as rows of k in LDS (bf16 only): the tile is
// [BK k-rows][128 columns], 256-byte rows whose 16-byte chunks are
// XOR-swizzled by 4*(row%4); fragments are read with ds_read_b64_tr_b16,
// which hands each lane 4 consecutive k of one column.  The global loads are
// the same 16-byte chunks the transposing loader reads, without the register
// transpose.
template <class C, int ROT>
struct NLoader {
  using T = typename C::elem;
  static_assert(sizeof(T) == 2, "transposing LDS reads are 16-bit");
  static constexpr int COLS = 128, CPRN = COLS / 8;
  static constexpr int ITEMS = C::BK * CPRN;
  static constexpr int NI = (ITEMS + C::NT - 1) / C::NT;
  int kr[NI], col[NI], loff[NI];
  bool on[NI], col_ok[NI];
  uint4 reg[2][NI];
  bool okm[2][NI];
  int kvalid;

  __device__ __forceinline__ void init(int mn_valid, int kvalid_) {
    kvalid = kvalid_;
    const int t = (threadIdx.x + ROT) % C::NT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = t + i * C::NT;
      on[i] = q < ITEMS;
      kr[i] = q / CPRN;
      const int c = q % CPRN;
      col[i] = c * 8;
      col_ok[i] = on[i] && col[i] < mn_valid;
      loff[i] = kr[i] * COLS + ((c ^ ((kr[i] & 3) << 2)) << 3);
    }
  }
  template <int SET, class KRow>
  __device__ __forceinline__ void load(int kt, KRow krow) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // unconditional load (row 0, column 0 of the tile when out of range;
      // a tile is only loaded when kvalid >= 1), masked in store()
      const int k = kt * C::BK + kr[i];
      const bool ok = col_ok[i] && k < kvalid;
      okm[SET][i] = ok;
      reg[SET][i] = *(const uint4*)(krow(ok ? k : 0) + (ok ? col[i] : 0));
    }
  }
  template <int SET>
  __device__ __forceinline__ void store(T* lds) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (on[i]) *(uint4*)(lds + loff[i]) = okm[SET][i] ? reg[SET][i] : make_uint4(0, 0, 0, 0);
  }
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// 32 columns x 16 k of an NLoader tile: lane -> column cb + lane%32,
// k = kk*16 + 8*(lane/32) + 0..7 (the layout of the K-contiguous fragments).
template <class C>
__device__ __forceinline__ bf16x8_t frag_n(const typename C::elem* tile, int cb, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = cb + ((g & 1) << 4) + ((s & 3) << 2);
  const int chunk = col >> 3, within = (col & 7) * 2;
  const lds_char* base = (const lds_char*)tile;
  s16x4_t r[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = kk * 16 + ((g >> 1) << 3) + h * 4 + (s >> 2);
    const lds_char* p = base + krow * 256 + ((chunk ^ ((krow & 3) << 2)) << 4) + within;
    r[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  }
  bf16x8_t out;
  s16x4_t* o = (s16x4_t*)&out;
  o[0] = r[0];
  o[1] = r[1];
  return out;
}

// ------------------------------------------------------------------ mainloop
template <class C, bool A_N = false, bool B_N = false>
__device__ __forceinline__ void mma_tile(const typename C::elem* As, const typename C::elem* Bs,
                                         f32x16 (&acc)[C::FM][C::FN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < C::BK / C::KSTEP; ++kk) {
    if constexpr (sizeof(typename C::elem) == 2) {
      bf16x8_t a[C::FM], b[C::FN];
      const int chunk = kk * 2 + half;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        a[fm] = A_N ? frag_n<C>(As, wm * C::WTM + fm * 32, kk, lane)
                    : *(const bf16x8_t*)(As + C::lds_off(wm * C::WTM + fm * 32 + r32, chunk));
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        b[fn] = B_N ? frag_n<C>(Bs, wn * C::WTN + fn * 32, kk, lane)
                    : *(const bf16x8_t*)(Bs + C::lds_off(wn * C::WTN + fn * 32 + r32, chunk));
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[fn], a[fm], acc[fm][fn], 0, 0, 0);
    } else {
      float a[C::FM], b[C::FN];
      const int k = kk * 2 + half;
      const int chunk = k / C::VEC, within = k % C::VEC;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) a[fm] = As[C::lds_off(wm * C::WTM + fm * 32 + r32, chunk) + within];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b[fn] = Bs[C::lds_off(wn * C::WTN + fn * 32 + r32, chunk) + within];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(b[fn], a[fm], acc[fm][fn], 0, 0, 0);
    }
  }
}

// Double-buffered LDS with two register sets: global loads for k-step kt+2
// are issued before k-step kt is multiplied, so each load has two steps of
// MFMA work to land; one barrier per step.  The load functors are called as
// fn(loader, kt, std::integral_constant<int, SET>{}).
template <int N> using Set = std::integral_constant<int, N>;

// One register set: the next k-step's loads are in flight while the current
// one is multiplied (used where two sets would not fit in 256 VGPRs).
template <class C, bool A_N = false, bool B_N = false, class AL, class BL, class ALoadFn, class BLoadFn>
__device__ __forceinline__ void mainloop_pf1(AL& al, BL& bl, ALoadFn aload, BLoadFn bload, int nk,
                                             typename C::elem* lds, f32x16 (&acc)[C::FM][C::FN]) {
  using T = typename C::elem;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  if (nk <= 0) return;
  T* As0 = lds;
  T* As1 = lds + C::A_ELEMS;
  T* Bs0 = lds + 2 * C::A_ELEMS;
  T* Bs1 = Bs0 + C::B_ELEMS;
  aload(al, 0, Set<0>{});
  bload(bl, 0, Set<0>{});
  al.template store<0>(As0);
  bl.template store<0>(Bs0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      aload(al, kt + 1, Set<0>{});
      bload(bl, kt + 1, Set<0>{});
    }
    mma_tile<C, A_N, B_N>(odd ? As1 : As0, odd ? Bs1 : Bs0, acc);
    if (more) {
      al.template store<0>(odd ? As0 : As1);
      bl.template store<0>(odd ? Bs0 : Bs1);
    }
    __syncthreads();
  }
}

template <class C, bool A_N = false, bool B_N = false, class AL, class BL, class ALoadFn, class BLoadFn>
__device__ __forceinline__ void mainloop(AL& al, BL& bl, ALoadFn aload, BLoadFn bload, int nk,
                                         typename C::elem* lds, f32x16 (&acc)[C::FM][C::FN]) {
  using T = typename C::elem;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  if (nk <= 0) return;
  T* As0 = lds;
  T* As1 = lds + C::A_ELEMS;
  T* Bs0 = lds + 2 * C::A_ELEMS;
  T* Bs1 = Bs0 + C::B_ELEMS;
  // Every prefetch is issued, clamped to the last step (a redundant reload of
  // a tile that is still in L2), so the number of loads in flight does not
  // depend on a branch and the LDS stores of one set wait only for that set.
  const int last = nk - 1;
  aload(al, 0, Set<0>{});
  bload(bl, 0, Set<0>{});
  aload(al, min(1, last), Set<1>{});
  bload(bl, min(1, last), Set<1>{});
  al.template store<0>(As0);
  bl.template store<0>(Bs0);
  __syncthreads();
  for (int kt = 0;;) {
    // even step: LDS buffer 0 holds step kt, register set 1 holds step kt+1
    aload(al, min(kt + 2, last), Set<0>{});
    bload(bl, min(kt + 2, last), Set<0>{});
    mma_tile<C, A_N, B_N>(As0, Bs0, acc);
    if (kt + 1 < nk) {
      al.template store<1>(As1);
      bl.template store<1>(Bs1);
    }
    __syncthreads();
    if (++kt >= nk) break;
    // odd step: LDS buffer 1 holds step kt, register set 0 holds step kt+1
    aload(al, min(kt + 2, last), Set<1>{});
    bload(bl, min(kt + 2, last), Set<1>{});
    mma_tile<C, A_N, B_N>(As1, Bs1, acc);
    if (kt + 1 < nk) {
      al.template store<0>(As0);
      bl.template store<0>(Bs0);
    }
    __syncthreads();
    if (++kt >= nk) break;
  }
}

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
};

// Token-row tiles: (expert, N-tile, M-tile of BM rows), ordered by expert,
// then N-tile, then M-tile, so the M-tiles of one expert that share a weight
// tile are neighbours.  The grid is sized for the worst case; the actual tile
// count is read from the routing tables and split into 8 equal contiguous
// ranges, one per XCD (hardware deals workgroup b to XCD b % 8).  Returns
// false for a workgroup without a tile.
template <int BM>
__device__ __forceinline__ bool row_tile(const GArgs& g, int& e, int& m0, int& rows, int& nt) {
  const int* tp = g.tile_prefix;
  const int ntn = g.ntn;
  const int total = tp[g.E] * ntn;
  const int per = (total + 7) >> 3;
  const int b = blockIdx.x, j = b >> 3;
  if (j >= per) return false;
  const int t = (b & 7) * per + j;
  if (t >= total) return false;
  const int q = t / ntn;
  int lo = 0, hi = g.E;            // largest e with tp[e] <= q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tp[mid] <= q) lo = mid; else hi = mid - 1;
  }
  e = lo;
  const int nm = tp[e + 1] - tp[e];
  const int local = t - tp[e] * ntn;
  nt = local / nm;
  const int mt = local - nt * nm;
  m0 = g.offsets[e] + mt * BM;
  rows = min(BM, g.offsets[e + 1] - m0);
  return true;
}

// Weight-gradient tiles: chunks of 8 consecutive tiles are dealt round-robin
// to the XCDs in launch order (experts longest first), so every XCD gets a
// similar share of long and short experts and a chunk's tiles share operands
// in one L2.  Returns -1 past the end.
__device__ __forceinline__ int dealt_tile(int total) {
  const int b = blockIdx.x, x = b & 7, j = b >> 3;
  const int t = (((j >> 3) << 3) + x) * 8 + (j & 7);
  return t < total ? t : -1;
}

#define GEMM_PROLOGUE(C)                                                   \
  using T = typename C::elem;                                              \
  __shared__ __attribute__((aligned(16))) char smem_raw[C::LDS_BYTES];     \
  T* lds = (T*)smem_raw;                                                   \
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;              \
  const int wm = wave / C::WN, wn = wave % C::WN;                          \
  (void)lane; (void)wm; (void)wn;

// MN-contiguous operands: rows of k in LDS read with transposing LDS reads for
// bf16, an in-register transpose for fp32.
template <class C, int ROT>
using MNLoader = std::conditional_t<sizeof(typename C::elem) == 2, NLoader<C, ROT>, TransLoader<C, 128, ROT>>;
template <class C> constexpr bool kNLayout = sizeof(typename C::elem) == 2;

// bf16 operands fit two register sets in 256 VGPRs; fp32 ones use one.
template <class C, class AL, class BL, class ALoadFn, class BLoadFn>
__device__ __forceinline__ void mainloop_rows(AL& al, BL& bl, ALoadFn aload, BLoadFn bload, int nk,
                                              typename C::elem* lds, f32x16 (&acc)[C::FM][C::FN]) {
  if constexpr (sizeof(typename C::elem) == 2) mainloop<C>(al, bl, aload, bload, nk, lds, acc);
  else mainloop_pf1<C>(al, bl, aload, bload, nk, lds, acc);
}

// ---------------------------------------------------------------- gate_up fwd
// Local B rows: 32-row groups alternate gate and up rows of the same 32
// activation columns, so the fn = 0 and fn = 1 fragments of a wave hold
// matching g and u values.
template <class C, bool WRITE_A, bool WRITE_Z>
__global__ __launch_bounds__(C::NT, 2) void gate_up_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  static_assert(C::FN == 2 && C::WTN == 64, "gate/up pairing assumes 64-column wave tiles");
  int e, m0, rows, nt;
  if (!row_tile<C::BM>(g, e, m0, rows, nt)) return;
  const int H = g.H, I = g.I;
  const T* X = (const T*)g.A;
  const T* W = (const T*)g.B + (size_t)e * 2 * I * H;
  const int j0 = nt * (C::BN / 2);
  const int layout = g.layout;
  const int* tok = g.tok_of_pos;

  RowLoader<C, C::BM, 0> al;
  RowLoader<C, C::BN, 0> bl;
  al.init([&](int r) { return X + (size_t)tok[m0 + min(r, rows - 1)] * H; }, H);
  bl.init([&](int r) {
    const int q = r >> 5;
    int j = j0 + ((q >> 1) << 5) + (r & 31);
    j = min(j, I - 1);
    const int wrow = layout ? (2 * j + (q & 1)) : ((q & 1) ? I + j : j);
    return W + (size_t)wrow * H;
  }, H);
  f32x16 acc[C::FM][C::FN];
  mainloop_rows<C>(al, bl, [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); },
                   [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); },
                   (H + C::BK - 1) / C::BK, lds, acc);

  T* a_out = (T*)g.out0;
  float* z_out = (float*)g.out1;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rl = wm * C::WTM + fm * 32 + (lane & 31);
    if (rl >= rows) continue;
    const size_t p = (size_t)(m0 + rl);
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      const int j = j0 + wn * 32 + acc_col4(vg, lane);
      if (j >= I) continue;
      float gv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gv[i] = acc[fm][0][vg * 4 + i];
        uv[i] = acc[fm][1][vg * 4 + i];
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

// ---------------------------------------------------------------- down fwd
template <class C>
__global__ __launch_bounds__(C::NT, 2) void down_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  int e, m0, rows, nt;
  if (!row_tile<C::BM>(g, e, m0, rows, nt)) return;
  const int H = g.H, I = g.I;
  const T* Aa = (const T*)g.A;
  const T* W = (const T*)g.B + (size_t)e * H * I;
  const int n0 = nt * C::BN;
  RowLoader<C, C::BM, 0> al;
  RowLoader<C, C::BN, 0> bl;
  al.init([&](int r) { return Aa + (size_t)(m0 + min(r, rows - 1)) * I; }, I);
  bl.init([&](int r) { return W + (size_t)min(n0 + r, H - 1) * I; }, I);
  f32x16 acc[C::FM][C::FN];
  mainloop_rows<C>(al, bl, [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); },
                   [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); },
                   (I + C::BK - 1) / C::BK, lds, acc);
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

// ---------------------------------------------------------------- down dgrad
// r[p, i] = sum_h dYp[p, h] * Wd[e][h, i]; epilogue: a = phi(Z), partial
// <r, a> per row for dTopkW, da = w r, dZ = phi'(Z) da, aw = w a.
template <class C>
__global__ __launch_bounds__(C::NT, 2) void down_dgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  int e, m0, rows, nt;
  if (!row_tile<C::BM>(g, e, m0, rows, nt)) return;
  const int H = g.H, I = g.I;
  const T* dYp = (const T*)g.A;    // d_out rows gathered into expert order
  const T* W = (const T*)g.B + (size_t)e * H * I;
  const int n0 = nt * C::BN;
  RowLoader<C, C::BM, 0> al;
  MNLoader<C, C::NT / 2> bl;
  al.init([&](int r) { return dYp + (size_t)(m0 + min(r, rows - 1)) * H; }, H);
  bl.init(I - n0, H);
  f32x16 acc[C::FM][C::FN];
  auto aload = [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); };
  auto bload = [&](auto& l, int kt, auto set) {
    l.template load<decltype(set)::value>(kt, [&](int k) { return W + (size_t)k * I + n0; });
  };
  if constexpr (kNLayout<C>) mainloop<C, false, true>(al, bl, aload, bload, (H + C::BK - 1) / C::BK, lds, acc);
  else mainloop_pf1<C>(al, bl, aload, bload, (H + C::BK - 1) / C::BK, lds, acc);

  const float* Z = (const float*)g.Z;
  T* dZ = (T*)g.out0;
  T* aw = (T*)g.out1;
  const int layout = g.layout;
  float* red = (float*)smem_raw;   // [WN][BM]; the K loop ended with a barrier
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rl = wm * C::WTM + fm * 32 + (lane & 31);
    float rs = 0.f;
    if (rl < rows) {
      const size_t p = (size_t)(m0 + rl);
      const float w = g.w_of_pos[p];
      const float* zr = Z + p * 2 * I;
      T* dzr = dZ + p * 2 * I;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int i = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
          if (i >= I) continue;
          float gv[4], uv[4];
          if (layout) {
            const float4 z0 = *(const float4*)(zr + 2 * i), z1 = *(const float4*)(zr + 2 * i + 4);
            gv[0] = z0.x; uv[0] = z0.y; gv[1] = z0.z; uv[1] = z0.w;
            gv[2] = z1.x; uv[2] = z1.y; gv[3] = z1.z; uv[3] = z1.w;
          } else {
            const float4 zg = *(const float4*)(zr + i), zu = *(const float4*)(zr + I + i);
            gv[0] = zg.x; gv[1] = zg.y; gv[2] = zg.z; gv[3] = zg.w;
            uv[0] = zu.x; uv[1] = zu.y; uv[2] = zu.z; uv[3] = zu.w;
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
  for (int r = threadIdx.x; r < rows; r += C::NT) {
    float s = 0.f;
    for (int q = 0; q < C::WN; ++q) s += red[q * C::BM + r];
    g.partials[(size_t)(m0 + r) * g.nparts + nt] = s;
  }
}

// ---------------------------------------------------------------- gate_up dgrad
// dXp[p, h] = sum_j dZ[p, j] * Wgu[e][j, h]
template <class C>
__global__ __launch_bounds__(C::NT, 2) void gate_up_dgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  int e, m0, rows, nt;
  if (!row_tile<C::BM>(g, e, m0, rows, nt)) return;
  const int H = g.H, I2 = 2 * g.I;
  const T* dZ = (const T*)g.A;
  const T* W = (const T*)g.B + (size_t)e * I2 * H;
  const int n0 = nt * C::BN;
  RowLoader<C, C::BM, 0> al;
  MNLoader<C, C::NT / 2> bl;
  al.init([&](int r) { return dZ + (size_t)(m0 + min(r, rows - 1)) * I2; }, I2);
  bl.init(H - n0, I2);
  f32x16 acc[C::FM][C::FN];
  auto aload = [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); };
  auto bload = [&](auto& l, int kt, auto set) {
    l.template load<decltype(set)::value>(kt, [&](int k) { return W + (size_t)k * H + n0; });
  };
  if constexpr (kNLayout<C>) mainloop<C, false, true>(al, bl, aload, bload, (I2 + C::BK - 1) / C::BK, lds, acc);
  else mainloop_pf1<C>(al, bl, aload, bload, (I2 + C::BK - 1) / C::BK, lds, acc);
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

// ---------------------------------------------------------------- weight grads
// dW[e][m, n] = sum over the expert's positions p of A[p, m] * B[p, n]; both
// operands are position-major rows (hidden and d_out pre-gathered into
// expert order), so both go through the transposing loader.  Experts are
// visited in descending token count (longest first).  The K loops are short
// (an expert's tokens), so four workgroups share a CU to hide latency.
template <class C, bool GATE_UP, typename OutT>
__global__ __launch_bounds__(C::NT, 4) void wgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  const int tiles = g.ntm * g.ntn;
  const int L = dealt_tile(g.E * tiles);
  if (L < 0) return;
  const int er = L / tiles, tt = L % tiles;
  const int mt = tt / g.ntn, nt = tt % g.ntn;
  const int e = g.expert_order[er];
  const int off = g.offsets[e], cnt = g.offsets[e + 1] - off;
  const int H = g.H, I = g.I;
  const int M = GATE_UP ? 2 * I : H, N = GATE_UP ? H : I;
  const int m0 = mt * C::BM, n0 = nt * C::BN;
  const T* Ap = (const T*)g.A;   // GATE_UP: dZ [S,2I]; else dYp [S,H]
  const T* Bp = (const T*)g.B;   // GATE_UP: Xp [S,H]; else aw [S,I]
  MNLoader<C, 0> al;
  MNLoader<C, C::NT / 2> bl;
  al.init(M - m0, cnt);
  bl.init(N - n0, cnt);
  f32x16 acc[C::FM][C::FN];
  auto aload = [&](auto& l, int kt, auto set) {
    l.template load<decltype(set)::value>(kt, [&](int k) {
      return GATE_UP ? Ap + (size_t)(off + k) * 2 * I + m0 : Ap + (size_t)(off + k) * H + m0;
    });
  };
  auto bload = [&](auto& l, int kt, auto set) {
    l.template load<decltype(set)::value>(kt, [&](int k) {
      return GATE_UP ? Bp + (size_t)(off + k) * H + n0 : Bp + (size_t)(off + k) * I + n0;
    });
  };
  if constexpr (kNLayout<C>) mainloop_pf1<C, true, true>(al, bl, aload, bload, (cnt + C::BK - 1) / C::BK, lds, acc);
  else mainloop_pf1<C>(al, bl, aload, bload, (cnt + C::BK - 1) / C::BK, lds, acc);
  OutT* dW = (OutT*)g.out0 + (size_t)e * M * N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int m = m0 + wm * C::WTM + fm * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int n = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
        if (n < N)
          store4<OutT>(dW + (size_t)m * N + n, acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1],
                       acc[fm][fn][vg * 4 + 2], acc[fm][fn][vg * 4 + 3]);
      }
  }
}

// ------------------------------------------------------------------ host side
using CfgB = Cfg<uint16_t, 128, 128, 64, 2, 2>;   // bf16
using CfgF = Cfg<float, 128, 128, 32, 2, 2>;      // fp32
// weight gradients: half the LDS per workgroup, so three share a CU
using CfgWB = Cfg<uint16_t, 128, 128, 32, 2, 2>;
using CfgWF = Cfg<float, 128, 128, 16, 2, 2>;

static constexpr int log2_bm_index(int bm) { return bm == 32 ? 0 : bm == 64 ? 1 : bm == 128 ? 2 : 3; }

static GArgs base_args(const GemmProblem& pb, int bm) {
  GArgs g = {};
  const RouteState& rs = *pb.rs;
  g.offsets = rs.offsets;
  g.tile_prefix = rs.tile_prefix + log2_bm_index(bm) * (pb.E + 1);
  g.tok_of_pos = rs.tok_of_pos;
  g.w_of_pos = rs.w_of_pos;
  g.expert_order = rs.expert_order;
  g.T = pb.T; g.H = pb.H; g.I = pb.I; g.E = pb.E; g.K = pb.K; g.S = pb.S;
  g.act = pb.act; g.layout = pb.layout; g.limit = pb.limit; g.alpha = pb.alpha;
  return g;
}

static int mtiles_upper(int S, int E, int bm) { return (S + bm - 1) / bm + (E < S ? E : S); }
// Token-row grids: worst-case tile count, rounded up to 8 plus 8 (see row_tile).
static long row_grid(const GemmProblem& pb, int bm, int ntn) {
  const long t = (long)mtiles_upper(pb.S, pb.E, bm) * ntn;
  return ((t + 7) / 8) * 8 + 8;
}

template <class C, bool A, bool Z>
static hipError_t gate_up_impl(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                               hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = X; g.B = Wgu; g.out0 = a_out; g.out1 = z_out;
  g.ntn = (pb.I + C::BN / 2 - 1) / (C::BN / 2);
  const long grid = row_grid(pb, C::BM, g.ntn);
  return run_kernel(A ? "gate_up_glu" : "gate_up_z", s, [&] { gate_up_kernel<C, A, Z><<<grid, C::NT, 0, s>>>(g); });
}

template <class C>
static hipError_t gate_up_dispatch(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                                   hipStream_t s) {
  if (a_out && z_out) return gate_up_impl<C, true, true>(pb, X, Wgu, a_out, z_out, s);
  if (a_out) return gate_up_impl<C, true, false>(pb, X, Wgu, a_out, z_out, s);
  return gate_up_impl<C, false, true>(pb, X, Wgu, a_out, z_out, s);
}

hipError_t launch_gate_up(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                          hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  return pb.dtype == 0 ? gate_up_dispatch<CfgB>(pb, X, Wgu, a_out, z_out, s)
                       : gate_up_dispatch<CfgF>(pb, X, Wgu, a_out, z_out, s);
}

template <class C>
static hipError_t down_impl(const GemmProblem& pb, const void* a, const void* Wd, void* Yp, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = a; g.B = Wd; g.out0 = Yp;
  g.ntn = (pb.H + C::BN - 1) / C::BN;
  const long grid = row_grid(pb, C::BM, g.ntn);
  return run_kernel("down_weighted", s, [&] { down_kernel<C><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t launch_down(const GemmProblem& pb, const void* a, const void* Wd, void* Yp, hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  return pb.dtype == 0 ? down_impl<CfgB>(pb, a, Wd, Yp, s) : down_impl<CfgF>(pb, a, Wd, Yp, s);
}

int down_dgrad_nparts(int I) { return (I + 127) / 128; }   // both configs use BN = 128

template <class C>
static hipError_t down_dgrad_impl(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ,
                                  void* aw, float* partials, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = dY; g.B = Wd; g.Z = Z; g.out0 = dZ; g.out1 = aw; g.partials = partials;
  g.ntn = (pb.I + C::BN - 1) / C::BN;
  g.nparts = g.ntn;
  const long grid = row_grid(pb, C::BM, g.ntn);
  return run_kernel("down_dgrad_glu_bwd", s, [&] { down_dgrad_kernel<C><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t launch_down_dgrad(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ,
                             void* aw, float* partials, int* nparts, hipStream_t s) {
  *nparts = down_dgrad_nparts(pb.I);
  if (pb.S == 0) return hipSuccess;
  return pb.dtype == 0 ? down_dgrad_impl<CfgB>(pb, dY, Wd, Z, dZ, aw, partials, s)
                       : down_dgrad_impl<CfgF>(pb, dY, Wd, Z, dZ, aw, partials, s);
}

template <class C>
static hipError_t gate_up_dgrad_impl(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp,
                                     hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = dZ; g.B = Wgu; g.out0 = dXp;
  g.ntn = (pb.H + C::BN - 1) / C::BN;
  const long grid = row_grid(pb, C::BM, g.ntn);
  return run_kernel("gate_up_dgrad", s, [&] { gate_up_dgrad_kernel<C><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t launch_gate_up_dgrad(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp, hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  return pb.dtype == 0 ? gate_up_dgrad_impl<CfgB>(pb, dZ, Wgu, dXp, s)
                       : gate_up_dgrad_impl<CfgF>(pb, dZ, Wgu, dXp, s);
}

template <class C, bool GU, typename OutT>
static hipError_t wgrad_impl(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = A; g.B = B; g.out0 = dW;
  const int M = GU ? 2 * pb.I : pb.H, N = GU ? pb.H : pb.I;
  g.ntm = (M + C::BM - 1) / C::BM;
  g.ntn = (N + C::BN - 1) / C::BN;
  const long total = (long)pb.E * g.ntm * g.ntn;
  const long grid = ((total + 63) / 64) * 64;   // whole chunks of 8 tiles on each of the 8 XCDs
  return run_kernel(GU ? "wgrad_gate_up" : "wgrad_down", s,
                    [&] { wgrad_kernel<C, GU, OutT><<<grid, C::NT, 0, s>>>(g); });
}

template <bool GU>
static hipError_t wgrad_dispatch(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  if (pb.dtype == 0)
    return pb.gdtype == 0 ? wgrad_impl<CfgWB, GU, uint16_t>(pb, A, B, dW, s)
                          : wgrad_impl<CfgWB, GU, float>(pb, A, B, dW, s);
  return pb.gdtype == 0 ? wgrad_impl<CfgWF, GU, uint16_t>(pb, A, B, dW, s)
                        : wgrad_impl<CfgWF, GU, float>(pb, A, B, dW, s);
}

hipError_t launch_wgrad_down(const GemmProblem& pb, const void* dY, const void* aw, void* dWd, hipStream_t s) {
  return wgrad_dispatch<false>(pb, dY, aw, dWd, s);
}

hipError_t launch_wgrad_gate_up(const GemmProblem& pb, const void* dZ, const void* X, void* dWgu, hipStream_t s) {
  return wgrad_dispatch<true>(pb, dZ, X, dWgu, s);
}

}  // namespace moe
