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

// Output layout of a 32x32 MFMA accumulator: lane l holds column l%32 and,
// for register v, row 8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ int acc_row(int v, int lane) { return ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3); }

// Hardware dispatches consecutive workgroups round-robin over the 8 XCDs.
// Remap so that each XCD walks a contiguous range of logical tiles (tiles
// that share operands then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb >> 3;
  if (b >= (per << 3)) return b;
  return (b & 7) * per + (b >> 3);
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
template <class C, int ROWS, int ROT>
struct RowLoader {
  using T = typename C::elem;
  static constexpr int ITEMS = ROWS * C::CPR;
  static constexpr int NI = (ITEMS + C::NT - 1) / C::NT;
  const T* ptr[NI];
  int koff[NI];
  int loff[NI];
  uint4 reg[NI];
  int kdim;

  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rowptr, int kdim_) {
    kdim = kdim_;
    const int t = (threadIdx.x + ROT) % C::NT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = t + i * C::NT;
      if (q < ITEMS) {
        const int row = q / C::CPR, c = q % C::CPR;
        ptr[i] = rowptr(row) + c * C::VEC;
        koff[i] = c * C::VEC;
        loff[i] = C::lds_off(row, c);
      } else {
        ptr[i] = nullptr;
      }
    }
  }
  __device__ __forceinline__ void load(int kt) {
    const int k0 = kt * C::BK;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (ptr[i] != nullptr && k0 + koff[i] < kdim) reg[i] = *(const uint4*)(ptr[i] + k0);
      else reg[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(T* lds) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (ptr[i] != nullptr) *(uint4*)(lds + loff[i]) = reg[i];
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
  uint32_t reg[NI][VEC][4];
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
  template <class KRow>
  __device__ __forceinline__ void load(int kt, KRow krow) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int k = kt * C::BK + kb[i] * VEC + j;
        if (mn_ok[i] && k < kvalid) {
          const uint4 v = *(const uint4*)(krow(k) + cb[i] * VEC);
          reg[i][j][0] = v.x; reg[i][j][1] = v.y; reg[i][j][2] = v.z; reg[i][j][3] = v.w;
        } else {
          reg[i][j][0] = reg[i][j][1] = reg[i][j][2] = reg[i][j][3] = 0u;
        }
      }
    }
  }
  __device__ __forceinline__ void store(T* lds) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!on[i]) continue;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        uint32_t o[4];
        if (sizeof(T) == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t a = reg[i][2 * q][c >> 1], b = reg[i][2 * q + 1][c >> 1];
            o[q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = reg[i][q][c];
        }
        const int row = cb[i] * VEC + c;
        *(uint4*)(lds + C::lds_off(row, kb[i])) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

// ------------------------------------------------------------------ mainloop
template <class C>
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
        a[fm] = *(const bf16x8_t*)(As + C::lds_off(wm * C::WTM + fm * 32 + r32, chunk));
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        b[fn] = *(const bf16x8_t*)(Bs + C::lds_off(wn * C::WTN + fn * 32 + r32, chunk));
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
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
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  }
}

// Double-buffered K loop: the next tile's global loads are in flight while
// the current tile is multiplied; one barrier per step.
template <class C, class AL, class BL, class ALoadFn, class BLoadFn>
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
  aload(al, 0);
  bload(bl, 0);
  al.store(As0);
  bl.store(Bs0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      aload(al, kt + 1);
      bload(bl, kt + 1);
    }
    mma_tile<C>(odd ? As1 : As0, odd ? Bs1 : Bs0, acc);
    if (more) {
      al.store(odd ? As0 : As1);
      bl.store(odd ? Bs0 : Bs1);
    }
    __syncthreads();
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

// Which (expert, first row, rows) an M-tile index maps to; false if past the end.
template <int BM>
__device__ __forceinline__ bool find_mtile(const GArgs& g, int mt, int& e, int& m0, int& rows) {
  const int* tp = g.tile_prefix;
  if (mt >= tp[g.E]) return false;
  int lo = 0, hi = g.E;            // largest e with tp[e] <= mt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tp[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  e = lo;
  m0 = g.offsets[e] + (mt - tp[e]) * BM;
  rows = min(BM, g.offsets[e + 1] - m0);
  return true;
}

#define GEMM_PROLOGUE(C)                                                   \
  using T = typename C::elem;                                              \
  __shared__ __attribute__((aligned(16))) char smem_raw[C::LDS_BYTES];     \
  T* lds = (T*)smem_raw;                                                   \
  const int L = xcd_remap(blockIdx.x, gridDim.x);                          \
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;              \
  const int wm = wave / C::WN, wn = wave % C::WN;                          \
  (void)lane; (void)wm; (void)wn;

// ---------------------------------------------------------------- gate_up fwd
// C[p, n] over local columns n: 32-column groups alternate gate / up for the
// same activation columns, so every lane holds matching g and u accumulators.
template <class C, bool WRITE_A, bool WRITE_Z>
__global__ __launch_bounds__(C::NT) void gate_up_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  const int mt = L / g.ntn, nt = L % g.ntn;
  int e, m0, rows;
  if (!find_mtile<C::BM>(g, mt, e, m0, rows)) return;
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
  mainloop<C>(al, bl, [](auto& l, int kt) { l.load(kt); }, [](auto& l, int kt) { l.load(kt); },
              (H + C::BK - 1) / C::BK, lds, acc);

  T* a_out = (T*)g.out0;
  float* z_out = (float*)g.out1;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int c = 0; c < C::FN / 2; ++c) {
      const int jl = ((wn * C::WTN / 32 + 2 * c) >> 1) * 32 + (lane & 31);
      const int j = j0 + jl;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = wm * C::WTM + fm * 32 + acc_row(v, lane);
        if (rl >= rows || j >= I) continue;
        const size_t p = (size_t)(m0 + rl);
        const float gv = acc[fm][2 * c][v], uv = acc[fm][2 * c + 1][v];
        if (WRITE_A) store_val<T>(a_out + p * I + j, glu_fwd(gv, uv, g.act, g.limit, g.alpha));
        if (WRITE_Z) {
          const int gcol = layout ? 2 * j : j, ucol = layout ? 2 * j + 1 : I + j;
          z_out[p * 2 * I + gcol] = gv;
          z_out[p * 2 * I + ucol] = uv;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down fwd
template <class C>
__global__ __launch_bounds__(C::NT) void down_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  const int mt = L / g.ntn, nt = L % g.ntn;
  int e, m0, rows;
  if (!find_mtile<C::BM>(g, mt, e, m0, rows)) return;
  const int H = g.H, I = g.I;
  const T* Aa = (const T*)g.A;
  const T* W = (const T*)g.B + (size_t)e * H * I;
  const int n0 = nt * C::BN;
  RowLoader<C, C::BM, 0> al;
  RowLoader<C, C::BN, 0> bl;
  al.init([&](int r) { return Aa + (size_t)(m0 + min(r, rows - 1)) * I; }, I);
  bl.init([&](int r) { return W + (size_t)min(n0 + r, H - 1) * I; }, I);
  f32x16 acc[C::FM][C::FN];
  mainloop<C>(al, bl, [](auto& l, int kt) { l.load(kt); }, [](auto& l, int kt) { l.load(kt); },
              (I + C::BK - 1) / C::BK, lds, acc);
  float* Y = (float*)g.out0;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = wm * C::WTM + fm * 32 + acc_row(v, lane);
      if (rl >= rows) continue;
      const int p = m0 + rl;
      const float w = g.w_of_pos[p];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int n = n0 + wn * C::WTN + fn * 32 + (lane & 31);
        if (n < H) Y[(size_t)p * H + n] = w * acc[fm][fn][v];
      }
    }
  }
}

// ---------------------------------------------------------------- down dgrad
// r[p, i] = sum_h dY[tok(p), h] * Wd[e][h, i]; epilogue: a = phi(Z), partial
// <r, a> per row for dTopkW, da = w r, dZ = phi'(Z) da, aw = w a.
template <class C>
__global__ __launch_bounds__(C::NT) void down_dgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  const int mt = L / g.ntn, nt = L % g.ntn;
  int e, m0, rows;
  if (!find_mtile<C::BM>(g, mt, e, m0, rows)) return;
  const int H = g.H, I = g.I;
  const T* dY = (const T*)g.A;
  const T* W = (const T*)g.B + (size_t)e * H * I;
  const int n0 = nt * C::BN;
  const int* tok = g.tok_of_pos;
  RowLoader<C, C::BM, 0> al;
  TransLoader<C, C::BN, C::NT / 2> bl;
  al.init([&](int r) { return dY + (size_t)tok[m0 + min(r, rows - 1)] * H; }, H);
  bl.init(I - n0, H);
  f32x16 acc[C::FM][C::FN];
  mainloop<C>(al, bl, [](auto& l, int kt) { l.load(kt); },
              [&](auto& l, int kt) { l.load(kt, [&](int k) { return W + (size_t)k * I + n0; }); },
              (H + C::BK - 1) / C::BK, lds, acc);

  const float* Z = (const float*)g.Z;
  T* dZ = (T*)g.out0;
  T* aw = (T*)g.out1;
  const int layout = g.layout;
  float rowsum[C::FM][16];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      rowsum[fm][v] = 0.f;
      const int rl = wm * C::WTM + fm * 32 + acc_row(v, lane);
      if (rl >= rows) continue;
      const size_t p = (size_t)(m0 + rl);
      const float w = g.w_of_pos[p];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int i = n0 + wn * C::WTN + fn * 32 + (lane & 31);
        if (i >= I) continue;
        const int gcol = layout ? 2 * i : i, ucol = layout ? 2 * i + 1 : I + i;
        const float gv = Z[p * 2 * I + gcol], uv = Z[p * 2 * I + ucol];
        const float r = acc[fm][fn][v];
        float dg, du;
        const float a = glu_bwd(gv, uv, w * r, g.act, g.limit, g.alpha, dg, du);
        rowsum[fm][v] += r * a;
        store_val<T>(dZ + p * 2 * I + gcol, dg);
        store_val<T>(dZ + p * 2 * I + ucol, du);
        store_val<T>(aw + p * I + i, w * a);
      }
    }
  }
  // Row sums over this block's columns: across the 32 lanes of a half-wave,
  // then across the WN waves in wave order (deterministic).
  float* red = (float*)smem_raw;   // [WN][BM]; the K loop ended with a barrier
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float s = rowsum[fm][v];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 8);
      s += __shfl_xor(s, 16);
      if ((lane & 31) == 0) red[wn * C::BM + wm * C::WTM + fm * 32 + acc_row(v, lane)] = s;
    }
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
__global__ __launch_bounds__(C::NT) void gate_up_dgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  const int mt = L / g.ntn, nt = L % g.ntn;
  int e, m0, rows;
  if (!find_mtile<C::BM>(g, mt, e, m0, rows)) return;
  const int H = g.H, I2 = 2 * g.I;
  const T* dZ = (const T*)g.A;
  const T* W = (const T*)g.B + (size_t)e * I2 * H;
  const int n0 = nt * C::BN;
  RowLoader<C, C::BM, 0> al;
  TransLoader<C, C::BN, C::NT / 2> bl;
  al.init([&](int r) { return dZ + (size_t)(m0 + min(r, rows - 1)) * I2; }, I2);
  bl.init(H - n0, I2);
  f32x16 acc[C::FM][C::FN];
  mainloop<C>(al, bl, [](auto& l, int kt) { l.load(kt); },
              [&](auto& l, int kt) { l.load(kt, [&](int k) { return W + (size_t)k * H + n0; }); },
              (I2 + C::BK - 1) / C::BK, lds, acc);
  float* dXp = (float*)g.out0;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = wm * C::WTM + fm * 32 + acc_row(v, lane);
      if (rl >= rows) continue;
      const size_t p = (size_t)(m0 + rl);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int n = n0 + wn * C::WTN + fn * 32 + (lane & 31);
        if (n < H) dXp[p * H + n] = acc[fm][fn][v];
      }
    }
  }
}

// ---------------------------------------------------------------- weight grads
// dW[e][m, n] = sum over the expert's positions p of A[p, m] * B[p, n]; both
// operands are token-major, so both go through the transposing loader.
// Experts are visited in descending token count (longest first).
template <class C, bool GATE_UP, typename OutT>
__global__ __launch_bounds__(C::NT) void wgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  const int tiles = g.ntm * g.ntn;
  const int er = L / tiles, tt = L % tiles;
  const int mt = tt / g.ntn, nt = tt % g.ntn;
  const int e = g.expert_order[er];
  const int off = g.offsets[e], cnt = g.offsets[e + 1] - off;
  const int H = g.H, I = g.I;
  const int M = GATE_UP ? 2 * I : H, N = GATE_UP ? H : I;
  const int m0 = mt * C::BM, n0 = nt * C::BN;
  const int* tok = g.tok_of_pos;
  const T* Ap = (const T*)g.A;   // GATE_UP: dZ [S,2I]; else dY [T,H] (gathered)
  const T* Bp = (const T*)g.B;   // GATE_UP: X [T,H] (gathered); else aw [S,I]
  TransLoader<C, C::BM, 0> al;
  TransLoader<C, C::BN, C::NT / 2> bl;
  al.init(M - m0, cnt);
  bl.init(N - n0, cnt);
  f32x16 acc[C::FM][C::FN];
  mainloop<C>(
      al, bl,
      [&](auto& l, int kt) {
        l.load(kt, [&](int k) {
          return GATE_UP ? Ap + (size_t)(off + k) * 2 * I + m0 : Ap + (size_t)tok[off + k] * H + m0;
        });
      },
      [&](auto& l, int kt) {
        l.load(kt, [&](int k) {
          return GATE_UP ? Bp + (size_t)tok[off + k] * H + n0 : Bp + (size_t)(off + k) * I + n0;
        });
      },
      (cnt + C::BK - 1) / C::BK, lds, acc);
  OutT* dW = (OutT*)g.out0 + (size_t)e * M * N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * C::WTM + fm * 32 + acc_row(v, lane);
      if (m >= M) continue;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int n = n0 + wn * C::WTN + fn * 32 + (lane & 31);
        if (n < N) store_val<OutT>(dW + (size_t)m * N + n, acc[fm][fn][v]);
      }
    }
  }
}

// ------------------------------------------------------------------ host side
using CfgB = Cfg<uint16_t, 128, 128, 64, 2, 2>;   // bf16
using CfgF = Cfg<float, 128, 128, 32, 2, 2>;      // fp32

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

template <class C, bool A, bool Z>
static hipError_t gate_up_impl(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                               hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = X; g.B = Wgu; g.out0 = a_out; g.out1 = z_out;
  g.ntn = (pb.I + C::BN / 2 - 1) / (C::BN / 2);
  const long grid = (long)mtiles_upper(pb.S, pb.E, C::BM) * g.ntn;
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
  const long grid = (long)mtiles_upper(pb.S, pb.E, C::BM) * g.ntn;
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
  const long grid = (long)mtiles_upper(pb.S, pb.E, C::BM) * g.ntn;
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
  const long grid = (long)mtiles_upper(pb.S, pb.E, C::BM) * g.ntn;
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
  const long grid = (long)pb.E * g.ntm * g.ntn;
  return run_kernel(GU ? "wgrad_gate_up" : "wgrad_down", s,
                    [&] { wgrad_kernel<C, GU, OutT><<<grid, C::NT, 0, s>>>(g); });
}

template <bool GU>
static hipError_t wgrad_dispatch(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  if (pb.dtype == 0)
    return pb.gdtype == 0 ? wgrad_impl<CfgB, GU, uint16_t>(pb, A, B, dW, s) : wgrad_impl<CfgB, GU, float>(pb, A, B, dW, s);
  return pb.gdtype == 0 ? wgrad_impl<CfgF, GU, uint16_t>(pb, A, B, dW, s) : wgrad_impl<CfgF, GU, float>(pb, A, B, dW, s);
}

hipError_t launch_wgrad_down(const GemmProblem& pb, const void* dY, const void* aw, void* dWd, hipStream_t s) {
  return wgrad_dispatch<false>(pb, dY, aw, dWd, s);
}

hipError_t launch_wgrad_gate_up(const GemmProblem& pb, const void* dZ, const void* X, void* dWgu, hipStream_t s) {
  return wgrad_dispatch<true>(pb, dZ, X, dWgu, s);
}

}  // namespace moe
