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
#include "gemm_common.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace moe {

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
  // LDS is read 16 lanes at a time, 16 bytes each: one 256-byte bank window.
  // A fragment read takes one 16-byte chunk from each of 16 consecutive rows,
  // so the chunk index is XORed with the row's window index (rows per window
  // = 16 / CPR) and 16 consecutive rows land in 16 distinct slots.
  static constexpr int SW = CPR < 16 ? CPR : 16;       // swizzle period
  static constexpr int RPW = CPR < 16 ? 16 / CPR : 1;  // rows per 256-byte window
  static constexpr int KSTEP = sizeof(T) == 2 ? 16 : 2;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static constexpr int LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * (int)sizeof(T);
  // workgroups per CU the launch bounds ask for: two while both fit in LDS
  static constexpr int OCC = LDS_BYTES > 80 * 1024 ? 1 : 2;
  // 32-bit registers per thread for one k-step of staged operands
  static constexpr int STAGE_REGS = (A_ELEMS + B_ELEMS) * (int)sizeof(T) / NT / 4;
  static_assert((CPR & (CPR - 1)) == 0, "chunks per row must be a power of two");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  __device__ static __forceinline__ int lds_off(int row, int chunk) {
    return row * BK + ((chunk ^ ((row / RPW) & (SW - 1))) * VEC);
  }
};

// v if ok, else zeros, as bitwise ANDs: a select on a condition shared by all
// of a thread's chunks is otherwise compiled into a divergent branch, which
// splits the k-step into basic blocks the scheduler cannot interleave.
__device__ __forceinline__ uint4 masked(uint4 v, bool ok) {
  const uint32_t m = 0u - (uint32_t)ok;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

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
  static constexpr int WRITES = NI;   // LDS stores per step
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
      if (on[i]) *(uint4*)(lds + loff[i]) = masked(reg[SET][i], okm[SET][i]);
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
  // Re-target to a tile with mn_valid columns and kvalid k rows.
  __device__ __forceinline__ void retarget(int mn_valid, int kvalid_) {
    kvalid = kvalid_;
#pragma unroll
    for (int i = 0; i < NI; ++i) mn_ok[i] = on[i] && cb[i] * VEC < mn_valid;
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
  static constexpr int WRITES = NI;   // LDS stores per step
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
  __device__ __forceinline__ void retarget(int mn_valid, int kvalid_) {
    kvalid = kvalid_;
#pragma unroll
    for (int i = 0; i < NI; ++i) col_ok[i] = on[i] && col[i] < mn_valid;
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
      if (on[i]) *(uint4*)(lds + loff[i]) = masked(reg[SET][i], okm[SET][i]);
  }
};


// 32 columns x 16 k of an NLoader tile: lane -> column cb + lane%32,
// k = kk*16 + 8*(lane/32) + 0..7 (the layout of the K-contiguous fragments).
// Configs whose MN-contiguous A tile is 256 columns wide, held as two
// [k][128] halves (see the long-K weight gradient).
template <class C> struct WideA { static constexpr bool value = false; };
// 256-column N tiles (bf16): the MN-contiguous B tile is two [k][128] halves too
// (NLoader2); only B is MN-contiguous in the kernels that use them.
template <class C> constexpr bool kWideMN = WideA<C>::value || C::BN == 256;

template <class C>
__device__ __forceinline__ bf16x8_t frag_n(const typename C::elem* tile, int cb, int kk, int lane) {
  if constexpr (kWideMN<C>) {   // columns 128.. live in the second [k][128] half
    tile += (cb >> 7) * 128 * C::BK;
    cb &= 127;
  }
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

// Fragments of one 16-wide k-slice of a wave's tile (bf16).
template <class C>
struct KFrags {
  bf16x8_t a[C::FM], b[C::FN];
};

template <class C, bool A_N, bool B_N>
__device__ __forceinline__ void read_kfrags(const typename C::elem* As, const typename C::elem* Bs, int kk,
                                            KFrags<C>& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r32 = lane & 31, chunk = kk * 2 + (lane >> 5);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
    f.a[fm] = A_N ? frag_n<C>(As, wm * C::WTM + fm * 32, kk, lane)
                  : *(const bf16x8_t*)(As + C::lds_off(wm * C::WTM + fm * 32 + r32, chunk));
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
    f.b[fn] = B_N ? frag_n<C>(Bs, wn * C::WTN + fn * 32, kk, lane)
                  : *(const bf16x8_t*)(Bs + C::lds_off(wn * C::WTN + fn * 32 + r32, chunk));
}

template <class C>
__device__ __forceinline__ void mma_kfrags(const KFrags<C>& f, f32x16 (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[fn], f.a[fm], acc[fm][fn], 0, 0, 0);
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
enum : int { kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200 };

// One k-step of the bf16 pipeline (LDS buffers As/Bs hold step kt).  Global
// loads go to register set SET; the next LDS stage is stored from STORE_SET:
// with two sets, SET receives step kt+2 while the other set (loaded a step
// ago) holds step kt+1; with one set, SET = STORE_SET receives step kt+1 and is
// stored at the end of the same step.  The k-slices are
// software-pipelined: slice kk+1's fragments are read from LDS while slice
// kk's MFMAs run, so LDS latency is exposed once per step instead of once per
// slice, and the next stage's LDS stores (which only wait for loads issued a
// step ago) and this step's global loads are spread between the MFMAs.
template <class C, bool A_N, bool B_N, int SET, int STORE_SET, class AL, class BL, class ALoadFn, class BLoadFn>
__device__ __forceinline__ void pipelined_step(AL& al, BL& bl, ALoadFn aload, BLoadFn bload, int kload,
                                               const typename C::elem* As, const typename C::elem* Bs,
                                               typename C::elem* As_next, typename C::elem* Bs_next,
                                               f32x16 (&acc)[C::FM][C::FN]) {
  constexpr int KK = C::BK / C::KSTEP;
  constexpr int READS = C::FM * (A_N ? 2 : 1) + C::FN * (B_N ? 2 : 1);   // LDS reads per slice
  constexpr int MFMAS = C::FM * C::FN;                                   // per slice
  constexpr int LOADS = AL::NI + BL::NI;                                 // global loads per step
  constexpr int WRITES = AL::WRITES + BL::WRITES;                        // LDS stores per step
  static_assert(KK >= 2, "at least two k-slices per step");
  KFrags<C> f[2];
  read_kfrags<C, A_N, B_N>(As, Bs, 0, f[0]);
  aload(al, kload, Set<SET>{});
  bload(bl, kload, Set<SET>{});
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk + 1 < KK) read_kfrags<C, A_N, B_N>(As, Bs, kk + 1, f[(kk + 1) & 1]);
    mma_kfrags<C>(f[kk & 1], acc);
  }
  al.template store<STORE_SET>(As_next);
  bl.template store<STORE_SET>(Bs_next);
  // order: slice 0 reads, global loads, then per slice the next slice's reads
  // followed by its MFMAs with this step's LDS stores spread between them
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS, 0);
  __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, LOADS, 0);
  constexpr int WPS = (WRITES + KK - 2) / (KK - 1);   // LDS stores per slice after the first
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (kk + 1 < KK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS, 0);
#pragma unroll
    for (int m = 0; m < MFMAS; ++m) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (kk >= 1 && m < WPS) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
    }
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
  // a tile that is still in L2), and every step stores the next stage (after
  // the last step into the buffer nothing reads again), so a step is one
  // basic block whose loads in flight do not depend on a branch.
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
    pipelined_step<C, A_N, B_N, 0, 1>(al, bl, aload, bload, min(kt + 2, last), As0, Bs0, As1, Bs1, acc);
    __syncthreads();
    if (++kt >= nk) break;
    // odd step: LDS buffer 1 holds step kt, register set 0 holds step kt+1
    pipelined_step<C, A_N, B_N, 1, 0>(al, bl, aload, bload, min(kt + 2, last), As1, Bs1, As0, Bs0, acc);
    __syncthreads();
    if (++kt >= nk) break;
  }
}

#define GEMM_PROLOGUE(C)                                                   \
  using T = typename C::elem;                                              \
  __shared__ __attribute__((aligned(16))) char smem_raw[C::LDS_BYTES];     \
  T* lds = (T*)smem_raw;                                                   \
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;              \
  const int wm = wave / C::WN, wn = wave % C::WN;                          \
  (void)lane; (void)wm; (void)wn;

// Two NLoaders for a 256-column MN-contiguous tile, held as two [k][128]
// halves (128 x 256 token-row tiles); the second half's columns start 128
// after the first's, and its rows past the valid columns load in range and
// are masked to zero like the first's.
template <class C, int ROT>
struct NLoader2 {
  using T = typename C::elem;
  NLoader<C, ROT> h0;
  NLoader<C, (ROT + C::NT / 4) % C::NT> h1;
  static constexpr int NI = 2 * NLoader<C, ROT>::NI;
  static constexpr int WRITES = NI;
  __device__ __forceinline__ void init(int mn_valid, int kvalid) {
    h0.init(mn_valid, kvalid);
    h1.init(mn_valid - 128, kvalid);
  }
  __device__ __forceinline__ void retarget(int mn_valid, int kvalid) {
    h0.retarget(mn_valid, kvalid);
    h1.retarget(mn_valid - 128, kvalid);
  }
  template <int SET, class KRow>
  __device__ __forceinline__ void load(int kt, KRow krow) {
    h0.template load<SET>(kt, krow);
    h1.template load<SET>(kt, [&](int k) { return krow(k) + 128; });
  }
  template <int SET>
  __device__ __forceinline__ void store(T* lds) {
    h0.template store<SET>(lds);
    h1.template store<SET>(lds + 128 * C::BK);
  }
};

// MN-contiguous operands: rows of k in LDS read with transposing LDS reads for
// bf16, an in-register transpose for fp32.
template <class C, int ROT>
using MNLoader = std::conditional_t<sizeof(typename C::elem) == 2,
                                    std::conditional_t<C::BN == 256, NLoader2<C, ROT>, NLoader<C, ROT>>,
                                    TransLoader<C, 128, ROT>>;
template <class C> constexpr bool kNLayout = sizeof(typename C::elem) == 2;

// bf16 operands fit the two-set pipeline in 256 registers when a wave's
// tile is at most 64x64 and a k-step stages at most 32 registers per thread
// (128x128 tiles on 4 waves, 256x128 on 8); 192-row tiles (96 rows per wave)
// and fp32 operands use the one-set loop.
template <class C>
constexpr bool kTwoSets = sizeof(typename C::elem) == 2 && C::FM * C::FN <= 4 && C::STAGE_REGS <= 32;
template <class C, class AL, class BL, class ALoadFn, class BLoadFn>
__device__ __forceinline__ void mainloop_rows(AL& al, BL& bl, ALoadFn aload, BLoadFn bload, int nk,
                                              typename C::elem* lds, f32x16 (&acc)[C::FM][C::FN]) {
  if constexpr (kTwoSets<C>) mainloop<C>(al, bl, aload, bload, nk, lds, acc);
  else mainloop_pf1<C>(al, bl, aload, bload, nk, lds, acc);
}

// ---------------------------------------------------------------- gate_up fwd
// Local B rows: 32-row groups alternate gate and up rows of the same 32
// activation columns, so the fn = 2p and fn = 2p+1 fragments of a wave hold
// matching g and u values (activation columns (wn*FN/2 + p)*32 + 0..31).
template <class C, bool WRITE_A, bool WRITE_Z>
__global__ __launch_bounds__(C::NT, C::OCC) void gate_up_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  static_assert(C::FN % 2 == 0, "gate/up pairing needs an even number of 32-column fragments");
  int e, m0, rows, nt;
  if (!row_tile<C::BM>(g, e, m0, rows, nt)) return;
  const int H = g.H, I = g.I;
  const T* X = (const T*)g.A;
  const int j0 = nt * (C::BN / 2);
  const int layout = g.layout;
  const int* tok = g.tok_of_pos;

  RowLoader<C, C::BM, 0> al;
  RowLoader<C, C::BN, 0> bl;
  al.init([&](int r) { return X + (size_t)tok[m0 + min(r, rows - 1)] * H; }, H);
  bl.init([&](int r) {
    const int q = r >> 5;
    const int j = min(j0 + ((q >> 1) << 5) + (r & 31), I - 1);
    return gu_row((const T*)g.gu_g, (const T*)g.gu_u, g.gu_es, g.gu_rs, e, q & 1, j);
  }, H);
  f32x16 acc[C::FM][C::FN];
  mainloop_rows<C>(al, bl, [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); },
                   [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); },
                   (H + C::BK - 1) / C::BK, lds, acc);
  epi_gate_up<C, T, WRITE_A, WRITE_Z>(g, acc, m0, rows, j0, wm, wn, lane);
}

// ---------------------------------------------------------------- down fwd
template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void down_kernel(GArgs g) {
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
  epi_down<C>(g, acc, m0, rows, n0, wm, wn, lane);
}

// ---------------------------------------------------------------- down dgrad
// r[p, i] = sum_h dYp[p, h] * Wd[e][h, i]; epilogue: a = phi(Z), partial
// <r, a> per row for dTopkW, da = w r, dZ = phi'(Z) da, aw = w a.
template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void down_dgrad_kernel(GArgs g) {
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
  const int nk = (H + C::BK - 1) / C::BK;
  if constexpr (kTwoSets<C>) mainloop<C, false, true>(al, bl, aload, bload, nk, lds, acc);
  else mainloop_pf1<C, false, kNLayout<C>>(al, bl, aload, bload, nk, lds, acc);

  // the K loop ended with a barrier, so LDS is free for the row reduction
  epi_down_dgrad<C, T>(g, acc, m0, rows, n0, nt, wm, wn, lane, (float*)smem_raw);
}

// ---------------------------------------------------------------- gate_up dgrad
// dXp[p, h] = sum over the 2I columns m of dZ[p, m] * (gate or up row of m)[h]
template <class C, bool SEP>
__global__ __launch_bounds__(C::NT, C::OCC) void gate_up_dgrad_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  int e, m0, rows, nt;
  if (!row_tile<C::BM>(g, e, m0, rows, nt)) return;
  const int H = g.H, I = g.I, I2 = 2 * g.I;
  const T* dZ = (const T*)g.A;
  const int n0 = nt * C::BN;
  RowLoader<C, C::BM, 0> al;
  MNLoader<C, C::NT / 2> bl;
  al.init([&](int r) { return dZ + (size_t)(m0 + min(r, rows - 1)) * I2; }, I2);
  bl.init(H - n0, I2);
  f32x16 acc[C::FM][C::FN];
  auto aload = [](auto& l, int kt, auto set) { l.template load<decltype(set)::value>(kt); };
  // Row k of the weights in dZ-column order: in both fused layouts the fused
  // rows are in that order already (bg + k*H); separate tensors (SEP) switch
  // to the up tensor at k = I.
  const T* bg = (const T*)g.gu_g + g.gu_es * e + n0;
  const T* bu = (const T*)g.gu_u + g.gu_es * e + n0;
  auto bload = [&](auto& l, int kt, auto set) {
    l.template load<decltype(set)::value>(kt, [&](int k) {
      if constexpr (SEP) return k >= I ? bu + (size_t)(k - I) * H : bg + (size_t)k * H;
      else return bg + (size_t)k * H;
    });
  };
  const int nk = (I2 + C::BK - 1) / C::BK;
  if constexpr (kTwoSets<C>) mainloop<C, false, true>(al, bl, aload, bload, nk, lds, acc);
  else mainloop_pf1<C, false, kNLayout<C>>(al, bl, aload, bload, nk, lds, acc);
  epi_gate_up_dgrad<C>(g, acc, m0, rows, n0, wm, wn, lane);
}

// ---------------------------------------------------------------- weight grads
// dW[e][m, n] = sum over the expert's positions p of A[p, m] * B[p, n]; both
// operands are position-major rows (hidden and d_out pre-gathered into
// expert order), so both are MN-contiguous.  This tiled kernel takes the
// experts above the resident-operand kernel's limit with bf16 operands, and
// every expert with fp32 operands.  The output (E x M x N,
// written once) dominates the traffic and the K loops can be short (an
// expert's positions), so the kernel is built around keeping the store
// stream busy:
//
// * One persistent workgroup per CU with two roles.  The MMA waves (C::NT
//   threads: 8 waves of 64x32 for bf16) load operands and run the MFMAs; four
//   more waves only write dW.  At the end of a tile the MMA waves put the
//   accumulators, converted to the output type, into an LDS staging tile and
//   go on with the next tile; the store waves copy the staging tile to dW in
//   whole row segments (256 bytes bf16, 512 bytes fp32).  A wave's vmcnt counts its loads and stores in
//   issue order, so a wave that did both would wait for its stores before
//   using later loads; split over two roles, neither stream waits for the
//   other.
// * The MMA waves run one pipelined step loop across all of their tiles:
//   the loads for the step after next (possibly of the next tile) are in
//   flight while a step is multiplied.
// * Both roles walk the same (tile, k-step) cursor and meet at the same
//   barriers: one per step, one more after a finished tile is staged.
//
// Tile placement (hardware deals workgroup b to XCD b % 8).  Experts are
// visited in descending position count.  Experts with at most g.big
// positions are pinned whole to one XCD, dealt round-robin, so their
// activations are fetched into one L2 only; larger experts come first and
// are split into 8 contiguous tile ranges, one per XCD, so skewed routing
// stays balanced.  An XCD's tile list (split experts' ranges, then its
// pinned experts) is dealt round-robin to its workgroups, so the workgroups
// of one XCD work on neighbouring tiles that share operands.
struct WgradPlan {
  int tiles, tpx;
};
__host__ __device__ inline WgradPlan wgrad_plan(int ntm, int ntn) {
  WgradPlan p;
  p.tiles = ntm * ntn;
  p.tpx = (p.tiles + 7) / 8;
  return p;
}

struct WItem {
  int e, off, cnt, nk, m0, n0;
};

// The routing tables are copied to LDS at kernel start: lookups from global
// memory inside the loops would be vector loads (the compiler cannot prove
// the dW stores do not alias them), and a wave's vmcnt would then make each
// lookup wait for every load and store the wave has in flight.
struct WgradTables {
  int order[MAX_E];
  int offsets[MAX_E + 1];
};

template <class C>
struct WgradList {
  const WgradTables* tab;   // in LDS
  int E, ntn, tiles, tpx, nb, x, len_x, count, base;

  // number of leading experts (descending count) with more than lim positions
  __device__ __forceinline__ int leading_above(int lim, int l, int h) const {
    while (l < h) {
      const int mid = (l + h) >> 1;
      const int e = tab->order[mid];
      if (tab->offsets[e + 1] - tab->offsets[e] > lim) l = mid + 1; else h = mid;
    }
    return l;
  }
  __device__ __forceinline__ void init(const GArgs& g, const WgradTables* t) {
    tab = t;
    ntn = g.ntn;
    const WgradPlan p = wgrad_plan(g.ntm, g.ntn);
    tiles = p.tiles;
    tpx = p.tpx;
    // the list is order[base .. hi): experts above hot_min are the long-K
    // kernel's, those at or below small_max the resident kernel's
    const int hi = g.small_max >= 0 ? leading_above(g.small_max, 0, g.E) : g.E;
    base = g.hot_min > 0 ? min(leading_above(g.hot_min, 0, g.E), hi) : 0;
    E = hi - base;
    nb = leading_above(g.big, base, hi) - base;   // experts with count > big, split over the XCDs
    x = blockIdx.x & 7;
    len_x = max(0, min((x + 1) * tpx, tiles) - x * tpx);
    const int npin = E - nb - x > 0 ? (E - nb - x + 7) / 8 : 0;
    count = nb * len_x + npin * tiles;
  }
  // Item i (0 <= i < count) of this XCD's list.  An expert without positions
  // gets one k-step whose loads are all masked (at row 0, which exists: the
  // kernel only runs with S > 0).
  __device__ __forceinline__ WItem item(int i) const {
    int er, t;
    if (i < nb * len_x) {
      er = i / len_x;
      t = x * tpx + (i - er * len_x);
    } else {
      i -= nb * len_x;
      const int q = i / tiles;
      t = i - q * tiles;
      er = nb + x + 8 * q;
    }
    WItem it;
    it.e = tab->order[base + er];
    it.off = tab->offsets[it.e];
    it.cnt = tab->offsets[it.e + 1] - it.off;
    if (it.cnt == 0) it.off = 0;
    it.nk = max(1, (it.cnt + C::BK - 1) / C::BK);
    it.m0 = (t / ntn) * C::BM;
    it.n0 = (t % ntn) * C::BN;
    return it;
  }
};

// Staging tile: [BM rows][BN values of the output type], 16-byte chunks
// XOR-swizzled by row, so the MMA lanes' writes (32 consecutive rows, one
// column group) and the store waves' reads (one row's chunks) spread over the
// banks.  bf16: a lane writes 8 bytes (4 values), half a chunk; the half is
// flipped for rows 16-31 of each 32-row group, so rows r and r+16 (same
// swizzled chunk) use different halves.
template <class C, typename OutT>
struct Stage {
  static constexpr int ROW = C::BN * (int)sizeof(OutT);   // bytes per row
  static constexpr int CPR = ROW / 16;                     // 16-byte chunks per row
  static constexpr int BYTES = C::BM * ROW;
  static_assert(CPR == 16 || CPR == 32, "staging rows of 256 or 512 bytes");
  __device__ static __forceinline__ int chunk(int r, int ch) { return r * ROW + ((ch ^ (r & (CPR - 1))) << 4); }
  // byte offset of output columns 4*c4 .. 4*c4+3 of row r
  __device__ static __forceinline__ int quad(int r, int c4) {
    if constexpr (sizeof(OutT) == 4) return chunk(r, c4);
    else return chunk(r, c4 >> 1) + ((((c4 & 1) ^ ((r >> 4) & 1))) << 3);
  }
  // 16-byte chunk ch of row r as stored (bf16 halves in column order)
  __device__ static __forceinline__ uint4 read(const char* stage, int r, int ch) {
    uint4 v = *(const uint4*)(stage + chunk(r, ch));
    if constexpr (sizeof(OutT) == 2)
      if ((r >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
    return v;
  }
};

constexpr int kStoreThreads = 256;   // four store waves

template <class C, bool GATE_UP, typename OutT>
__global__ __launch_bounds__(C::NT + kStoreThreads, 1) void wgrad_kernel(GArgs g) {
  using T = typename C::elem;
  static_assert(C::BN == 128, "store waves copy 32 chunks per row");
  using ST = Stage<C, OutT>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::LDS_BYTES + ST::BYTES];
  T* lds = (T*)smem_raw;
  char* stage = smem_raw + C::LDS_BYTES;
  const int H = g.H, I = g.I;
  const int M = GATE_UP ? 2 * I : H, N = GATE_UP ? H : I;
  const int lda = M, ldb = N;       // GATE_UP: dZ [S,2I], Xp [S,H]; else dYp [S,H], aw [S,I]
  OutT* dW = (OutT*)g.out0;
  // The host cannot tell without a sync whether any expert falls in this
  // kernel's range of positions; when the hottest expert does not, leave
  // before touching the tables.
  if (g.small_max >= 0) {
    const int e0 = g.expert_order[0];
    if (g.offsets[e0 + 1] - g.offsets[e0] <= g.small_max) return;
  }
  __shared__ WgradTables tab;
  for (int i = threadIdx.x; i <= g.E; i += C::NT + kStoreThreads) {
    if (i < g.E) tab.order[i] = g.expert_order[i];
    tab.offsets[i] = g.offsets[i];
  }
  __syncthreads();
  WgradList<C> list;
  list.init(g, &tab);
  const int K = gridDim.x >> 3;     // workgroups per XCD
  int ci = blockIdx.x >> 3;         // list item being multiplied / stored
  if (ci >= list.count) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Steps of this workgroup (one list item per lane, summed over the wave).
  int total = 0;
  for (int base = ci; base < list.count; base += 64 * K) {
    const int i = base + (threadIdx.x & 63) * K;
    int v = i < list.count ? list.item(i).nk : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    total += v;
  }
  total = __builtin_amdgcn_readfirstlane(total);
  const int total_even = (total + 1) & ~1;   // the MMA loop runs two steps per iteration
  WItem cur = list.item(ci);
  int ck = 0;
  // Advances the multiply cursor (stays on the last step at the end).
  auto next_step = [&]() {
    if (ck + 1 < cur.nk) ++ck;
    else if (ci + K < list.count) { ci += K; cur = list.item(ci); ck = 0; }
  };
  if (wave >= C::NT / 64) {
    // ---------------- store waves
    // A staged tile is read into registers at once (freeing the staging
    // tile) and written out a quarter at a time, one quarter per barrier
    // interval, with any rest flushed before the next tile is read.  Issuing
    // all of it at once would block the store waves on a saturated write
    // path and hold up the MMA waves at the next barrier.
    const int tid = threadIdx.x - C::NT;
    constexpr int PER = C::BM * ST::CPR / kStoreThreads;   // 16-byte chunks per thread
    constexpr int NQ = 4, QS = PER / NQ;
    constexpr int VPC = 16 / (int)sizeof(OutT);             // values per chunk
    static_assert(PER % NQ == 0, "store quarters");
    uint4 v[PER];
    OutT* dWt = dW;        // tile origin in dW of the registers' tile
    int next_q = NQ;       // next quarter to write (NQ: none pending)
    int stage_rows = 0, stage_cols = 0, stage_e = 0, stage_m0 = 0, stage_n0 = 0;
    auto write_quarter = [&](int q) {
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        if (qq != q) continue;
#pragma unroll
        for (int j = 0; j < QS; ++j) {
          const int i = qq * QS + j;
          const int idx = tid + i * kStoreThreads;
          const int r = idx / ST::CPR, c = (idx % ST::CPR) * VPC;
          if (r < stage_rows && c < stage_cols) {
            OutT* row = dWt + (size_t)r * N;   // fused dW: tile rows are consecutive rows
            if (GATE_UP && g.gu_sep) {           // separate dW_gate, dW_up: row m0 + r is a dZ column
              int up, j;
              zcol(stage_m0 + r, I, g.layout, up, j);
              row = gu_row((OutT*)g.dgu_g, (OutT*)g.dgu_u, g.gu_es, g.gu_rs, stage_e, up, j) + stage_n0;
            }
            *(uint4*)(row + c) = v[i];
          }
        }
      }
    };
    __syncthreads();   // prologue
    for (int st = 0; st < total_even; ++st) {
      __syncthreads();   // step done
      if (next_q < NQ) write_quarter(next_q++);
      if (st < total && ck + 1 == cur.nk) {
        while (next_q < NQ) write_quarter(next_q++);
        __syncthreads();   // tile staged
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int idx = tid + i * kStoreThreads;
          v[i] = ST::read(stage, idx / ST::CPR, idx % ST::CPR);
        }
        dWt = dW + ((size_t)cur.e * M + cur.m0) * N + cur.n0;
        stage_e = cur.e;
        stage_m0 = cur.m0;
        stage_n0 = cur.n0;
        stage_rows = min(C::BM, M - cur.m0);
        stage_cols = min(C::BN, N - cur.n0);
        next_q = 0;
        write_quarter(next_q++);
      }
      next_step();
    }
    while (next_q < NQ) write_quarter(next_q++);
    return;
  }

  // ---------------- MMA waves
  const int lane = threadIdx.x & 63;
  const int wm = wave / C::WN, wn = wave % C::WN;
  std::conditional_t<WideA<C>::value, NLoader2<C, 0>, MNLoader<C, 0>> al;   // 256 columns of M: two halves
  MNLoader<C, C::NT / 2> bl;
  al.init(M - cur.m0, cur.cnt);
  bl.init(N - cur.n0, cur.cnt);
  // Load cursor, two steps ahead of the multiply cursor.  It stops at the
  // last step, so loads past the end re-read that step and every step issues
  // the same loads.
  int li = ci, lk = 0;
  WItem ld = cur;
  const T* Ag = (const T*)g.A;
  const T* Bg = (const T*)g.B;
  auto issue = [&](auto set) {
    constexpr int SET = decltype(set)::value;
    al.retarget(M - ld.m0, ld.cnt);
    bl.retarget(N - ld.n0, ld.cnt);
    const T* Ap = Ag + (size_t)ld.off * lda + ld.m0;
    const T* Bp = Bg + (size_t)ld.off * ldb + ld.n0;
    al.template load<SET>(lk, [&](int k) { return Ap + (size_t)k * lda; });
    bl.template load<SET>(lk, [&](int k) { return Bp + (size_t)k * ldb; });
    if (lk + 1 < ld.nk) ++lk;
    else if (li + K < list.count) { li += K; ld = list.item(li); lk = 0; }
  };
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  // After the step's barrier: stage a finished tile, then a second barrier.
  auto finish_step = [&](int st) {
    if (st < total && ck + 1 == cur.nk) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int r = wm * C::WTM + fm * 32 + (lane & 31);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int vg = 0; vg < 4; ++vg) {
            const int c4 = (wn * C::WTN + fn * 32 + acc_col4(vg, lane)) >> 2;
            store4<OutT>((OutT*)(stage + ST::quad(r, c4)), acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1],
                         acc[fm][fn][vg * 4 + 2], acc[fm][fn][vg * 4 + 3]);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[fm][fn][vg * 4 + v] = 0.f;
          }
      }
      __syncthreads();   // tile staged
    }
  };
  T* As0 = lds;
  T* As1 = lds + C::A_ELEMS;
  T* Bs0 = lds + 2 * C::A_ELEMS;
  T* Bs1 = Bs0 + C::B_ELEMS;
  issue(Set<0>{});
  issue(Set<1>{});
  al.template store<0>(As0);
  bl.template store<0>(Bs0);
  __syncthreads();   // prologue
  // The step count is padded to even, so the loop has no exit between its
  // two halves and every half stores its register set to LDS (a branch
  // around those stores, or an exit between them, makes the compiler wait for
  // all loads at the loop head).  A padding step multiplies into accumulators
  // that are never staged.
  for (int st = 0; st < total_even; st += 2) {
    // even step: LDS buffer 0 holds this step, register set 1 the next one
    issue(Set<0>{});
    mma_tile<C, kNLayout<C>, kNLayout<C>>(As0, Bs0, acc);
    al.template store<1>(As1);
    bl.template store<1>(Bs1);
    __syncthreads();   // step done
    finish_step(st);
    next_step();
    // odd step: LDS buffer 1 holds this step, register set 0 the next one
    issue(Set<1>{});
    mma_tile<C, kNLayout<C>, kNLayout<C>>(As1, Bs1, acc);
    al.template store<0>(As0);
    bl.template store<0>(Bs0);
    __syncthreads();   // step done
    finish_step(st + 1);
    next_step();
  }
}

// ------------------------------------------------ weight gradients, resident
// Experts with at most KMAX positions, bf16 operands, bf16 or fp32 gradients.  The
// product dW[e] = A_e^T B_e (M x N) contracts over the expert's c <= KMAX
// positions, so each dW element carries only 2c flops and the kernel's work
// is mostly writing dW.  The tiled kernel reloads both operands for every
// 128 x 128 output tile and stages the tile through LDS, which moves several
// times more LDS bytes than the tile writes to HBM.  Here:
// * A work item is (expert, 256-column block of N).  Each of the 4 MMA waves
//   owns 64 of the columns and reads B_e for them x all c positions into
//   registers once per item: the resident operand, up to KMAX/2 bf16 per
//   lane per 32 columns.  B_e arrives as four 64-column LDS slices, one per
//   wave.
// * The item then sweeps M in 64-row steps.  The A_e tile (c positions x 64
//   rows of M) is stored as [k][64] rows with a transposing-read swizzle, in
//   one of two LDS buffers, while the MMA waves multiply the other (64 x 64
//   of dW per wave).  There is one barrier per tile.
// * Two groups of two loader waves take alternate tiles.  A group issues a
//   tile's loads two barrier intervals before the tile is due.  Loaders only
//   load and MMA waves only store, so neither waits on the other's memory
//   counter.
// * For bf16 gradients the MMA waves round the accumulators
//   (v_cvt_pk_bf16_f32), swap half-rows between the half-waves
//   (v_permlane32_swap) and stage the 64 x 64 block in wave-private LDS (two
//   buffers); fp32 accumulators are staged as they are (one buffer).  In the
//   next step they store the block as whole row segments (128 bytes bf16, 256
//   fp32), non-temporal, one store per k-slice, so the store stream drains
//   while the matrix cores work.  A store straight from the accumulator layout
//   touches 32 cache lines per instruction.
// * An expert without positions gets zeros, written before any operand is
//   resident.
// Items of one expert go to one XCD, dealt to its workgroups in order, so the
// workgroups of an XCD sweep the same A_e tiles at about the same time and
// share them in L2.
constexpr int kResThreads = 512;   // 4 MMA waves + 4 loader waves

// Workgroup barrier that orders LDS only: the wave's LDS operations complete,
// then s_barrier.  __syncthreads() also waits for the wave's global stores,
// which would hold the MMA waves at every barrier until their dW stores of
// the previous step are acknowledged.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
constexpr int kResN = 256;   // N columns per item (64 per MMA wave)
constexpr int kResM = 64;    // M rows per step

struct ResItem {
  int e, off, cnt, nkk, n0;
};

template <int KMAX>
struct ResList {
  const WgradTables* tab;
  int first, nx, nnb, count, x, K;
  __device__ __forceinline__ void init(const GArgs& g, const WgradTables* t, int N) {
    tab = t;
    int l = 0, h = g.E;   // first = experts (descending count) with more than KMAX positions
    while (l < h) {
      const int mid = (l + h) >> 1;
      const int e = tab->order[mid];
      if (tab->offsets[e + 1] - tab->offsets[e] > KMAX) l = mid + 1; else h = mid;
    }
    first = l;
    x = blockIdx.x & 7;
    K = gridDim.x >> 3;
    const int nsmall = g.E - first;
    nx = nsmall > x ? (nsmall - x + 7) / 8 : 0;   // experts first + x + 8q of this XCD
    nnb = (N + kResN - 1) / kResN;
    count = nx * nnb;
  }
  __device__ __forceinline__ ResItem item(int i) const {
    const int q = i / nnb;
    ResItem it;   // wave-uniform (the tables are read from LDS)
    it.e = __builtin_amdgcn_readfirstlane(tab->order[first + x + 8 * q]);
    it.off = __builtin_amdgcn_readfirstlane(tab->offsets[it.e]);
    it.cnt = __builtin_amdgcn_readfirstlane(tab->offsets[it.e + 1]) - it.off;
    it.nkk = (it.cnt + 15) >> 4;
    it.n0 = (i - q * nnb) * kResN;
    return it;
  }
};

// [k][64] bf16 operand tiles: 128-byte k-rows whose 16-byte chunks are XOR-ed
// with 4*((k/2 ^ k/8)%2).  A transposing fragment read takes k-rows
// k0..k0+3 (lanes 0-31) and k0+8..k0+11 (lanes 32-63), 64 bytes each: the
// k/2 term separates rows k0 and k0+2 within a 256-byte bank window, the k/8
// term rows k0 and k0+8 within a 512-byte one.
__device__ __forceinline__ int res_lds_off(int kr, int ch) {
  return kr * 128 + ((ch ^ ((((kr >> 1) ^ (kr >> 3)) & 1) << 2)) << 4);
}

// 32 columns (cb .. cb+31) x 16 k of a [k][64] tile: lane -> column cb + lane%32,
// k = kk*16 + 8*(lane/32) + 0..7 (the K-contiguous fragment layout).
__device__ __forceinline__ bf16x8_t frag_k64(const char* tile, int cb, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = cb + ((g & 1) << 4) + ((s & 3) << 2);
  const int chunk = col >> 3, within = (col & 7) * 2;
  const lds_char* base = (const lds_char*)tile;
  s16x4_t r[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = kk * 16 + ((g >> 1) << 3) + h * 4 + (s >> 2);
    r[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + res_lds_off(krow, chunk) + within));
  }
  bf16x8_t out;
  s16x4_t* o = (s16x4_t*)&out;
  o[0] = r[0];
  o[1] = r[1];
  return out;
}

// OutT: bf16 (uint16_t) or fp32 gradients.
template <bool GATE_UP, typename OutT, int KMAX>
__global__ __launch_bounds__(kResThreads, 1) void wgrad_res_kernel(GArgs g) {
  constexpr bool BF = sizeof(OutT) == 2;
  constexpr int NKK = KMAX / 16;
  constexpr int TILE_BYTES = KMAX * kResM * 2;
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * TILE_BYTES];
  __shared__ WgradTables tab;
  // Per MMA wave, the staging rows that re-tile a step's 64 x 64 accumulator
  // block into whole row segments: two buffers of 64 rows x 128 bytes for
  // bf16, one of 64 x 256 bytes for fp32.  One buffer suffices because a
  // block's stores are all issued before the next block is staged; the bf16
  // path keeps its measured two-buffer form.
  constexpr int SROW = 64 * (int)sizeof(OutT), CPRS = SROW / 16;   // bytes, chunks per staged row
  constexpr int STAGE_BUF = 64 * SROW, STAGE_WAVE = BF ? 2 * STAGE_BUF : STAGE_BUF;
  __shared__ __attribute__((aligned(16))) char stage_raw[4 * STAGE_WAVE];
  const int H = g.H, I = g.I;
  const int M = GATE_UP ? 2 * I : H, N = GATE_UP ? H : I;
  const int lda = M, ldb = N;   // GATE_UP: dZ [S,2I], Xp [S,H]; else dYp [S,H], aw [S,I]
  for (int i = threadIdx.x; i <= g.E; i += kResThreads) {
    if (i < g.E) tab.order[i] = g.expert_order[i];
    tab.offsets[i] = g.offsets[i];
  }
  __syncthreads();
  ResList<KMAX> list;
  list.init(g, &tab, N);
  const int ntm = (M + kResM - 1) / kResM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w0 = blockIdx.x >> 3;

  // Tiles of this workgroup: items with positions in list order; per item
  // 4 B tiles (the 64-column slices of the item's B block, one per MMA
  // wave), then its ntm A tiles.
  int total = 0;
  for (int i = w0; i < list.count; i += list.K) {
    const int c = list.item(i).cnt;
    total += c > 0 ? ntm + 4 : 0;
  }
  if (wave >= 4) {
    // ---------------- loader waves
    // Two groups of two waves take alternate tiles, so a group issues the
    // loads of its next tile two barrier intervals before that tile is due
    // (one register set per group; a wave waits only for its own loads).
    const int grp = (wave - 4) >> 1;
    const int t = threadIdx.x - 256 - 128 * grp;
    const int ch = t & 7, kr0 = t >> 3;   // 16-byte chunk of the row; rows kr0 + 16 r
    const uint16_t* Ag = (const uint16_t*)g.A;
    const uint16_t* Bg = (const uint16_t*)g.B;
    uint4 reg[NKK];
    uint32_t okm = 0;
    int rounds = 0;
    // cursor: tile u of item i (u < 4: B columns n0 + 64u.., else A rows (u-4)*64..)
    int i = w0, u = 0;
    ResItem it;
    auto settle = [&]() {   // move to the first tile at or after (i, u)
      while (i < list.count) {
        it = list.item(i);
        if (it.cnt > 0 && u < ntm + 4) return;
        i += list.K;
        u = 0;
      }
    };
    auto advance = [&]() { ++u; settle(); };
    auto load = [&]() {
      const uint16_t* src;
      int ld, cols;
      if (u < 4) {
        cols = N - (it.n0 + 64 * u);
        src = Bg + (size_t)it.off * ldb + (cols > 0 ? it.n0 + 64 * u : 0);
        ld = ldb;
      } else {
        cols = M - (u - 4) * kResM;
        src = Ag + (size_t)it.off * lda + (u - 4) * kResM;
        ld = lda;
      }
      const bool col_ok = ch * 8 < cols;
      rounds = it.nkk;
      okm = 0;
#pragma unroll
      for (int r = 0; r < NKK; ++r) {
        if (r < rounds) {
          const int kr = kr0 + 16 * r;
          const bool ok = col_ok && kr < it.cnt;
          okm |= (uint32_t)ok << r;
          reg[r] = *(const uint4*)(src + (ok ? (size_t)kr * ld + ch * 8 : 0));
        }
      }
    };
    auto store = [&](char* buf) {
#pragma unroll
      for (int r = 0; r < NKK; ++r)
        if (r < rounds) *(uint4*)(buf + res_lds_off(kr0 + 16 * r, ch)) = masked(reg[r], (okm >> r) & 1);
    };
    settle();
    if (grp == 1) advance();
    if (grp < total) load();
    for (int tile = 0; tile < total; ++tile) {
      if ((tile & 1) == grp) {
        store(smem_raw + (tile & 1) * TILE_BYTES);
        advance();
        advance();
        if (tile + 2 < total) load();
      }
      lds_barrier();   // tile ready (and the buffer it replaced consumed)
    }
    return;
  }

  // ---------------- MMA waves
  const int lane = threadIdx.x & 63;
  OutT* dW = (OutT*)g.out0;
  char* stage = stage_raw + wave * STAGE_WAVE;
  // byte offset of 16-byte chunk c of staging row r: chunks XOR-ed with
  // (r/2 ^ r/16)%8 for 128-byte rows, (r ^ r/16)%16 for 256-byte rows, so one
  // chunk of 32 consecutive rows (a half-wave's write) and whole rows (the
  // reads) spread over distinct 16-byte bank groups whether banks repeat
  // every 256 or every 512 bytes
  auto stage_off = [](int r, int c) {
    if constexpr (BF) return r * 128 + ((c ^ (((r >> 1) ^ (r >> 4)) & 7)) << 4);
    else return r * 256 + ((c ^ ((r ^ (r >> 4)) & 15)) << 4);
  };
  bf16x8_t bres[2][NKK];
  f32x16 acc[2][2];
  auto row_ptr = [&](int e, int m) -> OutT* {
    if (GATE_UP && g.gu_sep) {   // separate dW_gate, dW_up: row m is a dZ column
      int up, jj;
      zcol(m, I, g.layout, up, jj);
      return gu_row((OutT*)g.dgu_g, (OutT*)g.dgu_u, g.gu_es, g.gu_rs, e, up, jj);
    }
    return dW + ((size_t)e * M + m) * N;
  };
  // The 64 x 64 accumulator block of a step is rounded to bf16 and written to
  // the wave's staging rows (two buffers of 2 x 32 rows x 128 bytes); its
  // global stores are issued one per k-slice during the next step's MFMAs, so
  // the store stream drains while the matrix cores work instead of in a
  // burst that stalls the wave.
  auto stage_acc = [&](char* st) {
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const f32x16& a = acc[fm][fn];
        const int r = fm * 32 + (lane & 31);
        if constexpr (BF) {
          // Register groups 2p and 2p+1 hold columns 16p + 4h + 0..3 and
          // 16p + 8 + 4h + 0..3 (h = lane / 32).  Swapping group 2p+1 of the
          // lower half-wave with group 2p of the upper one gives lane h 8
          // consecutive columns 16p + 8h + 0..7 (16-byte chunk 4fn + 2p + h
          // of the row).
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const uint32_t p0 = pack_bf16(a[8 * p], a[8 * p + 1]);
            const uint32_t p1 = pack_bf16(a[8 * p + 2], a[8 * p + 3]);
            const uint32_t q0 = pack_bf16(a[8 * p + 4], a[8 * p + 5]);
            const uint32_t q1 = pack_bf16(a[8 * p + 6], a[8 * p + 7]);
            const auto s0 = __builtin_amdgcn_permlane32_swap(p0, q0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(p1, q1, false, false);
            const int c = 4 * fn + 2 * p + (lane >> 5);
            *(uint4*)(st + stage_off(r, c)) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
          }
        } else {
          // register group vg: columns 8vg + 4h + 0..3, chunk 8fn + 2vg + h
#pragma unroll
          for (int vg = 0; vg < 4; ++vg) {
            const int c = 8 * fn + 2 * vg + (lane >> 5);
            *(float4*)(st + stage_off(r, c)) = make_float4(a[4 * vg], a[4 * vg + 1], a[4 * vg + 2], a[4 * vg + 3]);
          }
        }
      }
  };

  // Pending staged block: rows pj*64.., columns pn0 + wave*64.. of expert pe.
  int pe = 0, pj = 0, pn0 = 0;
  bool pending = false;
  const char* pst = stage;
  // Store q (0..NQ-1) of the pending block: RPI staged rows, CPRS lanes per
  // row, one whole row segment (128 bytes bf16, 256 fp32) each, non-temporal
  // (dW is not read again here, so it need not displace the operand tiles in
  // L2).  The lane's row pointer and bounds are formed once per block (pbase:
  // row pj*64 + lane / CPRS at the lane's column; rows q RPI further on are
  // N elements apart), so a store costs one address add; separate gate / up
  // tensors map each row on its own.
  constexpr int RPI = 64 / CPRS, NQ = 64 / RPI, VPC = 16 / (int)sizeof(OutT);
  constexpr int NQI = NQ < 8 ? NQ : 8;   // stores issued between k-slices; the rest after them
  OutT* pbase = dW;
  int prows = 0;   // rows of the pending block from the lane's first row to M, 0 if its column is past N
  auto set_pending = [&](int e, int j, int n0) {
    const int r0 = lane / CPRS, n = n0 + wave * 64 + (lane % CPRS) * VPC;
    pe = e; pj = j; pn0 = n0;
    prows = n < N ? M - (j * kResM + r0) : 0;
    pbase = dW + ((size_t)e * M + j * kResM + r0) * N + n;
  };
  auto store_step = [&](int q) {
    const int r = q * RPI + lane / CPRS, c = lane % CPRS;
    const uint4 v = *(const uint4*)(pst + stage_off(r, c));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if (q * RPI < prows) {
      OutT* dst = pbase + (size_t)q * RPI * N;
      if (GATE_UP && g.gu_sep) dst = row_ptr(pe, pj * kResM + r) + pn0 + wave * 64 + c * VPC;
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)dst);
    }
  };
  // Experts without positions first (zeros in whole 16-byte chunks, no LDS),
  // while no resident operand is live.
  for (int i = w0; i < list.count; i += list.K) {
    const ResItem it = list.item(i);
    if (it.cnt != 0) continue;
    constexpr int VPC0 = 16 / (int)sizeof(OutT), CPR = kResN / VPC0;   // 16-byte chunks per row of the item
    const int c = (threadIdx.x % CPR) * VPC0;
    if (c < N - it.n0)
      for (int m = threadIdx.x / CPR; m < M; m += 256 / CPR)
        *(uint4*)(row_ptr(it.e, m) + it.n0 + c) = make_uint4(0u, 0u, 0u, 0u);
  }
  int tile = 0;
  for (int i = w0; i < list.count; i += list.K) {
    const ResItem it = list.item(i);
    if (it.cnt == 0) continue;
    // B slices: wave q reads its 64 columns when slice q is in LDS
#pragma unroll
    for (int q = 0; q < 4; ++q, ++tile) {
      lds_barrier();   // B slice q ready
      if (wave == q) {
        const char* buf = smem_raw + (tile & 1) * TILE_BYTES;
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
            if (kk < it.nkk) bres[fn][kk] = frag_k64(buf, fn * 32, kk, lane);
      }
    }
    for (int j = 0; j < ntm; ++j, ++tile) {
      lds_barrier();   // A tile j ready
      const char* buf = smem_raw + (tile & 1) * TILE_BYTES;
      bf16x8_t a[2][2];
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) a[0][fm] = frag_k64(buf, fm * 32, 0, lane);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk < it.nkk) {
          if (kk + 1 < it.nkk) {
#pragma unroll
            for (int fm = 0; fm < 2; ++fm) a[(kk + 1) & 1][fm] = frag_k64(buf, fm * 32, kk + 1, lane);
          }
#pragma unroll
          for (int fm = 0; fm < 2; ++fm)
#pragma unroll
            for (int fn = 0; fn < 2; ++fn)
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bres[fn][kk], a[kk & 1][fm],
                                                                     kk == 0 ? f32x16{} : acc[fm][fn], 0, 0, 0);
          if (kk < NQI && pending) store_step(kk);
        }
      }
      if (pending)
        for (int q = min(it.nkk, NQI); q < NQ; ++q) store_step(q);
      // stage this step's block (bf16: in the other buffer); it is stored during the next step
      char* st = stage + (BF && pst == stage ? STAGE_BUF : 0);
      stage_acc(st);
      pst = st;
      set_pending(it.e, j, it.n0);
      pending = true;
    }
  }
  if (pending)
    for (int q = 0; q < NQ; ++q) store_step(q);
}

// ------------------------------------------------ weight gradients, long K
// Experts with more than hot_min positions (bf16 operands).  Their K loop
// (the expert's positions) runs to thousands, so dW[e] = A_e^T B_e is a plain
// long-K GEMM whose stores are a small share of the time: 256 x 128 tiles on
// the token-row engine's two-set pipeline (8 waves of 64 x 64, one workgroup
// per CU), both operands position-major and read with transposing LDS reads
// (B as one [k][128] tile, A as two; 128 x 128 tiles at two workgroups per
// CU were 6 % slower).  A persistent grid deals chunks of 32 tiles
// round-robin to the XCDs, so each XCD gets a share of every expert (one hot
// expert can hold a fifth of all positions; contiguous ranges per XCD left
// one XCD with a third of the work, 2x slower).  Inside an expert, groups of
// 8 M-tiles run N-tile by N-tile, so a chunk's tiles share 4 B row blocks
// and 8 A row blocks in one L2.  The tiled kernel, built
// around short K loops and the dW store stream, took these experts at ~550
// TFLOP/s.
// 256 x 128 tiles on 8 waves (64 x 64 each), one workgroup per CU; the A
// tile (256 columns of M) is two [k][128] halves.
struct CfgL : Cfg<uint16_t, 256, 128, 64, 4, 2> {};
template <> struct WideA<CfgL> { static constexpr bool value = true; };

// Two NLoaders for the two 128-column halves of a 256-column A tile.
template <class C>
struct NLoaderWide {
  using T = typename C::elem;
  NLoader<C, 0> h0;
  NLoader<C, C::NT / 2> h1;
  static constexpr int NI = 2 * NLoader<C, 0>::NI;
  static constexpr int WRITES = NI;
  __device__ __forceinline__ void init(int mn_valid, int kvalid) {
    h0.init(mn_valid, kvalid);
    h1.init(mn_valid - 128, kvalid);
  }
  template <int SET>
  __device__ __forceinline__ void store(T* lds) {
    h0.template store<SET>(lds);
    h1.template store<SET>(lds + 128 * C::BK);
  }
};

template <class C, bool GATE_UP, typename OutT>
__global__ __launch_bounds__(C::NT, C::OCC) void wgrad_long_kernel(GArgs g) {
  GEMM_PROLOGUE(C)
  static_assert(C::BM == 256 && C::BN == 128 && WideA<C>::value, "A: two [k][128] halves; B: [k][128]");
  const int I = g.I, H = g.H;
  const int M = GATE_UP ? 2 * I : H, N = GATE_UP ? H : I;
  const int lda = M, ldb = N;   // GATE_UP: dZ [S,2I], Xp [S,H]; else dYp [S,H], aw [S,I]
  int l = 0, h = g.E;           // nhot = leading experts with more than hot_min positions
  {                             // none (the host cannot tell without a sync): leave at once
    const int e0 = g.expert_order[0];
    if (g.offsets[e0 + 1] - g.offsets[e0] <= g.hot_min) return;
  }
  while (l < h) {
    const int mid = (l + h) >> 1;
    const int e = g.expert_order[mid];
    if (g.offsets[e + 1] - g.offsets[e] > g.hot_min) l = mid + 1; else h = mid;
  }
  const int ntm = g.ntm, ntn = g.ntn, per_e = ntm * ntn;
  const int total = l * per_e;
  const int K = gridDim.x >> 3;
  const T* Ag = (const T*)g.A;
  const T* Bg = (const T*)g.B;
  OutT* dW = (OutT*)g.out0;
  // this XCD's j-th tile: chunks of 32 consecutive tiles (an XCD's 32
  // workgroups; 4 N-tiles of one group of 8 M-tiles) dealt round-robin to
  // the XCDs, increasing in j, so the first one past the end ends the loop.
  // Chunks of 8 tiles: gate_up 4.52 against 4.30-4.35 ms on the Zipf batch.
  for (int j = blockIdx.x >> 3;; j += K) {
    const int t = dealt_tile<32>(j, total);
    if (t < 0) break;
    const int er = t / per_e, local = t - er * per_e;
    const int e = g.expert_order[er];
    const int off = g.offsets[e], cnt = g.offsets[e + 1] - off;   // cnt > hot_min > 0
    const int gsz = kRowTileGroup * ntn;
    const int grp = local / gsz, rem = local - grp * gsz;
    const int gm = min(kRowTileGroup, ntm - grp * kRowTileGroup);
    const int nt = rem / gm, mt = grp * kRowTileGroup + (rem - nt * gm);
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    NLoaderWide<C> al;
    NLoader<C, C::NT / 4> bl;
    al.init(M - m0, cnt);
    bl.init(N - n0, cnt);
    const T* Ap = Ag + (size_t)off * lda + m0;
    const T* Ap1 = Ap + (M - m0 > 128 ? 128 : 0);   // second half (in range even when it is all masked)
    const T* Bp = Bg + (size_t)off * ldb + n0;
    auto aload = [&](auto& ld, int kt, auto set) {
      constexpr int SET = decltype(set)::value;
      ld.h0.template load<SET>(kt, [&](int k) { return Ap + (size_t)k * lda; });
      ld.h1.template load<SET>(kt, [&](int k) { return Ap1 + (size_t)k * lda; });
    };
    auto bload = [&](auto& ld, int kt, auto set) {
      ld.template load<decltype(set)::value>(kt, [&](int k) { return Bp + (size_t)k * ldb; });
    };
    f32x16 acc[C::FM][C::FN];
    mainloop<C, true, true>(al, bl, aload, bload, (cnt + C::BK - 1) / C::BK, lds, acc);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int m = m0 + wm * C::WTM + fm * 32 + (lane & 31);
      if (m >= M) continue;
      OutT* row;
      if (GATE_UP && g.gu_sep) {   // separate dW_gate, dW_up: row m is a dZ column
        int up, jj;
        zcol(m, I, g.layout, up, jj);
        row = gu_row((OutT*)g.dgu_g, (OutT*)g.dgu_u, g.gu_es, g.gu_rs, e, up, jj);
      } else {
        row = dW + ((size_t)e * M + m) * N;
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int n = n0 + wn * C::WTN + fn * 32 + acc_col4(vg, lane);
          if (n < N)
            store4<OutT>(row + n, acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1], acc[fm][fn][vg * 4 + 2],
                         acc[fm][fn][vg * 4 + 3]);
        }
    }
  }
}

// ------------------------------------------------------------------ host side
using CfgB = Cfg<uint16_t, 128, 128, 64, 2, 2>;   // bf16
// bf16 with 192-row M-tiles (96 rows per wave): when experts average a little
// over 128 positions, 128-row tiles leave a mostly empty second tile per
// expert that repeats the whole weight stream; one 192-row tile covers them.
// Not where the LDS-DMA engine takes the small experts (H and I multiples
// of 64): its 128-row tiles, with the experts of 129-256 slots on the
// 256-row tiles, measured faster on the large layer (step 20.55 -> 19.72 ms)
// and 0.7 % slower on the gpt-oss one.
using CfgB192 = Cfg<uint16_t, 192, 128, 64, 2, 2>;
static bool use_bm192(const GemmProblem& pb) {
  const long mean = pb.E > 0 ? (long)pb.S / pb.E : 0;
  return pb.dtype == 0 && mean > 100 && mean <= 176 && !dma_small_enabled(pb);
}
int small_tile_rows(const GemmProblem& pb) { return use_bm192(pb) ? 192 : 128; }
// bf16 with 256x128 tiles on 8 waves (64x64 each, one workgroup per CU):
// when experts average several hundred positions, a quarter fewer operand
// bytes per flop from L2 than 128x128 tiles (Zipf workload: gate_up 6.42 ->
// 6.24 ms, down 3.09 -> 2.97, gate_up_dgrad 6.32 -> 5.96).  The same tile on
// 4 waves of 128x64 was slower: with one wave per SIMD nothing covers a
// step's barrier and first LDS reads.
using CfgB256 = Cfg<uint16_t, 256, 128, 64, 4, 2>;
static bool use_bm256(const GemmProblem& pb) {
  const long mean = pb.E > 0 ? (long)pb.S / pb.E : 0;
  return pb.dtype == 0 && mean >= 320;
}
using CfgF = Cfg<float, 128, 128, 32, 2, 2>;      // fp32
using CfgBW = Cfg<uint16_t, 128, 256, 64, 2, 4>;  // bf16, 128 x 256 on 8 waves
// weight gradients (one persistent workgroup per CU: operands, staging tile and tables in LDS)
using CfgWB = Cfg<uint16_t, 128, 128, 64, 2, 4>;
// bf16 gradients of the tiled kernel: 256 x 128 tiles (8 waves of 64 x 64,
// BK = 32 to leave LDS for the 64 KB staging tile), the 256 columns of M
// held as two [k][128] halves: a quarter fewer operand bytes per flop than
// 128 x 128.
struct CfgWB256 : Cfg<uint16_t, 256, 128, 32, 4, 2> {};
template <> struct WideA<CfgWB256> { static constexpr bool value = true; };
using CfgWF = Cfg<float, 128, 128, 16, 2, 2>;

template <class C, bool A, bool Z>
static hipError_t gate_up_impl(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                               hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = X; g.B = Wgu; g.out0 = a_out; g.out1 = z_out;
  set_gu(g, pb, Wgu, nullptr, 0);
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

// With the large-tile engine on, a token-row GEMM runs as two launches: the
// large-tile experts (large_tile_expert) in 256 x 256 tiles (gemm_dma.hip),
// then the others in this engine's 128 x 256 tiles (192 x 128 when experts
// average 101-176 slots), each over its own tile table.
static GemmProblem small_experts(const GemmProblem& pb) {
  GemmProblem p = pb;
  p.tile_set = 2;
  return p;
}

hipError_t launch_gate_up(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                          hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  if (pb.dtype != 0) return gate_up_dispatch<CfgF>(pb, X, Wgu, a_out, z_out, s);
  if (dma_enabled(pb)) {
    const hipError_t e = dma_gate_up(pb, X, Wgu, a_out, z_out, s);
    if (e != hipSuccess) return e;
    const GemmProblem ps = small_experts(pb);
    if (use_bm192(pb)) return gate_up_dispatch<CfgB192>(ps, X, Wgu, a_out, z_out, s);
    return dma_small_enabled(pb) ? dma_gate_up_small(ps, X, Wgu, a_out, z_out, s)
                                 : gate_up_dispatch<CfgBW>(ps, X, Wgu, a_out, z_out, s);
  }
  if (use_bm256(pb)) return gate_up_dispatch<CfgB256>(pb, X, Wgu, a_out, z_out, s);
  return use_bm192(pb) ? gate_up_dispatch<CfgB192>(pb, X, Wgu, a_out, z_out, s)
                       : gate_up_dispatch<CfgB>(pb, X, Wgu, a_out, z_out, s);
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
  if (pb.dtype != 0) return down_impl<CfgF>(pb, a, Wd, Yp, s);
  if (dma_enabled(pb)) {
    const hipError_t e = dma_down(pb, a, Wd, Yp, s);
    if (e != hipSuccess) return e;
    const GemmProblem ps = small_experts(pb);
    if (use_bm192(pb)) return down_impl<CfgB192>(ps, a, Wd, Yp, s);
    return dma_small_enabled(pb) ? dma_down_small(ps, a, Wd, Yp, s) : down_impl<CfgBW>(ps, a, Wd, Yp, s);
  }
  if (use_bm256(pb)) return down_impl<CfgB256>(pb, a, Wd, Yp, s);
  return use_bm192(pb) ? down_impl<CfgB192>(pb, a, Wd, Yp, s) : down_impl<CfgB>(pb, a, Wd, Yp, s);
}

// Routing-weight partials of the down dgrad: one per 128 columns of I, for
// every tile width (a 256-column tile writes two).
int down_dgrad_nparts(int I) { return (I + 127) / 128; }

template <class C>
static hipError_t down_dgrad_impl(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ,
                                  void* aw, float* partials, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = dY; g.B = Wd; g.Z = Z; g.out0 = dZ; g.out1 = aw; g.partials = partials;
  g.ntn = (pb.I + C::BN - 1) / C::BN;
  g.nparts = down_dgrad_nparts(pb.I);   // one partial per 128 columns, BN / 128 per tile
  const long grid = row_grid(pb, C::BM, g.ntn);
  return run_kernel("down_dgrad_glu_bwd", s, [&] { down_dgrad_kernel<C><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t launch_down_dgrad(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ,
                             void* aw, float* partials, int* nparts, hipStream_t s) {
  *nparts = down_dgrad_nparts(pb.I);
  if (pb.S == 0) return hipSuccess;
  // 192-row tiles when experts average 101-176 positions (gpt-oss layer
  // 0.78 -> 0.71 ms); 256-row tiles for larger experts measured slower here
  // (Zipf batch 3.99 -> 4.04 ms), so those keep 128 rows.
  if (pb.dtype != 0) return down_dgrad_impl<CfgF>(pb, dY, Wd, Z, dZ, aw, partials, s);
  if (dma_enabled(pb)) {
    const hipError_t e = dma_down_dgrad(pb, dY, Wd, Z, dZ, aw, partials, *nparts, s);
    if (e != hipSuccess) return e;
    const GemmProblem ps = small_experts(pb);
    if (use_bm192(pb)) return down_dgrad_impl<CfgB192>(ps, dY, Wd, Z, dZ, aw, partials, s);
    return dma_small_enabled(pb) ? dma_down_dgrad_small(ps, dY, Wd, Z, dZ, aw, partials, down_dgrad_nparts(pb.I), s)
                                 : down_dgrad_impl<CfgBW>(ps, dY, Wd, Z, dZ, aw, partials, s);
  }
  return use_bm192(pb) ? down_dgrad_impl<CfgB192>(pb, dY, Wd, Z, dZ, aw, partials, s)
                       : down_dgrad_impl<CfgB>(pb, dY, Wd, Z, dZ, aw, partials, s);
}

template <class C>
static hipError_t gate_up_dgrad_impl(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp,
                                     hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = dZ; g.B = Wgu; g.out0 = dXp;
  set_gu(g, pb, Wgu, nullptr, 0);
  g.ntn = (pb.H + C::BN - 1) / C::BN;
  const long grid = row_grid(pb, C::BM, g.ntn);
  return run_kernel("gate_up_dgrad", s, [&] {
    if (g.gu_sep) gate_up_dgrad_kernel<C, true><<<grid, C::NT, 0, s>>>(g);
    else gate_up_dgrad_kernel<C, false><<<grid, C::NT, 0, s>>>(g);
  });
}

hipError_t launch_gate_up_dgrad(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp, hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  if (pb.dtype != 0) return gate_up_dgrad_impl<CfgF>(pb, dZ, Wgu, dXp, s);
  if (dma_enabled(pb)) {
    const hipError_t e = dma_gate_up_dgrad(pb, dZ, Wgu, dXp, s);
    if (e != hipSuccess) return e;
    const GemmProblem ps = small_experts(pb);
    if (use_bm192(pb)) return gate_up_dgrad_impl<CfgB192>(ps, dZ, Wgu, dXp, s);
    return dma_small_enabled(pb) ? dma_gate_up_dgrad_small(ps, dZ, Wgu, dXp, s)
                                 : gate_up_dgrad_impl<CfgBW>(ps, dZ, Wgu, dXp, s);
  }
  if (use_bm256(pb)) return gate_up_dgrad_impl<CfgB256>(pb, dZ, Wgu, dXp, s);
  return use_bm192(pb) ? gate_up_dgrad_impl<CfgB192>(pb, dZ, Wgu, dXp, s)
                       : gate_up_dgrad_impl<CfgB>(pb, dZ, Wgu, dXp, s);
}

// Compute units of the current device, looked up once per device (the
// persistent weight-gradient grids hold one workgroup per CU).
constexpr int kMaxDevices = 64;
static std::atomic<int> g_device_cus[kMaxDevices];
static int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 8;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int c = g_device_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 8;
  if (cached) g_device_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <class C, bool GU, typename OutT>
static hipError_t wgrad_impl(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s,
                             int small_max, int hot_min = 0) {
  const int M = GU ? 2 * pb.I : pb.H, N = GU ? pb.H : pb.I;
  if (pb.S == 0) {   // no positions
    if (GU && pb.dw_up) {
      const hipError_t e = launch_fill_zero(dW, (size_t)pb.E * pb.I * N * sizeof(OutT), s);
      return e != hipSuccess ? e : launch_fill_zero(pb.dw_up, (size_t)pb.E * pb.I * N * sizeof(OutT), s);
    }
    return launch_fill_zero(dW, (size_t)pb.E * M * N * sizeof(OutT), s);
  }
  GArgs g = base_args(pb, C::BM);
  g.A = A; g.B = B; g.out0 = dW;
  if (GU) set_gu(g, pb, nullptr, dW, sizeof(OutT));
  g.ntm = (M + C::BM - 1) / C::BM;
  g.ntn = (N + C::BN - 1) / C::BN;
  // split experts: more than twice the mean positions per expert (and more than 4 k-steps)
  const long mean = ((long)pb.S + pb.E - 1) / pb.E;
  g.big = (int)std::max<long>(2 * mean, 4 * C::BK);
  g.small_max = small_max;
  g.hot_min = hot_min;
  // one persistent workgroup per CU, a whole number per XCD
  const int cus = device_cus();
  const long grid = (cus / 8) * 8;
  const char* name = small_max >= 0 ? (GU ? "wgrad_gate_up_hot" : "wgrad_down_hot")
                                    : (GU ? "wgrad_gate_up" : "wgrad_down");
  return run_kernel(name, s, [&] { wgrad_kernel<C, GU, OutT><<<grid, C::NT + kStoreThreads, 0, s>>>(g); });
}

// Experts with at most this many positions take the resident-operand kernel.
constexpr int kResKmax = 240;

template <bool GU, typename OutT>
static hipError_t wgrad_res_impl(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  GArgs g = base_args(pb, 128);
  g.A = A; g.B = B; g.out0 = dW;
  if (GU) set_gu(g, pb, nullptr, dW, sizeof(OutT));
  const int cus = device_cus();
  const long grid = (cus / 8) * 8;
  return run_kernel(GU ? "wgrad_gate_up" : "wgrad_down", s, [&] {
    wgrad_res_kernel<GU, OutT, kResKmax><<<grid, kResThreads, 0, s>>>(g);
  });
}

// Experts with more than kLongMin positions take the register-staged long-K
// kernel (Zipf batch weight gradients: 8.87 ms at 512, 8.95 at 384, 9.16 at
// 1024; at 256 the backward workload's 257-296-position experts were slower
// than on the tiled kernel, 7.34 against 6.15 ms).  Where the large-tile
// engine applies, it takes every expert above kResKmax instead (backward
// workload: 4.89 ms against 5.95 on the tiled kernel for its 241-512-position
// experts; Zipf batch: 6.40 against 6.69 ms for all experts above 240).
constexpr int kLongMin = 512;

template <bool GU, typename OutT>
static hipError_t wgrad_long_impl(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  using C = CfgL;
  const int M = GU ? 2 * pb.I : pb.H, N = GU ? pb.H : pb.I;
  GArgs g = base_args(pb, C::BM);
  g.A = A; g.B = B; g.out0 = dW;
  if (GU) set_gu(g, pb, nullptr, dW, sizeof(OutT));
  g.ntm = (M + C::BM - 1) / C::BM;
  g.ntn = (N + C::BN - 1) / C::BN;
  g.hot_min = kLongMin;
  // persistent: C::OCC workgroups per CU, a whole number per XCD
  const int cus = device_cus();
  const long grid = (cus / 8) * 8 * C::OCC;
  return run_kernel(GU ? "wgrad_gate_up_long" : "wgrad_down_long", s,
                    [&] { wgrad_long_kernel<C, GU, OutT><<<grid, C::NT, 0, s>>>(g); });
}

template <bool GU>
static hipError_t wgrad_dispatch(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  if (pb.dtype == 0 && pb.S > 0) {
    // bf16 operands: experts with at most kResKmax positions (and those
    // without any) on the resident-operand kernel, then the rest: all on the
    // large-tile kernel where it applies, else up to kLongMin on the tiled
    // kernel and above on the long-K one
    const hipError_t e = pb.gdtype == 0 ? wgrad_res_impl<GU, uint16_t>(pb, A, B, dW, s)
                                        : wgrad_res_impl<GU, float>(pb, A, B, dW, s);
    if (e != hipSuccess) return e;
    if (dma_wgrad_enabled(pb)) return dma_wgrad(pb, GU, A, B, dW, kResKmax, s);
    const hipError_t e2 = pb.gdtype == 0 ? wgrad_impl<CfgWB256, GU, uint16_t>(pb, A, B, dW, s, kResKmax, kLongMin)
                                         : wgrad_impl<CfgWB, GU, float>(pb, A, B, dW, s, kResKmax, kLongMin);
    if (e2 != hipSuccess) return e2;
    return pb.gdtype == 0 ? wgrad_long_impl<GU, uint16_t>(pb, A, B, dW, s)
                          : wgrad_long_impl<GU, float>(pb, A, B, dW, s);
  }
  if (pb.dtype == 0)
    return pb.gdtype == 0 ? wgrad_impl<CfgWB, GU, uint16_t>(pb, A, B, dW, s, -1)
                          : wgrad_impl<CfgWB, GU, float>(pb, A, B, dW, s, -1);
  return pb.gdtype == 0 ? wgrad_impl<CfgWF, GU, uint16_t>(pb, A, B, dW, s, -1)
                        : wgrad_impl<CfgWF, GU, float>(pb, A, B, dW, s, -1);
}

hipError_t launch_wgrad_down(const GemmProblem& pb, const void* dY, const void* aw, void* dWd, hipStream_t s) {
  return wgrad_dispatch<false>(pb, dY, aw, dWd, s);
}

hipError_t launch_wgrad_gate_up(const GemmProblem& pb, const void* dZ, const void* X, void* dWgu, hipStream_t s) {
  return wgrad_dispatch<true>(pb, dZ, X, dWgu, s);
}

}  // namespace moe
