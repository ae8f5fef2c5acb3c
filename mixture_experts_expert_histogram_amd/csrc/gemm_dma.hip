// Large-tile engine for the token-row GEMMs and weight gradients of experts
// with many slots.
//
// When an expert holds hundreds to tens of thousands of slots its products
// are dense GEMMs bound by the matrix cores, not by the weight stream.  For
// those experts this engine computes 256 x 256 tiles on 8 waves (2 x 4,
// 128 x 64 per wave) of v_mfma_f32_32x32x16_bf16, with both operands moved
// from global memory straight into LDS by global_load_lds_dwordx4 (no staging
// registers, no ds_write), through a ring of LDS stages: two of BK = 64
// (128 KB) in the token-row kernels when H and I are multiples of 64, five
// of BK = 32 (all 160 KB of LDS) otherwise and in the weight gradients:
//
// * Ping-pong: the two row halves of waves (one wave of each per SIMD) run
//   half a 32-k sub-step apart, so on every SIMD one wave issues MFMAs while
//   the other refills a stage and reads its fragments (pp_step).
// * Every stage starts with a wait for the wave's own loads of that stage
//   (vmcnt; NSTAGE - 2 stages of loads stay in flight) and a plain
//   s_barrier; __syncthreads() would also wait for every load in flight.
// * The stages are distinct __shared__ arrays, the ring is unrolled by its
//   length and every refill is issued unconditionally (clamped to the last
//   stage), so the wait counts are constants.
// * A load writes 64 lanes x 16 bytes to consecutive LDS bytes; the tiles'
//   XOR swizzles come from permuting which 16 bytes of global memory each
//   lane reads (no LDS bank conflicts, measured).
//
// Measured limits (rocprofv3 counters on the Zipf batch): the token-row
// kernels keep the texture data path that feeds LDS 86-94 % busy at about
// half the MFMA rate.  It moves about 17 bytes per clock and CU with 64-byte
// row segments per load (k-contiguous operands at BK = 32) and about 28 with
// 128-byte ones (BK = 64), which is what the 64-k stages are for: the Zipf
// batch's token-row kernels ran 5-8 % faster on them than on the five 32-k
// stages, despite loads issued only one stage ahead.  hipBLASLt reaches
// about 1.35 PFLOP/s on a plain 24576 x 5632 x 2880 product against about
// 1.0 here.
//
// Operands contiguous along k are [row][BK] tiles (16-byte chunks XORed
// with (row / 4) % 4 for 64-byte rows, (row / 2) % 8 for 128-byte ones);
// operands contiguous along m or n (the weights of the input gradients, both
// operands of the weight gradients) are [BK][128] column halves read with
// ds_read_b64_tr_b16, like the other engine's.  K must be a multiple of BK
// (the weight gradients' ragged k is handled by clamped rows and zeroed LDS
// rows).
#include <type_traits>

#include "gemm_common.h"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_vp;

// A pointer made provably wave-uniform (both halves read from lane 0), for
// the scalar base of a load.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from base + off (base wave-uniform, off a per-lane byte
// offset below 2^31) to LDS at dst + 16 * lane (dst wave-uniform).
//
// Written as one asm block (M0 = LDS address, the one wait state an M0 write
// needs before an LDS DMA, the load): the compiler's wait insertion then
// does not track these loads, and the mainloop orders them itself with an
// explicit vmcnt before every barrier and vmcnt(0) at the end.  Tracked, they
// made the compiler wait for every load in flight before each transposing
// LDS read (ds_read_b64_tr_b16 carries no LDS alias information), which
// drained the ring in every step of the input-gradient kernels.  The load
// has no output register; the compiler's own vmcnt waits stay correct
// because vector memory counts complete in order, so untracked loads issued
// after one of its own only make its waits stricter.  The scalar base with a
// 32-bit offset keeps one VGPR per load instead of a 64-bit address.
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, uint16_t* dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_vp)dst;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory", "m0");
}

// BK = 32 or 64 k per stage.  With 64, a k-contiguous operand's load covers
// 8 rows x 128 bytes (whole cache lines) instead of 16 rows x 64 bytes; the
// texture data path that returns the loads to LDS moves about 28 bytes per
// clock and CU with whole lines and about 17 with half lines.  A stage of
// 64 k is consumed in two 32-k sub-steps of the ping-pong schedule.
template <int BM_, int BN_, int WM_, int WN_, int NSTAGE_ = 4, int BK_ = 32>
struct DCfg {
  using elem = uint16_t;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NSTAGE = NSTAGE_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int NBA = BM * BK * 2 / 1024 / NW, NBB = BN * BK * 2 / 1024 / NW;   // 1 KB loads per wave and stage
  static constexpr int PER = NBA + NBB;
  static constexpr int SUB = BK / 32;   // 32-k sub-steps per stage
  static_assert(BK == 32 || BK == 64, "stages of 32 or 64 k");
  static_assert((BM * BK * 2) % (1024 * NW) == 0 && (BN * BK * 2) % (1024 * NW) == 0, "whole 1 KB loads per wave");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "column halves of 128");
};
using DCfgB = DCfg<256, 256, 2, 4, 5>;         // 5 stages of 32 k (160 KB)
using DCfgB64 = DCfg<256, 256, 2, 4, 2, 64>;   // 2 stages of 64 k (128 KB)
using DCfgS = DCfg<128, 256, 2, 4, 3, 64>;     // 3 stages of 64 k (144 KB), 128-row tiles
// The weight gradients: 4 stages of 32 k (128 KB, the least the LDS epilogue
// needs).  Both operands already load whole 256-byte row segments at 32 k; against
// 5 stages the Zipf batch's dW_gate_up took 4.17 ms instead of 4.21 and the
// backward workload's (experts of ~250-500 positions) 3.33 instead of 3.48;
// two 64-k stages were faster only at short k (4.43 on Zipf, 3.23).
using DCfgW = DCfg<256, 256, 2, 4, 4>;

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): vmcnt <= n and lgkmcnt = 0.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Swizzle of a [row][BK] k-contiguous tile: 16-byte chunk c of row r is
// stored at slot c ^ kswz(r), so 16 lanes reading one chunk of 16
// consecutive rows hit 16 bank groups (64-byte rows: (r / 4) % 4; 128-byte
// rows: (r / 2) % 8).
template <int BK>
__device__ __forceinline__ int kswz(int row) { return BK == 32 ? (row >> 2) & 3 : (row >> 1) & 7; }
template <int BK>
__device__ __forceinline__ int krow_off(int row, int chunk) { return row * BK + ((chunk ^ kswz<BK>(row)) << 3); }

// A k-contiguous operand: NB loads per wave per stage, load j of wave w
// holds tile rows (w * NB + j) * RPL .. +RPL (RPL = 16 rows of 64 bytes at
// BK = 32, 8 rows of 128 bytes at BK = 64); lane l reads 16 bytes of row
// RPL b + l / LPR, the chunk whose swizzled slot is l % LPR.  A load's rows
// share one scalar base (rows of one 32-row gate or up group).
template <int NB, int BK = 32>
struct RowSrc {
  static constexpr int LPR = BK / 8, RPL = 64 / LPR;   // lanes per row, rows per load
  const char* base[NB];
  uint32_t off[NB];
  // rowsrc(r, base, off): tile row r (clamped by the caller) starts `off`
  // bytes after `base`, which is the same for the RPL rows of a load
  template <class RowSrcFn>
  __device__ __forceinline__ void init(RowSrcFn rowsrc, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int row = (wave * NB + j) * RPL + lane / LPR;
      const int chunk = (lane % LPR) ^ kswz<BK>(row);
      const char* b;
      uint32_t o;
      rowsrc(row, b, o);
      base[j] = uniform_ptr(b);
      off[j] = o + chunk * 16;
    }
  }
  __device__ __forceinline__ void issue(int kt, uint16_t* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < NB; ++j) lds_dma16(base[j], off[j] + kt * (BK * 2), tile + (wave * NB + j) * 512);
  }
};

// An operand contiguous along m or n (k rows of columns): the tile is
// [BK k][COLS] held as COLS / 128 halves of [BK][128] (256-byte rows, chunks
// XORed with 4 * (k % 4)); with KPH = BK / 4 loads per half, load b covers
// half b / KPH, k rows 4 (b % KPH) .. +4; lane l reads 16 bytes of k row
// 4 (b % KPH) + l / 16.  k rows below ksplit are rows of base0, the others
// rows k - ksplit of base1 (ksplit a multiple of BK, so a stage takes one
// side); ld elements per row; columns past the valid ones are clamped.
//
// CLAMP (the weight gradients, whose k is an expert's positions): k rows
// past kmax read row kmax instead, so the ragged last step stays inside the
// expert's rows; the kernel zeroes what those rows put into LDS where it
// matters (dma_zero_rows).
template <int NB, bool CLAMP = false, int BK = 32>
struct ColSrc {
  static constexpr int KPH = BK / 4;   // loads per 128-column half
  const char* b0;
  const char* b1;
  uint32_t off[NB];   // bytes from a step's first k row to this lane's 16 bytes (no CLAMP)
  uint32_t coff[NB];  // bytes of this lane's 16 bytes within a k row (CLAMP)
  int kr[NB];         // this lane's k row within a step (CLAMP)
  uint32_t row_bytes;
  int ksplit, kmax;
  __device__ __forceinline__ void init(const uint16_t* base0, const uint16_t* base1, long ld, int ksplit_,
                                       int ncols, int c0, int wave, int lane, int kmax_ = 0x7fffffff) {
    b0 = uniform_ptr(base0);
    b1 = uniform_ptr(base1);
    row_bytes = (uint32_t)(ld * 2);
    ksplit = ksplit_;
    kmax = kmax_;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int b = wave * NB + j;
      const int krow = (b % KPH) * 4 + (lane >> 4);
      const int chunk = (lane & 15) ^ ((krow & 3) << 2);
      const int col = min(c0 + (b / KPH) * 128 + chunk * 8, ncols - 8);
      off[j] = krow * row_bytes + col * 2;
      coff[j] = col * 2;
      kr[j] = krow;
    }
  }
  __device__ __forceinline__ void issue(int kt, uint16_t* tile, int wave) const {
    const int k0 = kt * BK;
    if constexpr (CLAMP) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        lds_dma16(b0, (uint32_t)min(k0 + kr[j], kmax) * row_bytes + coff[j], tile + (wave * NB + j) * 512);
    } else {
      const bool lo = k0 < ksplit;
      const char* b = lo ? b0 : b1;
      const uint32_t koff = (uint32_t)(lo ? k0 : k0 - ksplit) * row_bytes;
#pragma unroll
      for (int j = 0; j < NB; ++j) lds_dma16(b, koff + off[j], tile + (wave * NB + j) * 512);
    }
  }
};

// Zero the k rows from kvalid on that this wave's NB loads of a [BK][COLS]
// column-half tile wrote (each lane its own 16 bytes), so rows past an
// expert's last position add nothing.  The wave's own loads must have landed.
template <int NB, int BK>
__device__ __forceinline__ void dma_zero_rows(uint16_t* tile, int kvalid, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int b = wave * NB + j;
    if ((b % (BK / 4)) * 4 + (lane >> 4) >= kvalid) *(uint4*)(tile + b * 512 + lane * 8) = make_uint4(0, 0, 0, 0);
  }
}

// 32 columns x 16 k of a [32][128]-half tile (columns from cb), in the
// fragment layout of the k-contiguous reads: lane -> column cb + lane % 32,
// k = kk * 16 + 8 (lane / 32) + 0..7.
template <int BK>
__device__ __forceinline__ bf16x8_t frag_cols(const uint16_t* tile, int cb, int kk, int lane) {
  tile += (cb >> 7) * (BK * 128);
  cb &= 127;
  const int g = lane >> 4, s = lane & 15;
  const int col = cb + ((g & 1) << 4) + ((s & 3) << 2);
  const int chunk = col >> 3, within = (col & 7) * 2;
  const lds_char* base = (const lds_char*)tile;
  s16x4_t r[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = kk * 16 + ((g >> 1) << 3) + h * 4 + (s >> 2);
    r[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + krow * 256 + ((chunk ^ ((krow & 3) << 2)) << 4) + within));
  }
  bf16x8_t out;
  s16x4_t* o = (s16x4_t*)&out;
  o[0] = r[0];
  o[1] = r[1];
  return out;
}

template <class C>
struct DFrags {
  bf16x8_t a[C::FM], b[C::FN];
};

template <class C, bool A_MN, bool B_MN>
__device__ __forceinline__ void dma_read(const uint16_t* As, const uint16_t* Bs, int kk, DFrags<C>& f, int wm,
                                         int wn, int lane) {
  const int r32 = lane & 31, chunk = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    f.a[i] = A_MN ? frag_cols<C::BK>(As, wm * C::WTM + i * 32, kk, lane)
                  : *(const bf16x8_t*)(As + krow_off<C::BK>(wm * C::WTM + i * 32 + r32, chunk));
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    f.b[j] = B_MN ? frag_cols<C::BK>(Bs, wn * C::WTN + j * 32, kk, lane)
                  : *(const bf16x8_t*)(Bs + krow_off<C::BK>(wn * C::WTN + j * 32 + r32, chunk));
}

template <class C>
__device__ __forceinline__ void dma_mma(const DFrags<C>& f, f32x16 (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Loads of step kt into stage St (A tile, then B tile).
template <class C, class AS, class BS>
__device__ __forceinline__ void dma_issue(const AS& as, const BS& bs, int kt, uint16_t* St, int wave) {
  as.issue(kt, St, wave);
  bs.issue(kt, St + C::A_ELEMS, wave);
}

// Ping-pong schedule of the ring: the two row halves of waves (wm = 0, 1;
// one wave of each on every SIMD) run half a sub-step apart, so that on
// every SIMD one wave issues MFMAs while the other reads fragments and
// issues loads.  A sub-step is 32 k (a stage of 64 k has two).  Every wave
// runs the same sub-step (barrier, refill + reads, barrier, MFMAs); the
// upper half passes one extra barrier first and the lower half one at the
// end, so with barriers A_q, B_q of sub-step q:
//
//   after A_q:  wm = 0 reads sub-step q (refills at a stage's first) | wm = 1 MFMAs of q-1
//   after B_q:  wm = 0 MFMAs of sub-step q                            | wm = 1 reads q (refills ...)
//
// Before the A barrier of a stage's first sub-step every wave's own loads of
// that stage have landed (the lower half waits before it, the upper one
// after its reads of the previous sub-step) and, with a ragged k, its rows
// of A past klast are zeroed.  The stage refilled with stage t+NS-1 was read
// in stage t-1 by both halves, before that barrier (the upper half waits for
// its reads with the same wait).  NS-2 stages of loads stay in flight at
// each wait.
template <class C, bool ZERO>
__device__ __forceinline__ void pp_land(int kt, int last, uint16_t* St, int wave, int lane, int klast) {
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((C::NSTAGE - 2) * C::PER));   // own loads of stage kt landed
  if constexpr (ZERO) {
    if (kt == last && klast < C::BK) {
      asm volatile("" ::: "memory");   // the zeros follow the wait for the loads they overwrite
      dma_zero_rows<C::NBA, C::BK>(St, klast, wave, lane);
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((C::NSTAGE - 2) * C::PER));
    }
  }
}

// Sub-step H of stage kt on stage buffer Sc; at H = 0, Sp (read in stage
// kt-1) is refilled with stage kt+NS-1; Sn holds stage kt+1.
template <class C, bool A_MN, bool B_MN, bool ZERO, int H, class AS, class BS>
__device__ __forceinline__ void pp_step(const AS& as, const BS& bs, int kt, int last, uint16_t* Sc, uint16_t* Sp,
                                        uint16_t* Sn, f32x16 (&acc)[C::FM][C::FN], bool hi, int wave, int wm, int wn,
                                        int lane, int klast, bool idle) {
  if (H == 0 && !hi) pp_land<C, ZERO>(kt, last, Sc, wave, lane, klast);
  // The reads below stay below this barrier and the previous sub-step's
  // MFMAs above it (the compiler does not treat s_barrier as a fence).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();   // lower half: A_q; upper half: B_q
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (H == 0) dma_issue<C>(as, bs, min(kt + C::NSTAGE - 1, last), Sp, wave);
  DFrags<C> f0, f1;
  if (!idle) {
    dma_read<C, A_MN, B_MN>(Sc, Sc + C::A_ELEMS, 2 * H, f0, wm, wn, lane);
    dma_read<C, A_MN, B_MN>(Sc, Sc + C::A_ELEMS, 2 * H + 1, f1, wm, wn, lane);
  }
  if (H == C::SUB - 1 && hi) pp_land<C, ZERO>(kt + 1, last, Sn, wave, lane, klast);
  __builtin_amdgcn_sched_barrier(0);   // no MFMA moves above the barrier
  __builtin_amdgcn_s_barrier();   // lower half: B_q; upper half: A_q+1
  __builtin_amdgcn_sched_barrier(0);
  if (!idle) {
    dma_mma<C>(f0, acc);
    dma_mma<C>(f1, acc);
  }
}

// Every sub-step of stage kt (buffers Sc, Sp, Sn as in pp_step).
template <class C, bool A_MN, bool B_MN, bool ZERO, class AS, class BS>
__device__ __forceinline__ void pp_stage(const AS& as, const BS& bs, int kt, int last, uint16_t* Sc, uint16_t* Sp,
                                         uint16_t* Sn, f32x16 (&acc)[C::FM][C::FN], bool hi, int wave, int wm, int wn,
                                         int lane, int klast, bool idle) {
  pp_step<C, A_MN, B_MN, ZERO, 0>(as, bs, kt, last, Sc, Sp, Sn, acc, hi, wave, wm, wn, lane, klast, idle);
  if constexpr (C::SUB == 2)
    pp_step<C, A_MN, B_MN, ZERO, 1>(as, bs, kt, last, Sc, Sp, Sn, acc, hi, wave, wm, wn, lane, klast, idle);
}

// acc = A . B^T over nk stages of C::BK k; St are the kernel's stage arrays.
// A wave whose whole block lies past the tile's valid rows or columns
// (idle, wave-uniform) still issues its share of the loads and passes every
// barrier but reads no fragments and issues no MFMAs (its accumulators stay
// zero): on the Zipf batch, whose H = I = 2880 leaves 64 valid columns in
// the last 256-wide N tile, the token-row kernels ran 1-1.5 % faster.  The
// weight gradients keep every wave busy (idle there made wgrad_gate_up 3 %
// slower).
// Ends with every wave past its last LDS read and the wave's own loads
// landed.  The last NS - 1 stages still refill stages (with the last stage's
// data, so that the wait counts stay constant): another wave's refill can
// land in a stage after this wave returns, so a workgroup barrier must
// follow before the stages are written for anything else.
template <class C, bool A_MN, bool B_MN, bool ZERO = false, class AS, class BS>
__device__ __forceinline__ void pp_mainloop(const AS& as, const BS& bs, int nk, uint16_t* const (&St)[5],
                                            f32x16 (&acc)[C::FM][C::FN], int wave, int wm, int wn, int lane,
                                            int klast, bool idle) {
  static_assert(C::WM == 2, "two row halves of waves");
  constexpr int NS = C::NSTAGE;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const bool hi = wm == 1;
  const int last = nk - 1;
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) dma_issue<C>(as, bs, min(u, last), St[u], wave);
  if (hi) {   // A_0
    pp_land<C, ZERO>(0, last, St[0], wave, lane, klast);
    __builtin_amdgcn_s_barrier();
  }
  int kt = 0;
  for (; kt + NS <= nk; kt += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      pp_stage<C, A_MN, B_MN, ZERO>(as, bs, kt + u, last, St[u], St[(u + NS - 1) % NS], St[(u + 1) % NS], acc, hi,
                                    wave, wm, wn, lane, klast, idle);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (kt + u < nk)
      pp_stage<C, A_MN, B_MN, ZERO>(as, bs, kt + u, last, St[u], St[(u + NS - 1) % NS], St[(u + 1) % NS], acc, hi,
                                    wave, wm, wn, lane, klast, idle);
  if (!hi) __builtin_amdgcn_s_barrier();   // the upper half's last A barrier
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
}

// Persistent workgroups, one per CU, over the token-row tile order: chunks
// of 32 consecutive tiles (an XCD's 32 workgroups, 4 N-tiles of a group of
// 8 M-tiles) are dealt round-robin to the XCDs, and workgroup b walks
// positions b / 8, b / 8 + gridDim / 8, ... of XCD b % 8's chunks
// (TILE_LOOP).  So the 8 XCDs work on neighbouring chunks of one expert at
// once and miss in their L2s on the same token rows and weight tiles at
// about the same time, which the last-level cache can then serve to all but
// the first; with 8 equal contiguous ranges each XCD streamed its own
// experts (Zipf batch: step 23.15 -> 22.10 ms, the token-row kernels of the
// 256-row tiles 5-9 % faster; chunks of 16 and 64 measured 22.2 and
// 22.55 ms).  A position's
// tile index grows with the position, so the first past the end ends the
// walk.  The barrier between tiles keeps a tile's first loads out of stages
// that slower waves may still be reading for the previous one (its epilogue
// included); every wave's own loads have landed before it.
constexpr int kTileChunk = 32;
template <int BM>
__device__ __forceinline__ bool row_tile_dealt(const GArgs& g, int xcd, int j, int& e, int& m0, int& rows, int& nt) {
  const int t = ((j / kTileChunk) * 8 + xcd) * kTileChunk + j % kTileChunk;
  if (t >= g.tile_prefix[g.E] * g.ntn) return false;
  row_tile_of<BM>(g, t, e, m0, rows, nt);
  return true;
}

#define TILE_LOOP(C)                                                                              \
  int e, m0, rows, nt;                                                                            \
  for (int jt = blockIdx.x >> 3; row_tile_dealt<C::BM>(g, blockIdx.x & 7, jt, e, m0, rows, nt); \
       jt += gridDim.x >> 3)

#define TILE_SYNC()                                        \
  if (jt != (int)(blockIdx.x >> 3)) lds_barrier();

// The stages are consecutive in one LDS array (the epilogue's 32 KB regions
// cross stage boundaries when a stage is 48 KB).
template <class C>
struct alignas(1024) DmaLds {
  uint16_t s[C::NSTAGE * C::STAGE];
};

#define DMA_PROLOGUE(C)                                                                   \
  static_assert(C::NSTAGE >= 2 && C::NSTAGE <= 5, "ring of 2 to 5 stages");                \
  static_assert(sizeof(DmaLds<C>) <= 160 * 1024, "the stages fit in LDS");                \
  __shared__ DmaLds<C> lds;                                                              \
  uint16_t* const St[5] = {lds.s, lds.s + 1 * C::STAGE, lds.s + (C::NSTAGE > 2 ? 2 : 0) * C::STAGE, \
                           lds.s + (C::NSTAGE > 3 ? 3 : 0) * C::STAGE,                    \
                           lds.s + (C::NSTAGE > 4 ? 4 : 0) * C::STAGE};                   \
  const int lane = threadIdx.x & 63;                                                \
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);                \
  const int wm = wave / C::WN, wn = wave % C::WN;

// ---------------------------------------------------------------- epilogues through LDS
// After the mainloop the stages are free (every wave is past its last read):
// the epilogues put the tile's 256 x 256 fp32 results into them in two halves
// of 128 rows (the waves of row half h write theirs: fragment fm into 32 KB
// region fm, 32 rows x 256 columns, 16-byte chunks XORed with row % 16), then
// each wave takes rows 8q + wave of the half (q = 0..15), so that every
// global access moves whole row segments: a store of 64 lanes x 16 bytes
// writes 1 KB of one row (8 cache lines), where the accumulator layout
// spreads a store over 32 rows.  Between the halves and the tiles a barrier
// waits only for LDS (lds_barrier): the previous rows' global stores stay in
// flight.

// Non-temporal stores (whole-row segments written once and not read again by
// the same kernel): the epilogues' outputs stream past L2 instead of evicting
// the operand blocks that the tiles in flight share there.  On the Zipf batch
// the step went 21.88 -> 21.69 ms, the backward workload 15.37 -> 15.08 and
// the gpt-oss layer 5.55 -> 5.35 (its forward, which streams the weights
// once, 1.77 -> 1.63 ms).
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x2_nt __attribute__((ext_vector_type(2)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
template <typename T> __device__ __forceinline__ void store4_nt(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4_nt<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  __builtin_nontemporal_store(u32x2_nt{pack_bf16(a, b), pack_bf16(c, d)}, (u32x2_nt*)p);
}
template <> __device__ __forceinline__ void store4_nt<float>(float* p, float a, float b, float c, float d) {
  __builtin_nontemporal_store(f32x4_nt{a, b, c, d}, (f32x4_nt*)p);
}
// bf16 interleaved pairs (g0 u0 g1 u1 g2 u2 g3 u3), 16 bytes
__device__ __forceinline__ void store4x2_nt_bf16(uint16_t* p, const float* g, const float* u) {
  __builtin_nontemporal_store(u32x4_nt{pack_bf16(g[0], u[0]), pack_bf16(g[1], u[1]), pack_bf16(g[2], u[2]),
                                       pack_bf16(g[3], u[3])},
                              (u32x4_nt*)p);
}

// A workgroup barrier that orders LDS accesses only (global stores in flight
// stay in flight; __syncthreads would wait for them).  The asm statements
// keep the compiler's memory accesses on their side of it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Float index of chunk `chunk` (4 floats) of row `row` of a 32-row region.
__device__ __forceinline__ int epi_chunk(int row, int chunk) { return (row << 8) + ((chunk ^ (row & 15)) << 2); }

template <class C>
__device__ __forceinline__ void epi_r_to_lds(f32x16 (&acc)[C::FM][C::FN], float* const (&st)[4], int wm, int wn,
                                             int lane) {
  static_assert(C::BN == 256 && C::WM == 2 && (C::FM == 4 || C::FM == 2), "128-row passes of 256 columns");
  const int row = lane & 31;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    // rows wm WTM + 32 fm .. +31 of the tile: region (wm FM + fm) % 4 of their pass
    float* const reg = C::FM == 4 ? st[fm] : (wm == 0 ? st[fm] : st[2 + fm]);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int chunk = (wn * C::WTN + fn * 32 + acc_col4(vg, lane)) >> 2;
        *(float4*)(reg + epi_chunk(row, chunk)) =
            make_float4(acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1], acc[fm][fn][vg * 4 + 2], acc[fm][fn][vg * 4 + 3]);
      }
  }
}

// The four 32 KB regions at the start of the stages.
template <class C>
__device__ __forceinline__ void epi_regions(uint16_t* const (&St)[5], float* (&st)[4]) {
  static_assert(C::NSTAGE * C::STAGE * 2 >= 4 * 32768, "four 32 KB regions in the stages");
#pragma unroll
  for (int q = 0; q < 4; ++q) st[q] = (float*)(St[0] + q * 16384);
}

// Routing weights of the tile rows a wave takes in dma_epi_rows, one per lane
// (lane 16 h + q: row 128 h + 8 q + wave), loaded before any epilogue store:
// a load issued after the stores would wait for all of them (vector memory
// counts complete in order).  epi_row_weight reads row tr's back.
__device__ __forceinline__ float epi_row_weights(const float* w_of_pos, int m0, int rows, int wave, int lane) {
  const int tr = ((lane >> 4) & 1) * 128 + (lane & 15) * 8 + wave;
  return w_of_pos[m0 + min(tr, rows - 1)];
}
__device__ __forceinline__ float epi_row_weight(float wl, int tr) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl),
                                                             ((tr >> 7) << 4) + ((tr & 127) >> 3)));
}

// The tile through LDS: row(tr, lr, r) for every tile row tr < rows, with lr
// the row's LDS floats (chunk c at lr + ((c ^ r) << 2), r = tr % 16), called
// by wave tr % 8.
template <class C, class RowFn>
__device__ __forceinline__ void dma_epi_rows(f32x16 (&acc)[C::FM][C::FN], int rows, int wave, int wm, int wn,
                                             int lane, float* const (&st)[4], RowFn row) {
  static_assert(C::NW == 8 && C::WM == 2 && C::BM % 128 == 0, "8 waves over rows 8q + wave of a 128-row pass");
  lds_barrier();   // every wave's loads into the stages have landed (see pp_mainloop)
#pragma unroll
  for (int h = 0; h < C::BM / 128; ++h) {   // 128-row passes: wave half h's rows, or the whole tile
    if (C::BM == 128 || wm == h) epi_r_to_lds<C>(acc, st, wm, wn, lane);
    lds_barrier();
    const int hrows = rows - h * 128;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float* reg = st[qq];
#pragma unroll 2
      for (int q4 = 0; q4 < 4; ++q4) {
        const int hr = (qq * 4 + q4) * 8 + wave;
        if (hr < hrows) row(h * 128 + hr, reg + ((hr & 31) << 8), hr & 15);
      }
    }
    if (h + 1 < C::BM / 128) lds_barrier();   // half 0 read before half 1 overwrites it
  }
}

// ---------------------------------------------------------------- gate_up fwd
// B rows: 32-row groups alternate gate and up rows of the same 32 activation
// columns (see epi_gate_up).
template <class C, bool WRITE_A, bool WRITE_Z, int ACT, int LAYOUT>
__global__ __launch_bounds__(C::NT, 1) void dma_gate_up_kernel(GArgs g) {
  DMA_PROLOGUE(C)
  TILE_LOOP(C) {
    TILE_SYNC()
    const int H = g.H, I = g.I;
    const uint16_t* X = (const uint16_t*)g.A;
    const int j0 = nt * (C::BN / 2);
    const int* tok = g.tok_of_pos;
    RowSrc<C::NBA, C::BK> as;
    RowSrc<C::NBB, C::BK> bs;
    // hidden rows of the expert's tokens (byte offsets from X); gate or up
    // rows of the expert's weights (a 16-row load stays in one 32-row group)
    as.init([&](int r, const char*& b, uint32_t& o) {
      b = (const char*)X;
      o = (uint32_t)((size_t)tok[m0 + min(r, rows - 1)] * H * 2);
    }, wave, lane);
    bs.init([&](int r, const char*& b, uint32_t& o) {
      const int q = r >> 5;
      const int j = min(j0 + ((q >> 1) << 5) + (r & 31), I - 1);
      b = (const char*)gu_row((const uint16_t*)g.gu_g, (const uint16_t*)g.gu_u, g.gu_es, g.gu_rs, e, q & 1, 0);
      o = (uint32_t)((size_t)g.gu_rs * j * 2);
    }, wave, lane);
    f32x16 acc[C::FM][C::FN];
    pp_mainloop<C, false, false>(as, bs, H / C::BK, St, acc, wave, wm, wn, lane, C::BK,
                                 wm * C::WTM >= rows || j0 + wn * (C::WTN / 2) >= I);
    float* st[4];
    epi_regions<C>(St, st);
    // lane l: activation columns j0 + 2l, 2l + 1, i.e. tile columns c, c + 1
    // (gate) and c + 32, c + 33 (up) with c = 64 (l / 16) + 2 (l % 16)
    const int j = j0 + 2 * lane;
    const int c = ((lane >> 4) << 6) + ((lane & 15) << 1);
    const bool col_ok = j < I;   // I is even, so j + 1 < I too
    uint16_t* a_out = (uint16_t*)g.out0;
    float* z_out = (float*)g.out1;
    dma_epi_rows<C>(acc, rows, wave, wm, wn, lane, st, [&](int tr, const float* lr, int r) {
      const float2 gv = *(const float2*)(lr + (((c >> 2) ^ r) << 2) + (c & 3));
      const float2 uv = *(const float2*)(lr + ((((c + 32) >> 2) ^ r) << 2) + (c & 3));
      if (!col_ok) return;
      const size_t p = (size_t)(m0 + tr);
      if (WRITE_A)
        __builtin_nontemporal_store(pack_bf16(glu_fwd_t<ACT>(gv.x, uv.x, g.limit, g.alpha),
                                              glu_fwd_t<ACT>(gv.y, uv.y, g.limit, g.alpha)),
                                    (uint32_t*)(a_out + p * I + j));
      if (WRITE_Z) {
        float* zr = z_out + p * 2 * I;
        if constexpr (LAYOUT) {
          store4_nt<float>(zr + 2 * j, gv.x, uv.x, gv.y, uv.y);
        } else {
          __builtin_nontemporal_store(f32x2_nt{gv.x, gv.y}, (f32x2_nt*)(zr + j));
          __builtin_nontemporal_store(f32x2_nt{uv.x, uv.y}, (f32x2_nt*)(zr + I + j));
        }
      }
    });
  }
}

// ---------------------------------------------------------------- down fwd
template <class C>
__global__ __launch_bounds__(C::NT, 1) void dma_down_kernel(GArgs g) {
  DMA_PROLOGUE(C)
  TILE_LOOP(C) {
    TILE_SYNC()
    const int H = g.H, I = g.I;
    const uint16_t* Aa = (const uint16_t*)g.A;
    const uint16_t* W = (const uint16_t*)g.B + (size_t)e * H * I;
    const int n0 = nt * C::BN;
    RowSrc<C::NBA, C::BK> as;
    RowSrc<C::NBB, C::BK> bs;
    as.init([&](int r, const char*& b, uint32_t& o) {
      b = (const char*)(Aa + (size_t)m0 * I);
      o = (uint32_t)(min(r, rows - 1) * I * 2);
    }, wave, lane);
    bs.init([&](int r, const char*& b, uint32_t& o) {
      b = (const char*)W;
      o = (uint32_t)((size_t)min(n0 + r, H - 1) * I * 2);
    }, wave, lane);
    f32x16 acc[C::FM][C::FN];
    pp_mainloop<C, false, false>(as, bs, I / C::BK, St, acc, wave, wm, wn, lane, C::BK,
                                 wm * C::WTM >= rows || n0 + wn * C::WTN >= H);
    float* st[4];
    epi_regions<C>(St, st);
    // Y fp32 [S,H] = routing weight * (a . Wd^T); lane l: columns n0 + 4l .. +3
    const int n = n0 + 4 * lane;
    float* Y = (float*)g.out0;
    const float wl = epi_row_weights(g.w_of_pos, m0, rows, wave, lane);
    dma_epi_rows<C>(acc, rows, wave, wm, wn, lane, st, [&](int tr, const float* lr, int r) {
      const float4 v = *(const float4*)(lr + ((lane ^ r) << 2));
      const float w = epi_row_weight(wl, tr);
      if (n < H) store4_nt<float>(Y + (size_t)(m0 + tr) * H + n, w * v.x, w * v.y, w * v.z, w * v.w);
    });
  }
}

// ---------------------------------------------------------------- down dgrad
// The epilogue goes through LDS (as above) with its own row loop: lane l
// takes columns 4l .. 4l + 3 of a row, so Z (2 KB), dZ (1 KB) and aw (512 B)
// move as one contiguous access per row and wave, in batches of 2 rows with
// the next batch's Z loads in flight.

// Sum of the 16 lanes of each DPP row, in every lane of the row: quad
// sums (quad_perm 1,0,3,2 then 2,3,0,1), then the half-row and row mirrors.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_sum16(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Z of one row at columns ic .. ic + 3 (interleaved: g, u pairs over 8 floats;
// concatenated: gate, then up at + I).
template <int LAYOUT>
__device__ __forceinline__ void epi_z_load(const float* zr, int ic, int I, float4& z0, float4& z1) {
  z0 = *(const float4*)(zr + (LAYOUT ? 2 * ic : ic));
  z1 = *(const float4*)(zr + (LAYOUT ? 2 * ic + 4 : I + ic));
}

template <class C, int RB, int ACT, int LAYOUT>
__device__ __forceinline__ void dma_epi_down_dgrad(const GArgs& g, f32x16 (&acc)[C::FM][C::FN], int m0, int rows,
                                                   int n0, int nt, int wave, int wm, int wn, int lane,
                                                   float* const (&st)[4]) {
  static_assert(C::NW == 8 && C::WM == 2 && C::BM % 128 == 0, "8 waves over rows 8q + wave of a 128-row pass");
  const int I = g.I;
  const float* Z = (const float*)g.Z;
  uint16_t* dZ = (uint16_t*)g.out0;
  uint16_t* aw = (uint16_t*)g.out1;
  const int i = n0 + lane * 4;
  const bool col_ok = i < I;
  const int ic = col_ok ? i : I - 4;   // I is a multiple of 4
  const int slot = nt * 2 + (lane >> 5);   // 128-column partial slot of this lane's columns
  const float wl = epi_row_weights(g.w_of_pos, m0, rows, wave, lane);
  lds_barrier();   // every wave's loads into the stages have landed (see pp_mainloop)
#pragma unroll
  for (int h = 0; h < C::BM / 128; ++h) {   // 128-row passes: wave half h's rows, or the whole tile
    if (C::BM == 128 || wm == h) epi_r_to_lds<C>(acc, st, wm, wn, lane);
    lds_barrier();
    const int hrows = rows - h * 128;   // valid rows of this half (may be <= 0)
    if (hrows > 0) {
      float4 za[2][RB], zb[2][RB];
      auto pos = [&](int q) { return m0 + h * 128 + min(q * 8 + wave, hrows - 1); };
      auto load = [&](int b, int buf) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
          epi_z_load<LAYOUT>(Z + (size_t)pos(b * RB + r) * 2 * I, ic, I, za[buf][r], zb[buf][r]);
      };
      auto process = [&](int b, int buf) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int q = b * RB + r, hr = q * 8 + wave;
          const size_t p = (size_t)pos(q);
          const float w = epi_row_weight(wl, h * 128 + hr);
          const float4 rv = *(const float4*)(st[q >> 2] + epi_chunk(hr & 31, lane));
          const float4 z0 = za[buf][r], z1 = zb[buf][r];
          float gv[4], uv[4];
          if constexpr (LAYOUT) {
            gv[0] = z0.x; uv[0] = z0.y; gv[1] = z0.z; uv[1] = z0.w;
            gv[2] = z1.x; uv[2] = z1.y; gv[3] = z1.z; uv[3] = z1.w;
          } else {
            gv[0] = z0.x; gv[1] = z0.y; gv[2] = z0.z; gv[3] = z0.w;
            uv[0] = z1.x; uv[1] = z1.y; uv[2] = z1.z; uv[3] = z1.w;
          }
          const float rr[4] = {rv.x, rv.y, rv.z, rv.w};
          float dg[4], du[4], a[4], rs = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            a[c] = glu_bwd_t<ACT>(gv[c], uv[c], w * rr[c], g.limit, g.alpha, dg[c], du[c]);
            rs += rr[c] * a[c];
          }
          if (!col_ok) rs = 0.f;   // columns past I hold clamped weight columns
          // sum over the 32 lanes of each 128-column slot, in a fixed order:
          // 16-lane row sums by DPP, then lanes 0 + 16 and 32 + 48
          rs = dpp_row_sum16(rs);
          const float rs_lo = readlane_f(rs, 0) + readlane_f(rs, 16), rs_hi = readlane_f(rs, 32) + readlane_f(rs, 48);
          rs = lane < 32 ? rs_lo : rs_hi;
          if (hr < hrows) {
            uint16_t* dzr = dZ + p * 2 * I;
            if (col_ok) {
              if constexpr (LAYOUT) {
                store4x2_nt_bf16(dzr + 2 * i, dg, du);
              } else {
                store4_nt<uint16_t>(dzr + i, dg[0], dg[1], dg[2], dg[3]);
                store4_nt<uint16_t>(dzr + I + i, du[0], du[1], du[2], du[3]);
              }
              store4_nt<uint16_t>(aw + p * I + i, w * a[0], w * a[1], w * a[2], w * a[3]);
            }
            if ((lane & 31) == 0 && slot * 128 < I) g.partials[p * g.nparts + slot] = rs;
          }
        }
      };
      constexpr int NB = 16 / RB;
      load(0, 0);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b + 1 < NB) load(b + 1, (b + 1) & 1);
        process(b, b & 1);
      }
    }
    if (h + 1 < C::BM / 128) lds_barrier();   // half 0 read before half 1 overwrites it
  }
}

// r[p, i] = sum_h dYp[p, h] Wd[e][h, i]: the weights are k (= h) rows of I columns.
template <class C, int ACT, int LAYOUT>
__global__ __launch_bounds__(C::NT, 1) void dma_down_dgrad_kernel(GArgs g) {
  DMA_PROLOGUE(C)
  TILE_LOOP(C) {
    TILE_SYNC()
    const int H = g.H, I = g.I;
    const uint16_t* dYp = (const uint16_t*)g.A;
    const uint16_t* W = (const uint16_t*)g.B + (size_t)e * H * I;
    const int n0 = nt * C::BN;
    RowSrc<C::NBA, C::BK> as;
    ColSrc<C::NBB, false, C::BK> bs;
    as.init([&](int r, const char*& b, uint32_t& o) {
      b = (const char*)(dYp + (size_t)m0 * H);
      o = (uint32_t)(min(r, rows - 1) * H * 2);
    }, wave, lane);
    bs.init(W, W, I, H, I, n0, wave, lane);
    f32x16 acc[C::FM][C::FN];
    pp_mainloop<C, false, true>(as, bs, H / C::BK, St, acc, wave, wm, wn, lane, C::BK,
                                wm * C::WTM >= rows || n0 + wn * C::WTN >= I);
    float* st[4];
    epi_regions<C>(St, st);
    dma_epi_down_dgrad<C, 2, ACT, LAYOUT>(g, acc, m0, rows, n0, nt, wave, wm, wn, lane, st);
  }
}

// ---------------------------------------------------------------- gate_up dgrad
// dXp[p, h] = sum over the 2I dZ columns m of dZ[p, m] (gate or up row of m)[h]:
// the weights are k (= m) rows of H columns, in dZ-column order (the fused
// layouts' row order; separate tensors switch to the up tensor at m = I).
template <class C>
__global__ __launch_bounds__(C::NT, 1) void dma_gate_up_dgrad_kernel(GArgs g) {
  DMA_PROLOGUE(C)
  TILE_LOOP(C) {
    TILE_SYNC()
    const int H = g.H, I = g.I, I2 = 2 * g.I;
    const uint16_t* dZ = (const uint16_t*)g.A;
    const int n0 = nt * C::BN;
    const uint16_t* bg = (const uint16_t*)g.gu_g + g.gu_es * e;
    const uint16_t* bu = (const uint16_t*)g.gu_u + g.gu_es * e;
    RowSrc<C::NBA, C::BK> as;
    ColSrc<C::NBB, false, C::BK> bs;
    as.init([&](int r, const char*& b, uint32_t& o) {
      b = (const char*)(dZ + (size_t)m0 * I2);
      o = (uint32_t)(min(r, rows - 1) * I2 * 2);
    }, wave, lane);
    if (g.gu_sep) bs.init(bg, bu, H, I, H, n0, wave, lane);
    else bs.init(bg, bg, H, I2, H, n0, wave, lane);
    f32x16 acc[C::FM][C::FN];
    pp_mainloop<C, false, true>(as, bs, I2 / C::BK, St, acc, wave, wm, wn, lane, C::BK,
                                wm * C::WTM >= rows || n0 + wn * C::WTN >= H);
    float* st[4];
    epi_regions<C>(St, st);
    // dXp fp32 [S,H]; lane l: columns n0 + 4l .. +3
    const int n = n0 + 4 * lane;
    float* dXp = (float*)g.out0;
    dma_epi_rows<C>(acc, rows, wave, wm, wn, lane, st, [&](int tr, const float* lr, int r) {
      const float4 v = *(const float4*)(lr + ((lane ^ r) << 2));
      if (n < H) store4_nt<float>(dXp + (size_t)(m0 + tr) * H + n, v.x, v.y, v.z, v.w);
    });
  }
}

// ---------------------------------------------------------------- weight gradients
// dW[e] = A_e^T B_e over the expert's positions (k), for experts with more
// than hot_min positions: GATE_UP, A = dZ [S, 2I] and B = Xp [S, H]; else
// A = dYp [S, H] and B = aw [S, I].  Both operands are position-major, so
// both tiles are [32 k][256] column halves.  The expert's k count is ragged:
// the last step's k rows past it read the expert's last position and are
// zeroed in A's tile.  A persistent grid deals chunks of 32 tiles (an XCD's
// 32 workgroups) round-robin to the XCDs, so every XCD gets a share of every
// expert (one hot expert can hold a fifth of all positions); inside an
// expert, groups of 8 M-tiles run N-tile by N-tile, so a chunk's tiles share
// 4 B column blocks and 8 A column blocks in one L2.
template <class C, bool GATE_UP, typename OutT>
__global__ __launch_bounds__(C::NT, 1) void dma_wgrad_kernel(GArgs g) {
  DMA_PROLOGUE(C)
  const int I = g.I, H = g.H;
  const int M = GATE_UP ? 2 * I : H, N = GATE_UP ? H : I;
  {   // no expert above hot_min (the host cannot tell without a sync): leave at once
    const int e0 = g.expert_order[0];
    if (g.offsets[e0 + 1] - g.offsets[e0] <= g.hot_min) return;
  }
  int l = 0, h = g.E;   // l = leading experts (by count, descending) above hot_min
  while (l < h) {
    const int mid = (l + h) >> 1;
    const int e = g.expert_order[mid];
    if (g.offsets[e + 1] - g.offsets[e] > g.hot_min) l = mid + 1; else h = mid;
  }
  const int ntm = g.ntm, ntn = g.ntn, per_e = ntm * ntn;
  const int total = l * per_e;
  const uint16_t* Ag = (const uint16_t*)g.A;
  const uint16_t* Bg = (const uint16_t*)g.B;
  OutT* dW = (OutT*)g.out0;
  // this XCD's j-th tile, increasing in j: the first one past the end ends the loop
  for (int j = blockIdx.x >> 3;; j += gridDim.x >> 3) {
    const int t = dealt_tile<32>(j, total);
    if (t < 0) break;
    if (j != (int)(blockIdx.x >> 3)) lds_barrier();   // the previous tile's stage reads are done
    const int er = t / per_e, local = t - er * per_e;
    const int e = g.expert_order[er];
    const int off = g.offsets[e], cnt = g.offsets[e + 1] - off;   // cnt > hot_min > 0
    const int gsz = kRowTileGroup * ntn;
    const int grp = local / gsz, rem = local - grp * gsz;
    const int gm = min(kRowTileGroup, ntm - grp * kRowTileGroup);
    const int nt = rem / gm, mt = grp * kRowTileGroup + (rem - nt * gm);
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    const uint16_t* Ae = Ag + (size_t)off * M;
    const uint16_t* Be = Bg + (size_t)off * N;
    ColSrc<C::NBA, true, C::BK> as;
    ColSrc<C::NBB, true, C::BK> bs;
    as.init(Ae, Ae, M, 0, M, m0, wave, lane, cnt - 1);
    bs.init(Be, Be, N, 0, N, n0, wave, lane, cnt - 1);
    const int nk = (cnt + C::BK - 1) / C::BK;
    f32x16 acc[C::FM][C::FN];
    pp_mainloop<C, true, true, true>(as, bs, nk, St, acc, wave, wm, wn, lane, cnt - (nk - 1) * C::BK, false);
    float* st[4];
    epi_regions<C>(St, st);
    // through LDS, whole row segments (512 bytes bf16, 1 KB fp32), written
    // once and not read again here (non-temporal); lane l: columns n0 + 4l .. +3
    const int n = n0 + 4 * lane;
    dma_epi_rows<C>(acc, min(M - m0, C::BM), wave, wm, wn, lane, st, [&](int tr, const float* lr, int r) {
      const float4 v = *(const float4*)(lr + ((lane ^ r) << 2));
      const int m = m0 + tr;
      OutT* row;
      if (GATE_UP && g.gu_sep) {   // separate dW_gate, dW_up: row m is a dZ column
        int up, jj;
        zcol(m, I, g.layout, up, jj);
        row = gu_row((OutT*)g.dgu_g, (OutT*)g.dgu_u, g.gu_es, g.gu_rs, e, up, jj);
      } else {
        row = dW + ((size_t)e * M + m) * N;
      }
      if (n < N) store4_nt<OutT>(row + n, v.x, v.y, v.z, v.w);
    });
  }
}

// ------------------------------------------------------------------ host side
// One workgroup per CU, a whole number per XCD (the tile loop walks the rest).
static long persistent_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  return (cus / 8) * 8;
}

// bf16, k dimensions in whole steps of 32, and every byte offset the loads
// form below 2^31: hidden rows from the start of hidden (T * H * 2), an
// expert's weight rows from its gate or up base (2 * I * H * 2), a tile's
// rows from its first row (256 * 2I * 2).
bool dma_enabled(const GemmProblem& pb) {
  const long lim = 1L << 31;
  return pb.dtype == 0 && pb.H % 32 == 0 && pb.I % 32 == 0 && (long)pb.T * pb.H * 2 < lim &&
         4L * pb.I * pb.H < lim && 256L * 4 * pb.I < lim && 256L * 2 * pb.H < lim;
}

// Experts of fewer slots keep the other engine's 128- or 192-row tiles: a
// 256-row tile over a few hundred slots is mostly empty.
constexpr int kLargeTileMinSlots = 512;
int large_tile_min_slots(const GemmProblem& pb) { return dma_enabled(pb) ? kLargeTileMinSlots : 0x7fffffff; }

// 64-k stages (whole cache lines per k-contiguous load) when every k
// dimension of the token-row products (H, I, and I as the split point of
// separate gate / up tensors) is a multiple of 64; 32-k stages otherwise.
static bool dma_bk64(const GemmProblem& pb) { return pb.H % 64 == 0 && pb.I % 64 == 0; }

// f(A, L) with the activation kind and the gate / up layout of the problem
// as compile-time constants (A::value, L::value), so that the epilogues that
// use them are instantiated per kind instead of branching per element.
template <class F>
static void act_layout(const GemmProblem& pb, F&& f) {
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (pb.act) {
    if (pb.layout) f(I1{}, I1{});
    else f(I1{}, I0{});
  } else {
    if (pb.layout) f(I0{}, I1{});
    else f(I0{}, I0{});
  }
}

// The launchers take the problem with its tile set chosen (1: the experts of
// the 256-row tiles, 2: the others) and the kernel's timing name.
static GemmProblem big_experts(const GemmProblem& pb) {
  GemmProblem p = pb;
  p.tile_set = 1;
  return p;
}

template <class C>
static hipError_t dma_gate_up_impl(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                                   const char* name, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = X; g.B = Wgu; g.out0 = a_out; g.out1 = z_out;
  set_gu(g, pb, Wgu, nullptr, 0);
  g.ntn = (pb.I + C::BN / 2 - 1) / (C::BN / 2);
  const long grid = persistent_grid();
  return run_kernel(name, s, [&] {
    act_layout(pb, [&](auto A, auto L) {
      if (a_out && z_out) dma_gate_up_kernel<C, true, true, A.value, L.value><<<grid, C::NT, 0, s>>>(g);
      else if (a_out) dma_gate_up_kernel<C, true, false, A.value, L.value><<<grid, C::NT, 0, s>>>(g);
      else dma_gate_up_kernel<C, false, true, A.value, L.value><<<grid, C::NT, 0, s>>>(g);
    });
  });
}

hipError_t dma_gate_up(const GemmProblem& pb, const void* X, const void* Wgu, void* a_out, void* z_out,
                       hipStream_t s) {
  const char* name = a_out ? "gate_up_glu_big" : "gate_up_z_big";
  return dma_bk64(pb) ? dma_gate_up_impl<DCfgB64>(big_experts(pb), X, Wgu, a_out, z_out, name, s)
                      : dma_gate_up_impl<DCfgB>(big_experts(pb), X, Wgu, a_out, z_out, name, s);
}

template <class C>
static hipError_t dma_down_impl(const GemmProblem& pb, const void* a, const void* Wd, void* Yp, const char* name,
                                hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = a; g.B = Wd; g.out0 = Yp;
  g.ntn = (pb.H + C::BN - 1) / C::BN;
  const long grid = persistent_grid();
  return run_kernel(name, s, [&] { dma_down_kernel<C><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t dma_down(const GemmProblem& pb, const void* a, const void* Wd, void* Yp, hipStream_t s) {
  const char* name = "down_weighted_big";
  return dma_bk64(pb) ? dma_down_impl<DCfgB64>(big_experts(pb), a, Wd, Yp, name, s)
                      : dma_down_impl<DCfgB>(big_experts(pb), a, Wd, Yp, name, s);
}

template <class C>
static hipError_t dma_down_dgrad_impl(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ,
                                      void* aw, float* partials, int nparts, const char* name, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = dY; g.B = Wd; g.Z = Z; g.out0 = dZ; g.out1 = aw; g.partials = partials;
  g.ntn = (pb.I + C::BN - 1) / C::BN;
  g.nparts = nparts;
  const long grid = persistent_grid();
  return run_kernel(name, s, [&] {
    act_layout(pb, [&](auto A, auto L) { dma_down_dgrad_kernel<C, A.value, L.value><<<grid, C::NT, 0, s>>>(g); });
  });
}

hipError_t dma_down_dgrad(const GemmProblem& pb, const void* dY, const void* Wd, const void* Z, void* dZ, void* aw,
                          float* partials, int nparts, hipStream_t s) {
  const char* name = "down_dgrad_glu_bwd_big";
  return dma_bk64(pb) ? dma_down_dgrad_impl<DCfgB64>(big_experts(pb), dY, Wd, Z, dZ, aw, partials, nparts, name, s)
                      : dma_down_dgrad_impl<DCfgB>(big_experts(pb), dY, Wd, Z, dZ, aw, partials, nparts, name, s);
}

template <class C>
static hipError_t dma_gate_up_dgrad_impl(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp,
                                         const char* name, hipStream_t s) {
  GArgs g = base_args(pb, C::BM);
  g.A = dZ; g.B = Wgu; g.out0 = dXp;
  set_gu(g, pb, Wgu, nullptr, 0);
  g.ntn = (pb.H + C::BN - 1) / C::BN;
  const long grid = persistent_grid();
  return run_kernel(name, s, [&] { dma_gate_up_dgrad_kernel<C><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t dma_gate_up_dgrad(const GemmProblem& pb, const void* dZ, const void* Wgu, void* dXp, hipStream_t s) {
  const char* name = "gate_up_dgrad_big";
  return dma_bk64(pb) ? dma_gate_up_dgrad_impl<DCfgB64>(big_experts(pb), dZ, Wgu, dXp, name, s)
                      : dma_gate_up_dgrad_impl<DCfgB>(big_experts(pb), dZ, Wgu, dXp, name, s);
}

// The experts of the other engine's 128-row tiles (tile set 2) on 128 x 256
// tiles of this engine: three stages of 64 k (48 KB each), the same
// ping-pong with 64 x 64 per wave.  H and I multiples of 64.
bool dma_small_enabled(const GemmProblem& pb) { return dma_enabled(pb) && dma_bk64(pb); }

hipError_t dma_gate_up_small(const GemmProblem& ps, const void* X, const void* Wgu, void* a_out, void* z_out,
                             hipStream_t s) {
  return dma_gate_up_impl<DCfgS>(ps, X, Wgu, a_out, z_out, a_out ? "gate_up_glu" : "gate_up_z", s);
}
hipError_t dma_down_small(const GemmProblem& ps, const void* a, const void* Wd, void* Yp, hipStream_t s) {
  return dma_down_impl<DCfgS>(ps, a, Wd, Yp, "down_weighted", s);
}
hipError_t dma_down_dgrad_small(const GemmProblem& ps, const void* dY, const void* Wd, const void* Z, void* dZ,
                                void* aw, float* partials, int nparts, hipStream_t s) {
  return dma_down_dgrad_impl<DCfgS>(ps, dY, Wd, Z, dZ, aw, partials, nparts, "down_dgrad_glu_bwd", s);
}
hipError_t dma_gate_up_dgrad_small(const GemmProblem& ps, const void* dZ, const void* Wgu, void* dXp,
                                   hipStream_t s) {
  return dma_gate_up_dgrad_impl<DCfgS>(ps, dZ, Wgu, dXp, "gate_up_dgrad", s);
}

// Weight gradients of the experts with more than hot_min positions; every
// position row of either operand must sit below 2^31 bytes from the start.
bool dma_wgrad_enabled(const GemmProblem& pb) {
  const long lim = 1L << 31;
  return dma_enabled(pb) && (long)pb.S * 4 * pb.I < lim && (long)pb.S * 2 * pb.H < lim;
}

template <bool GU, typename OutT>
static hipError_t dma_wgrad_impl(const GemmProblem& pb, const void* A, const void* B, void* dW, int hot_min,
                                 hipStream_t s) {
  using C = DCfgW;
  const int M = GU ? 2 * pb.I : pb.H, N = GU ? pb.H : pb.I;
  GArgs g = base_args(pb, C::BM);
  g.A = A; g.B = B; g.out0 = dW;
  if (GU) set_gu(g, pb, nullptr, dW, sizeof(OutT));
  g.ntm = (M + C::BM - 1) / C::BM;
  g.ntn = (N + C::BN - 1) / C::BN;
  g.hot_min = hot_min;
  const long grid = persistent_grid();
  return run_kernel(GU ? "wgrad_gate_up_long" : "wgrad_down_long", s,
                    [&] { dma_wgrad_kernel<C, GU, OutT><<<grid, C::NT, 0, s>>>(g); });
}

hipError_t dma_wgrad(const GemmProblem& pb, bool gate_up, const void* A, const void* B, void* dW, int hot_min,
                     hipStream_t s) {
  if (gate_up)
    return pb.gdtype == 0 ? dma_wgrad_impl<true, uint16_t>(pb, A, B, dW, hot_min, s)
                          : dma_wgrad_impl<true, float>(pb, A, B, dW, hot_min, s);
  return pb.gdtype == 0 ? dma_wgrad_impl<false, uint16_t>(pb, A, B, dW, hot_min, s)
                        : dma_wgrad_impl<false, float>(pb, A, B, dW, hot_min, s);
}

}  // namespace moe
