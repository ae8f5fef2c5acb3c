// bf16 grouped GEMMs of the routed MoE expert computation (CDNA4 / gfx950).
//
// Forward ("Sparse expert dispatch and combine", "MoE training token repeat
// and expert computation", descriptions): gate_up projection with the gated
// activation in its epilogue; down projection with the routing weight in its
// epilogue.  Backward ("MoE expert parallel execution backward",
// description): down-projection input gradient with the activation backward
// and the routing-weight gradient partials in its epilogue; gate_up input
// gradient; the two weight gradients, which contract over each expert's
// tokens.
//
// Engine
//  * Persistent workgroups (one per CU) walk a list of 128x128 output tiles;
//    the (tile, k-step) sequence is flattened, so loads of the next tile are
//    in flight while the current tile's epilogue runs.
//  * Every operand tile goes global -> LDS with global_load_lds_dwordx4 (no
//    register staging) through NSTAGE LDS stages; one workgroup barrier per
//    k-step.  Out-of-range 16-byte chunks are redirected to a zero page, so
//    every lane issues every load and tails contribute zeros.
//  * K-contiguous operands live in LDS as [row][64 k] (128-byte rows, 16-byte
//    chunks XOR-swizzled by row) and are read with ds_read_b128.
//    MN-contiguous operands (weights in the input gradients, all operands of
//    the weight gradients) live as [64 k][128 col] (256-byte rows, chunks
//    XOR-swizzled by 4*(row%4)) and are read with ds_read_b64_tr_b16, which
//    hands each lane 4 consecutive k of one column.
//  * v_mfma_f32_32x32x16_bf16 with the B tile as the first operand: a lane
//    holds one output row and 4 consecutive output columns per register
//    group, so epilogue stores are 16 (fp32) or 8 (bf16) bytes wide.
//  * XCD-aware static schedule: tiles are dealt to the 8 XCDs in chunks of 8
//    consecutive tiles, so tiles sharing an operand run together in one L2.
#include "moe_internal.h"

namespace moe {
namespace bf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int NT = 256;              // 4 waves
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int WTM = 64, WTN = 64;    // wave tile (2 x 2 waves)
constexpr int FM = 2, FN = 2;        // 32x32 fragments per wave tile
constexpr int TILE_BYTES = 128 * BK * 2;      // 16 KiB per operand tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int NSTAGE = 4;
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;   // 128 KiB
constexpr int LOADS_PER_STEP = 8;    // global_load_lds per wave per k-step (4 per operand)
constexpr int XCD = 8, CHUNK = 8;

__device__ __attribute__((aligned(64))) uint32_t g_zero_page[16];   // zero-initialised

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(bf16_bits(a) | (bf16_bits(b) << 16), bf16_bits(c) | (bf16_bits(d) << 16));
}
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }
__device__ __forceinline__ float glu_fwd(float g, float u, int act, float L, float al) {
  if (act == 0) return g * sigmoid_f(g) * u;
  const float gc = fminf(g, L);
  const float uc = fminf(fmaxf(u, -L), L);
  return (uc + 1.f) * gc * sigmoid_f(al * gc);
}
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

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Make a loaded value "used" here, so its load is waited for once at this
// point instead of inside each predicated store block that consumes it.
__device__ __forceinline__ void force_ready(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void force_ready(float4& x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}
__device__ __forceinline__ void block_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}
// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt_const() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane, global -> LDS (lane i writes lds + 16*i).  Issued from
// inline assembly so that the compiler does not treat every later LDS read as
// dependent on every outstanding DMA (it would wait for vmcnt(0)); the stage
// waits in the main loop are explicit.  M0 holds the wave-uniform LDS byte
// address.  On gfx9 an SALU write of M0 needs one wait state before an LDS
// DMA reads it (the compiler's hazard recognizer cannot see into inline
// assembly), hence the s_nop.
__device__ __forceinline__ void dma16(const void* gptr, lds_char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(base)
               : "memory", "m0");
}
// M0 starts undefined in a wave; give it an in-range LDS address before the
// first DMA.
__device__ __forceinline__ void init_m0() { asm volatile("s_mov_b32 m0, 0\n\ts_nop 0" ::: "m0"); }

// ------------------------------------------------------------------ operands
// K-contiguous operand tile: 128 rows (m or n) x 64 k.  Row r of the tile
// starts at rowp[r]; k in [0, kdim) is valid.
struct KOperand {
  const uint16_t* row_ptr[4];   // this lane's 4 rows (one per load instruction)
  int kdim;
  int chunk_k;                  // this lane's k offset (elements) inside a k-step
  __device__ __forceinline__ void issue(lds_char* tile, int kt, int wave, int lane) const {
    const int k = kt * BK + chunk_k;
    const bool ok = k < kdim;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const void* src = ok ? (const void*)(row_ptr[j] + k) : (const void*)g_zero_page;
      dma16(src, tile + (wave * 4 + j) * 1024);
    }
  }
};
// Lane mapping of a K-contiguous load instruction q: row 8q + lane/8, LDS
// chunk lane%8 holding logical chunk (lane%8) ^ (row%8).
__device__ __forceinline__ int kop_row(int wave, int j, int lane) { return 8 * (wave * 4 + j) + (lane >> 3); }
__device__ __forceinline__ int kop_chunk(int lane) { return (lane & 7) ^ ((lane >> 3) & 7); }

// MN-contiguous operand tile: 64 k-rows x 128 columns.  k-row k (absolute)
// starts at base + k*ld; columns [0, ncols) and k < kvalid are valid.
struct NOperand {
  const uint16_t* base;   // element (k=0, first column of the tile)
  long ld;
  int kvalid;
  int col;                // this lane's column offset (elements)
  bool col_ok;
  __device__ __forceinline__ void issue(lds_char* tile, int kt, int wave, int lane) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kt * BK + 4 * (wave * 4 + j) + (lane >> 4);
      const bool ok = col_ok && k < kvalid;
      const void* src = ok ? (const void*)(base + (long)k * ld + col) : (const void*)g_zero_page;
      dma16(src, tile + (wave * 4 + j) * 1024);
    }
  }
};
__device__ __forceinline__ int nop_chunk(int lane) { return (lane & 15) ^ (((lane >> 4) & 3) << 2); }

// ------------------------------------------------------------------ fragments
// 32 rows x 16 k of a K-contiguous tile: lane -> row rb + lane%32, k 8*(lane/32)..+7
__device__ __forceinline__ bf16x8_t frag_k(const lds_char* tile, int rb, int kk, int lane) {
  const int row = rb + (lane & 31);
  const int chunk = kk * 2 + (lane >> 5);
  return *(const __attribute__((address_space(3))) bf16x8_t*)(tile + row * 128 + ((chunk ^ (row & 7)) << 4));
}
// 32 columns x 16 k of an MN-contiguous tile via two transposing reads.
__device__ __forceinline__ bf16x8_t frag_n(const lds_char* tile, int cb, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = cb + ((g & 1) << 4) + ((s & 3) << 2);
  const int chunk = col >> 3, within = (col & 7) * 2;
  s16x4_t r[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = kk * 16 + ((g >> 1) << 3) + h * 4 + (s >> 2);
    const lds_char* p = tile + krow * 256 + ((chunk ^ ((krow & 3) << 2)) << 4) + within;
    r[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  }
  bf16x8_t out;
  s16x4_t* o = (s16x4_t*)&out;
  o[0] = r[0];
  o[1] = r[1];
  return out;
}

template <bool A_K, bool B_K>
__device__ __forceinline__ void mma_step(const lds_char* At, const lds_char* Bt, int wm, int wn, int lane,
                                         f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8_t a[FM], b[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      a[fm] = A_K ? frag_k(At, wm * WTM + fm * 32, kk, lane) : frag_n(At, wm * WTM + fm * 32, kk, lane);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      b[fn] = B_K ? frag_k(Bt, wn * WTN + fn * 32, kk, lane) : frag_n(Bt, wn * WTN + fn * 32, kk, lane);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[fn], a[fm], acc[fm][fn], 0, 0, 0);
  }
}
// Accumulator element (fm, fn, v) of lane: row wm*64 + fm*32 + lane%32,
// column wn*64 + fn*32 + 8*(v/4) + 4*(lane/32) + v%4.
__device__ __forceinline__ int acc_col(int fn, int vg, int lane, int wn) {
  return wn * WTN + fn * 32 + vg * 8 + ((lane >> 5) << 2);
}

// ------------------------------------------------------------------ schedule
// Tile index of the i-th tile a workgroup processes (tiles dealt to XCDs in
// chunks of CHUNK consecutive tiles; inside an XCD, round-robin over its
// workgroups).  Returns -1 past the end.
__device__ __forceinline__ int sched_tile(int i, int total) {
  const int b = blockIdx.x, x = b % XCD, lb = b / XCD, per = gridDim.x / XCD;
  const int li = lb + i * per;
  const int t = ((li / CHUNK) * XCD + x) * CHUNK + (li % CHUNK);
  return t < total ? t : -1;
}

// ------------------------------------------------------------------ arguments
struct Args {
  const int32_t* offsets;       // [E+1]
  const int32_t* tile_prefix;   // [E+1] M-tiles of 128 rows per expert
  const int32_t* expert_order;  // [E] by descending count
  const float* w_of_pos;        // [S]
  const void* A;
  const void* B;
  const void* Z;
  void* out0;
  void* out1;
  float* partials;
  int H, I, E, S;
  int act, layout;
  float limit, alpha;
  int ntn, ntm, nparts;
};
// Kernel arguments must have one layout on the host and on the device: only
// global pointers, ints and floats (an LDS pointer is 4 bytes on the device
// and 8 on the host).
static_assert(sizeof(Args) == 10 * 8 + 11 * 4 + 4, "Args layout must match between host and device");

// LDS copies of the routing tables, built by each workgroup on entry.
typedef const __attribute__((address_space(3))) int32_t* lds_i32;
struct Tabs {
  lds_i32 offsets;       // [E+1]
  lds_i32 tile_prefix;   // [E+1]
  lds_i32 expert_order;  // [E]
};

// Row-tile (expert, first row, rows) of tile t in the token-row schedule:
// tiles ordered by expert, then N-tile, then M-tile.
__device__ __forceinline__ void row_tile(const Args& g, const Tabs& tb, int t, int& e, int& m0, int& rows,
                                         int& nt) {
  lds_i32 tp = tb.tile_prefix;
  const int q = t / g.ntn;
  int lo = 0, hi = g.E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tp[mid] <= q) lo = mid; else hi = mid - 1;
  }
  e = lo;
  const int nm = tp[e + 1] - tp[e];
  const int local = t - tp[e] * g.ntn;
  nt = local / nm;
  const int mt = local - nt * nm;
  m0 = tb.offsets[e] + mt * BM;
  rows = min(BM, tb.offsets[e + 1] - m0);
}

// ------------------------------------------------------------------ policies
// Row pointers of a K-contiguous operand whose tile rows are consecutive
// rows r0 + r of a row-major matrix (rows past `rows` repeat the last row).
__device__ __forceinline__ void k_rows(KOperand& op, const uint16_t* base, long ld, int r0, int rows, int kdim,
                                       int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) op.row_ptr[j] = base + (long)(r0 + min(kop_row(wave, j, lane), rows - 1)) * ld;
  op.kdim = kdim;
  op.chunk_k = kop_chunk(lane) * 8;
}
__device__ __forceinline__ void n_cols(NOperand& op, const uint16_t* base, long ld, int kvalid, int ncols,
                                       int lane) {
  op.base = base;
  op.ld = ld;
  op.kvalid = kvalid;
  op.col = nop_chunk(lane) * 8;
  op.col_ok = op.col < ncols;
}

// gate_up projection + gated activation.  B rows of a tile: 32 gate rows and
// 32 up rows of activation columns j0..j0+31, then the next 32 columns.
template <bool WRITE_A, bool WRITE_Z>
struct GateUp {
  static constexpr bool A_K = true, B_K = true;
  struct Tile {
    KOperand a, b;
    int e, m0, rows, nt;
  };
  __device__ static int total(const Args& g, const Tabs& tb) { return tb.tile_prefix[g.E] * g.ntn; }
  __device__ static void setup(const Args& g, const Tabs& tb, int t, Tile& T, int wave, int lane) {
    row_tile(g, tb, t, T.e, T.m0, T.rows, T.nt);
    const int H = g.H, I = g.I;
    k_rows(T.a, (const uint16_t*)g.A, H, T.m0, T.rows, H, wave, lane);
    const uint16_t* W = (const uint16_t*)g.B + (size_t)T.e * 2 * I * H;
    const int j0 = T.nt * (BN / 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = kop_row(wave, j, lane);
      const int q = r >> 5;
      const int ja = min(j0 + ((q >> 1) << 5) + (r & 31), I - 1);
      const int wrow = g.layout ? 2 * ja + (q & 1) : ((q & 1) ? I + ja : ja);
      T.b.row_ptr[j] = W + (size_t)wrow * H;
    }
    T.b.kdim = H;
    T.b.chunk_k = kop_chunk(lane) * 8;
  }
  __device__ static void epilogue(const Args& g, const Tile& T, f32x16 (&acc)[FM][FN], int wm, int wn, int lane,
                                  lds_char*) {
    const int I = g.I;
    uint16_t* a_out = (uint16_t*)g.out0;
    float* z_out = (float*)g.out1;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int rl = wm * WTM + fm * 32 + (lane & 31);
      if (rl >= T.rows) continue;
      const size_t p = (size_t)(T.m0 + rl);
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int j = T.nt * (BN / 2) + wn * 32 + vg * 8 + ((lane >> 5) << 2);
        if (j >= I) continue;
        float gv[4], uv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[i] = acc[fm][0][vg * 4 + i];
          uv[i] = acc[fm][1][vg * 4 + i];
        }
        if (WRITE_A) {
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = glu_fwd(gv[i], uv[i], g.act, g.limit, g.alpha);
          *(uint2*)(a_out + p * I + j) = pack4_bf16(a[0], a[1], a[2], a[3]);
        }
        if (WRITE_Z) {
          float* zr = z_out + p * 2 * I;
          if (g.layout) {
            *(float4*)(zr + 2 * j) = make_float4(gv[0], uv[0], gv[1], uv[1]);
            *(float4*)(zr + 2 * j + 4) = make_float4(gv[2], uv[2], gv[3], uv[3]);
          } else {
            *(float4*)(zr + j) = make_float4(gv[0], gv[1], gv[2], gv[3]);
            *(float4*)(zr + I + j) = make_float4(uv[0], uv[1], uv[2], uv[3]);
          }
        }
      }
    }
  }
};

// down projection, routing weight in the epilogue: Yp fp32 [S, H]
struct Down {
  static constexpr bool A_K = true, B_K = true;
  struct Tile {
    KOperand a, b;
    int e, m0, rows, nt;
  };
  __device__ static int total(const Args& g, const Tabs& tb) { return tb.tile_prefix[g.E] * g.ntn; }
  __device__ static void setup(const Args& g, const Tabs& tb, int t, Tile& T, int wave, int lane) {
    row_tile(g, tb, t, T.e, T.m0, T.rows, T.nt);
    const int H = g.H, I = g.I;
    k_rows(T.a, (const uint16_t*)g.A, I, T.m0, T.rows, I, wave, lane);
    const uint16_t* W = (const uint16_t*)g.B + (size_t)T.e * H * I;
    const int n0 = T.nt * BN;
    k_rows(T.b, W, I, n0, H - n0, I, wave, lane);
  }
  __device__ static void epilogue(const Args& g, const Tile& T, f32x16 (&acc)[FM][FN], int wm, int wn, int lane,
                                  lds_char*) {
    // loads first and unconditional (clamped rows), stores predicated afterwards
    const int H = g.H;
    float* Y = (float*)g.out0;
    float w[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      w[fm] = g.w_of_pos[T.m0 + min(wm * WTM + fm * 32 + (lane & 31), T.rows - 1)];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) force_ready(w[fm]);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int rl = wm * WTM + fm * 32 + (lane & 31);
      const size_t p = (size_t)(T.m0 + rl);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int n = T.nt * BN + acc_col(fn, vg, lane, wn);
          if (rl < T.rows && n < H)
            *(float4*)(Y + p * H + n) = make_float4(w[fm] * acc[fm][fn][vg * 4], w[fm] * acc[fm][fn][vg * 4 + 1],
                                                    w[fm] * acc[fm][fn][vg * 4 + 2], w[fm] * acc[fm][fn][vg * 4 + 3]);
        }
    }
  }
};

// down-projection input gradient r = dYp . Wd[e] with the activation backward:
// dZ (bf16, stored layout), aw = w * a (bf16), per-tile partial <r, a>.
struct DownDgrad {
  static constexpr bool A_K = true, B_K = false;
  struct Tile {
    KOperand a;
    NOperand b;
    int e, m0, rows, nt;
  };
  __device__ static int total(const Args& g, const Tabs& tb) { return tb.tile_prefix[g.E] * g.ntn; }
  __device__ static void setup(const Args& g, const Tabs& tb, int t, Tile& T, int wave, int lane) {
    row_tile(g, tb, t, T.e, T.m0, T.rows, T.nt);
    const int H = g.H, I = g.I;
    k_rows(T.a, (const uint16_t*)g.A, H, T.m0, T.rows, H, wave, lane);
    const int n0 = T.nt * BN;
    n_cols(T.b, (const uint16_t*)g.B + (size_t)T.e * H * I + n0, I, H, I - n0, lane);
  }
  __device__ static void epilogue(const Args& g, const Tile& T, f32x16 (&acc)[FM][FN], int wm, int wn, int lane,
                                  lds_char* red_area) {
    const int I = g.I;
    const float* Z = (const float*)g.Z;
    uint16_t* dZ = (uint16_t*)g.out0;
    uint16_t* aw = (uint16_t*)g.out1;
    float* red = (float*)red_area;     // [2][BM]
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int rl = wm * WTM + fm * 32 + (lane & 31);
      const bool rv = rl < T.rows;
      const size_t p = (size_t)(T.m0 + min(rl, T.rows - 1));
      // unconditional loads (clamped columns): w and this row's g/u values
      const float w = g.w_of_pos[p];
      const float* zr = Z + p * 2 * I;
      float4 za[FN][4], zb[FN][4];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int i = min(T.nt * BN + acc_col(fn, vg, lane, wn), I - 4);
          if (g.layout) {
            za[fn][vg] = *(const float4*)(zr + 2 * i);
            zb[fn][vg] = *(const float4*)(zr + 2 * i + 4);
          } else {
            za[fn][vg] = *(const float4*)(zr + i);
            zb[fn][vg] = *(const float4*)(zr + I + i);
          }
        }
      float wr = w;
      force_ready(wr);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          force_ready(za[fn][vg]);
          force_ready(zb[fn][vg]);
        }
      float rs = 0.f;
      uint16_t* dzr = dZ + p * 2 * I;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int i = T.nt * BN + acc_col(fn, vg, lane, wn);
          const bool ok = rv && i < I;
          float gv[4], uv[4];
          if (g.layout) {
            gv[0] = za[fn][vg].x; uv[0] = za[fn][vg].y; gv[1] = za[fn][vg].z; uv[1] = za[fn][vg].w;
            gv[2] = zb[fn][vg].x; uv[2] = zb[fn][vg].y; gv[3] = zb[fn][vg].z; uv[3] = zb[fn][vg].w;
          } else {
            gv[0] = za[fn][vg].x; gv[1] = za[fn][vg].y; gv[2] = za[fn][vg].z; gv[3] = za[fn][vg].w;
            uv[0] = zb[fn][vg].x; uv[1] = zb[fn][vg].y; uv[2] = zb[fn][vg].z; uv[3] = zb[fn][vg].w;
          }
          float dg[4], du[4], a[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float r = acc[fm][fn][vg * 4 + q];
            a[q] = glu_bwd(gv[q], uv[q], wr * r, g.act, g.limit, g.alpha, dg[q], du[q]);
            rs += ok ? r * a[q] : 0.f;
          }
          if (ok) {
            if (g.layout) {
              *(uint4*)(dzr + 2 * i) = make_uint4(bf16_bits(dg[0]) | (bf16_bits(du[0]) << 16),
                                                  bf16_bits(dg[1]) | (bf16_bits(du[1]) << 16),
                                                  bf16_bits(dg[2]) | (bf16_bits(du[2]) << 16),
                                                  bf16_bits(dg[3]) | (bf16_bits(du[3]) << 16));
            } else {
              *(uint2*)(dzr + i) = pack4_bf16(dg[0], dg[1], dg[2], dg[3]);
              *(uint2*)(dzr + I + i) = pack4_bf16(du[0], du[1], du[2], du[3]);
            }
            *(uint2*)(aw + p * I + i) = pack4_bf16(wr * a[0], wr * a[1], wr * a[2], wr * a[3]);
          }
        }
      rs += __shfl_xor(rs, 32);
      if (lane < 32) red[wn * BM + wm * WTM + fm * 32 + lane] = rs;
    }
    block_barrier();
    if (threadIdx.x < T.rows)
      g.partials[(size_t)(T.m0 + threadIdx.x) * g.nparts + T.nt] = red[threadIdx.x] + red[BM + threadIdx.x];
  }
};

// gate_up input gradient dXp = dZ . Wgu[e], fp32 [S, H]
struct GateUpDgrad {
  static constexpr bool A_K = true, B_K = false;
  struct Tile {
    KOperand a;
    NOperand b;
    int e, m0, rows, nt;
  };
  __device__ static int total(const Args& g, const Tabs& tb) { return tb.tile_prefix[g.E] * g.ntn; }
  __device__ static void setup(const Args& g, const Tabs& tb, int t, Tile& T, int wave, int lane) {
    row_tile(g, tb, t, T.e, T.m0, T.rows, T.nt);
    const int H = g.H, I2 = 2 * g.I;
    k_rows(T.a, (const uint16_t*)g.A, I2, T.m0, T.rows, I2, wave, lane);
    const int n0 = T.nt * BN;
    n_cols(T.b, (const uint16_t*)g.B + (size_t)T.e * I2 * H + n0, H, I2, H - n0, lane);
  }
  __device__ static void epilogue(const Args& g, const Tile& T, f32x16 (&acc)[FM][FN], int wm, int wn, int lane,
                                  lds_char*) {
    const int H = g.H;
    float* dX = (float*)g.out0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int rl = wm * WTM + fm * 32 + (lane & 31);
      if (rl >= T.rows) continue;
      const size_t p = (size_t)(T.m0 + rl);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int n = T.nt * BN + acc_col(fn, vg, lane, wn);
          if (n < H)
            *(float4*)(dX + p * H + n) = make_float4(acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1],
                                                     acc[fm][fn][vg * 4 + 2], acc[fm][fn][vg * 4 + 3]);
        }
    }
  }
};

// Weight gradients: dW[e][m, n] = sum over the expert's positions p of
// A[p, m] * B[p, n], both operands token-major.  Experts longest first.
//   GU:  M = 2I (rows of dWgu), A = dZ [S,2I],  B = Xp [S,H]
//   !GU: M = H  (rows of dWd),  A = dYp [S,H],  B = aw [S,I]
template <bool GU, bool OUT_BF16>
struct Wgrad {
  static constexpr bool A_K = false, B_K = false;
  struct Tile {
    NOperand a, b;
    int e, cnt, m0, n0;
  };
  __device__ static int total(const Args& g, const Tabs&) { return g.E * g.ntm * g.ntn; }
  __device__ static void setup(const Args& g, const Tabs& tb, int t, Tile& T, int wave, int lane) {
    const int per = g.ntm * g.ntn;
    const int er = t / per, tt = t - er * per;
    const int mt = tt / g.ntn, nt = tt - mt * g.ntn;
    T.e = tb.expert_order[er];
    const int off = tb.offsets[T.e];
    T.cnt = tb.offsets[T.e + 1] - off;
    T.m0 = mt * BM;
    T.n0 = nt * BN;
    const int H = g.H, I = g.I;
    const int M = GU ? 2 * I : H, N = GU ? H : I;
    const long lda = GU ? 2 * I : H, ldb = GU ? H : I;
    n_cols(T.a, (const uint16_t*)g.A + (size_t)off * lda + T.m0, lda, T.cnt, M - T.m0, lane);
    n_cols(T.b, (const uint16_t*)g.B + (size_t)off * ldb + T.n0, ldb, T.cnt, N - T.n0, lane);
  }
  __device__ static void epilogue(const Args& g, const Tile& T, f32x16 (&acc)[FM][FN], int wm, int wn, int lane,
                                  lds_char*) {
    const int H = g.H, I = g.I;
    const int M = GU ? 2 * I : H, N = GU ? H : I;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = T.m0 + wm * WTM + fm * 32 + (lane & 31);
      if (m >= M) continue;
      const size_t rowoff = ((size_t)T.e * M + m) * N;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int n = T.n0 + acc_col(fn, vg, lane, wn);
          if (n >= N) continue;
          if (OUT_BF16)
            *(uint2*)((uint16_t*)g.out0 + rowoff + n) =
                pack4_bf16(acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1], acc[fm][fn][vg * 4 + 2],
                           acc[fm][fn][vg * 4 + 3]);
          else
            *(float4*)((float*)g.out0 + rowoff + n) = make_float4(acc[fm][fn][vg * 4], acc[fm][fn][vg * 4 + 1],
                                                                  acc[fm][fn][vg * 4 + 2], acc[fm][fn][vg * 4 + 3]);
        }
    }
  }
};

template <class P> struct Steps;
template <bool A, bool Z> struct Steps<GateUp<A, Z>> {
  __device__ static int nk(const Args& g, const typename GateUp<A, Z>::Tile&) { return (g.H + BK - 1) / BK; }
};
template <> struct Steps<Down> {
  __device__ static int nk(const Args& g, const Down::Tile&) { return (g.I + BK - 1) / BK; }
};
template <> struct Steps<DownDgrad> {
  __device__ static int nk(const Args& g, const DownDgrad::Tile&) { return (g.H + BK - 1) / BK; }
};
template <> struct Steps<GateUpDgrad> {
  __device__ static int nk(const Args& g, const GateUpDgrad::Tile&) { return (2 * g.I + BK - 1) / BK; }
};
template <bool GU, bool OB> struct Steps<Wgrad<GU, OB>> {
  __device__ static int nk(const Args&, const typename Wgrad<GU, OB>::Tile& T) { return (T.cnt + BK - 1) / BK; }
};

// ------------------------------------------------------------------ the loop
// Kind-specific parts come from a policy P:
//   P::total(g, tabs)                      number of tiles
//   P::setup(g, tabs, t, tile, wave, lane) operand addressing + epilogue information
//   Steps<P>::nk(g, tile)            k-steps of the tile
//   P::epilogue(g, tile, acc, ...)   fused epilogue and stores
// One wave-level zero-page DMA per operand load instruction: keeps the number
// of loads per k-step constant once the tile list is exhausted.
__device__ __forceinline__ void issue_dummy(lds_char* st, int wave) {
#pragma unroll
  for (int j = 0; j < LOADS_PER_STEP; ++j)
    dma16((const void*)g_zero_page, st + (j >> 2) * TILE_BYTES + (wave * 4 + (j & 3)) * 1024);
}

template <class P>
__global__ __launch_bounds__(NT) void persistent_kernel(Args g) {
  extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];
  lds_char* lds = (lds_char*)smem_dyn;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  init_m0();

  // routing tables -> LDS
  __attribute__((address_space(3))) int32_t* tab = (__attribute__((address_space(3))) int32_t*)(lds + LDS_BYTES + 2 * BM * 4);
  for (int i = threadIdx.x; i <= g.E; i += NT) {
    tab[i] = g.offsets[i];
    tab[(g.E + 1) + i] = g.tile_prefix[i];
    if (i < g.E) tab[2 * (g.E + 1) + i] = g.expert_order[i];
  }
  const Tabs tb = {tab, tab + (g.E + 1), tab + 2 * (g.E + 1)};
  __syncthreads();
  const int total = P::total(g, tb);

  typename P::Tile it;          // issue-side tile
  int it_i = 0, it_t = sched_tile(0, total), it_k = 0, it_nk = 0;
  if (it_t >= 0) { P::setup(g, tb, it_t, it, wave, lane); it_nk = Steps<P>::nk(g, it); }
  int issued = 0;
  auto issue_next = [&]() {
    while (it_t >= 0 && it_k >= it_nk) {
      it_t = sched_tile(++it_i, total);
      it_k = 0;
      if (it_t >= 0) { P::setup(g, tb, it_t, it, wave, lane); it_nk = Steps<P>::nk(g, it); }
    }
    lds_char* st = lds + (issued % NSTAGE) * STAGE_BYTES;
    if (it_t >= 0) {
      it.a.issue(st, it_k, wave, lane);
      it.b.issue(st + TILE_BYTES, it_k, wave, lane);
      ++it_k;
    } else {
      issue_dummy(st, wave);
    }
    ++issued;
  };
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) issue_next();

  int step = 0;
  for (int ci = 0;; ++ci) {
    const int t = sched_tile(ci, total);
    if (t < 0) break;
    typename P::Tile ct;
    P::setup(g, tb, t, ct, wave, lane);
    const int nk = Steps<P>::nk(g, ct);
    f32x16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      // step `step` was issued NSTAGE-1 issues ago; NSTAGE-2 newer steps may stay in flight
      wait_vmcnt_const<(NSTAGE - 2) * LOADS_PER_STEP>();
      block_barrier();
      issue_next();
      const lds_char* st = lds + (step % NSTAGE) * STAGE_BYTES;
      mma_step<P::A_K, P::B_K>(st, st + TILE_BYTES, wm, wn, lane, acc);
      ++step;
    }
    P::epilogue(g, ct, acc, wm, wn, lane, lds + LDS_BYTES);
  }
  wait_vmcnt_const<0>();    // no LDS DMA may be outstanding when the workgroup ends
}

// ------------------------------------------------------------------ host side
constexpr int SMEM_BYTES = LDS_BYTES + 2 * BM * 4 + 3 * (MAX_E + 1) * 4;   // stages + reduction + tables

static int grid_size() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < XCD)
      cus = 256;
    cached[dev] = (cus / XCD) * XCD;
  }
  return cached[dev];
}

// This engine faulted the GPU on its first parity run (cause not yet found on
// the CPU); it is compiled but switched off until it is.  Define
// MOE_ENABLE_LDS_DMA_ENGINE=1 to build it in.
#ifndef MOE_ENABLE_LDS_DMA_ENGINE
#define MOE_ENABLE_LDS_DMA_ENGINE 0
#endif

template <class P>
static hipError_t launch(const char* name, const Args& g, hipStream_t s) {
  if (!MOE_ENABLE_LDS_DMA_ENGINE) return hipErrorNotSupported;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)persistent_kernel<P>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int grid = grid_size();
  return run_kernel(name, s, [&] { persistent_kernel<P><<<grid, NT, SMEM_BYTES, s>>>(g); });
}

static Args base_args(const GemmProblem& pb) {
  Args g = {};
  const RouteState& rs = *pb.rs;
  g.offsets = rs.offsets;
  g.tile_prefix = rs.tile_prefix + 2 * (pb.E + 1);   // 128-row M-tiles
  g.expert_order = rs.expert_order;
  g.w_of_pos = rs.w_of_pos;
  g.H = pb.H; g.I = pb.I; g.E = pb.E; g.S = pb.S;
  g.act = pb.act; g.layout = pb.layout; g.limit = pb.limit; g.alpha = pb.alpha;
  return g;
}

}  // namespace bf

hipError_t launch_gate_up_bf16(const GemmProblem& pb, const void* Xp, const void* Wgu, void* a_out, void* z_out,
                               hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  bf::Args g = bf::base_args(pb);
  g.A = Xp; g.B = Wgu; g.out0 = a_out; g.out1 = z_out;
  g.ntn = (pb.I + bf::BN / 2 - 1) / (bf::BN / 2);
  if (a_out && z_out) return bf::launch<bf::GateUp<true, true>>("gate_up_glu", g, s);
  if (a_out) return bf::launch<bf::GateUp<true, false>>("gate_up_glu", g, s);
  return bf::launch<bf::GateUp<false, true>>("gate_up_z", g, s);
}

hipError_t launch_down_bf16(const GemmProblem& pb, const void* a, const void* Wd, float* Yp, hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  bf::Args g = bf::base_args(pb);
  g.A = a; g.B = Wd; g.out0 = Yp;
  g.ntn = (pb.H + bf::BN - 1) / bf::BN;
  return bf::launch<bf::Down>("down_weighted", g, s);
}

hipError_t launch_down_dgrad_bf16(const GemmProblem& pb, const void* dYp, const void* Wd, const float* Z, void* dZ,
                                  void* aw, float* partials, int* nparts, hipStream_t s) {
  bf::Args g = bf::base_args(pb);
  g.ntn = (pb.I + bf::BN - 1) / bf::BN;
  *nparts = g.ntn;
  if (pb.S == 0) return hipSuccess;
  g.A = dYp; g.B = Wd; g.Z = Z; g.out0 = dZ; g.out1 = aw; g.partials = partials; g.nparts = g.ntn;
  return bf::launch<bf::DownDgrad>("down_dgrad_glu_bwd", g, s);
}

hipError_t launch_gate_up_dgrad_bf16(const GemmProblem& pb, const void* dZ, const void* Wgu, float* dXp,
                                     hipStream_t s) {
  if (pb.S == 0) return hipSuccess;
  bf::Args g = bf::base_args(pb);
  g.A = dZ; g.B = Wgu; g.out0 = dXp;
  g.ntn = (pb.H + bf::BN - 1) / bf::BN;
  return bf::launch<bf::GateUpDgrad>("gate_up_dgrad", g, s);
}

template <bool GU>
static hipError_t wgrad_bf16(const GemmProblem& pb, const void* A, const void* B, void* dW, hipStream_t s) {
  bf::Args g = bf::base_args(pb);
  g.A = A; g.B = B; g.out0 = dW;
  const int M = GU ? 2 * pb.I : pb.H, N = GU ? pb.H : pb.I;
  g.ntm = (M + bf::BM - 1) / bf::BM;
  g.ntn = (N + bf::BN - 1) / bf::BN;
  const char* name = GU ? "wgrad_gate_up" : "wgrad_down";
  return pb.gdtype == 0 ? bf::launch<bf::Wgrad<GU, true>>(name, g, s) : bf::launch<bf::Wgrad<GU, false>>(name, g, s);
}

hipError_t launch_wgrad_down_bf16(const GemmProblem& pb, const void* dYp, const void* aw, void* dWd, hipStream_t s) {
  return wgrad_bf16<false>(pb, dYp, aw, dWd, s);
}

hipError_t launch_wgrad_gate_up_bf16(const GemmProblem& pb, const void* dZ, const void* Xp, void* dWgu,
                                     hipStream_t s) {
  return wgrad_bf16<true>(pb, dZ, Xp, dWgu, s);
}

}  // namespace moe
