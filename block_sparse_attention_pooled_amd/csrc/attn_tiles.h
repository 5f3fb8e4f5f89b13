// Tile staging and MFMA operand gathers shared by the attention kernels.
#pragma once

#include "spa_common.h"

namespace spa {

// LDS layout of a row-major [rows, D] bf16 tile: rows are unpadded and the 16-byte chunks
// of row r are XOR-permuted by swz(r), a rotation of the row's low four bits.  With it
//   - the 16 rows read by 16 consecutive lanes of a perm32-ordered A operand
//     (ds_read_b128) fall on 16 distinct 16-byte chunks of a 256-byte bank window;
//   - the 4 rows x 64 bytes read by 32 consecutive lanes of ds_read_b64_tr_b16 fall on
//     16 distinct chunks;
// and the LDS bank-conflict counter reads zero for all three attention kernels (D = 128).
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int ROWS = kBlkK;         // rows of a K or V tile
  static constexpr int ELEMS = ROWS * D;
  __device__ __forceinline__ static int swz(int r) {
    if constexpr (D == 128)
      return ((r & 3) << 2) | ((r >> 2) & 3);
    else
      return ((r & 3) << 1) | ((r >> 3) & 1);
  }
  // element offset of (row, col); col is a multiple of 4
  __device__ __forceinline__ static int off(int r, int col) {
    return r * D + (((col >> 3) ^ swz(r)) << 3) + (col & 7);
  }
};

// Stage rows [row0, row0 + NROWS) of a [N, D] bf16 matrix into registers, NT threads.
// Rows at or beyond N are read from row N-1 instead: their values are never used
// (scores of such keys are masked, queries beyond N are not written).
template <int D, int NROWS, int NT>
struct Stager {
  static constexpr int CHUNKS = NROWS * D / 8;
  static constexpr int PER = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile chunks must divide among the threads");
  uint4 r[PER];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int row0, int N) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = threadIdx.x + NT * u;
      const int row = min(row0 + x / Tile<D>::CPR, N - 1);
      r[u] = *reinterpret_cast<const uint4*>(base + (size_t)row * D + (x % Tile<D>::CPR) * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = threadIdx.x + NT * u;
      *reinterpret_cast<uint4*>(lds + Tile<D>::off(x / Tile<D>::CPR, (x % Tile<D>::CPR) * 8)) = r[u];
    }
  }
};

// Direct global -> LDS staging (global_load_lds_dwordx4): each wave instruction writes
// 64 lanes x 16 bytes to one contiguous 1 KB LDS segment (lane l at byte 16*l), so the
// swizzle is applied on the global side: lane l of segment s fetches the chunk that
// belongs at LDS chunk 64*s + l.  Rows at or beyond N are fetched from row N-1.
// The caller waits (vmcnt) and synchronises before reading the tile.
template <int D, int NROWS, int NWAVES>
__device__ __forceinline__ void tile_load_lds(const uint16_t* __restrict__ base, int row0, int N,
                                              uint16_t* lds) {
  constexpr int SEGS = NROWS * D * 2 / 1024;   // 1 KB segments per tile
  constexpr int PER = SEGS / NWAVES;
  constexpr int RPS = 1024 / (D * 2);          // rows per segment
  static_assert(SEGS % NWAVES == 0, "segments must divide among the waves");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int seg = wv * PER + u;
    const int row = seg * RPS + lane / Tile<D>::CPR;
    const int pc = lane % Tile<D>::CPR;
    const int cc = pc ^ Tile<D>::swz(row);
    const int grow = min(row0 + row, N - 1);
    __builtin_amdgcn_global_load_lds(base + (size_t)grow * D + cc * 8,
                                     (SPA_LDS void*)(lds + seg * 512), 16, 0, 0);
  }
}

// Raw buffer resource over [base, base + bytes): loads beyond the range return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The same tile staging through a buffer resource over one head's [N, D] matrix: the
// per-lane offsets are loop invariant (the tile's first row enters as a scalar offset), and
// rows at or beyond N read as zeros (the range check of the resource) instead of being
// clamped.
template <int D, int NROWS, int NWAVES>
__device__ __forceinline__ void tile_load_lds_rsrc(__amdgpu_buffer_rsrc_t rsrc, int row0,
                                                   uint16_t* lds) {
  constexpr int SEGS = NROWS * D * 2 / 1024;
  constexpr int PER = SEGS / NWAVES;
  constexpr int RPS = 1024 / (D * 2);
  static_assert(SEGS % NWAVES == 0, "segments must divide among the waves");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int seg = wv * PER + u;
    const int row = seg * RPS + lane / Tile<D>::CPR;
    const int cc = (lane % Tile<D>::CPR) ^ Tile<D>::swz(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SPA_LDS void*)(lds + seg * 512), 16,
                                             (row * D + cc * 8) * 2, row0 * D * 2, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A (or B) operand holding X[r0 + perm32(c)][16*kk + 8*h .. +7] for lane c + 32*h.
template <int D>
__device__ __forceinline__ bf16x8 lds_rowfrag(const uint16_t* lds, int r0, int kk, int lane) {
  const int c = lane & 31, h = lane >> 5;
  return *reinterpret_cast<const bf16x8*>(lds + Tile<D>::off(r0 + perm32(c), 16 * kk + 8 * h));
}

// Operand holding X[r0 + 8h + t][c0 + lane%32] for t = 0..7 (X row-major in LDS),
// gathered with two transpose reads.
template <int D>
__device__ __forceinline__ bf16x8 lds_colfrag(const uint16_t* lds, int r0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = r0 + 8 * (g >> 1) + (s >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const i16x4 lo = lds_read_tr16((const SPA_LDS void*)(lds + Tile<D>::off(row, col)));
  const i16x4 hi = lds_read_tr16((const SPA_LDS void*)(lds + Tile<D>::off(row + 4, col)));
  return join_bf16x8(lo, hi);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// round-to-nearest-even of a float pair into one packed register (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& x, int half) {
  uint32_t w[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = pk_bf16(x[8 * half + 2 * t], x[8 * half + 2 * t + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// Elements 8*half .. 8*half+7 of x as a bf16 pair hi + lo with hi = RNE(x) and
// lo = RNE(x - hi): the pair carries about 16 significant bits, so an MFMA fed with
// both halves loses almost nothing to the bf16 operand format.
__device__ __forceinline__ void split_bf16x8(const f32x16& x, int half, bf16x8& hi, bf16x8& lo) {
  uint32_t wh[4], wl[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float a = x[8 * half + 2 * t], b = x[8 * half + 2 * t + 1];
    const uint32_t p = pk_bf16(a, b);
    wh[t] = p;
    wl[t] = pk_bf16(a - __uint_as_float(p << 16), b - __uint_as_float(p & 0xFFFF0000u));
  }
  hi = __builtin_bit_cast(bf16x8, wh);
  lo = __builtin_bit_cast(bf16x8, wl);
}

// Workgroup order: the hardware deals consecutive workgroup ids round-robin to the 8
// XCDs (each with its own L2).  Map them so that each XCD receives a contiguous run of
// logical tiles (neighbouring query or key blocks of one head share kept tiles).
__device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int X = 8;
  const int whole = total - total % X;
  if (id >= whole) return id;
  return (id % X) * (whole / X) + id / X;
}

}  // namespace spa
