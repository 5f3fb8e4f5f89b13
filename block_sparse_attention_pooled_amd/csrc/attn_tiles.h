// Tile staging and MFMA operand gathers shared by the attention kernels.
#pragma once

#include "spa_common.h"

namespace spa {

// LDS layout of a row-major [rows, D] bf16 tile: rows are unpadded and the 16-byte chunks
// of row r are XOR-permuted by swz(r).  With this permutation
//   - the 16 rows read by 16 consecutive lanes of a perm32-ordered A operand
//     (ds_read_b128) fall on 16 distinct 16-byte bank groups, and every 8 consecutive
//     lanes on 8 distinct ones;
//   - the 4 rows x 32 bytes read by a 16-lane group of ds_read_b64_tr_b16 fall on
//     8 distinct 16-byte bank groups;
// so neither access pattern has bank conflicts (for D = 128).
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int ROWS = kBlkK;         // rows of a K or V tile
  static constexpr int ELEMS = ROWS * D;
  __device__ __forceinline__ static int swz(int r) {
    if constexpr (D == 128)
      return ((r & 3) << 1) | ((r >> 3) & 1) | ((r & 4) << 1);
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

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& x, int half) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)x[8 * half + t];
  return r;
}

// Elements 8*half .. 8*half+7 of x as a bf16 pair hi + lo with hi = RNE(x) and
// lo = RNE(x - hi): the pair carries about 16 significant bits, so an MFMA fed with
// both halves loses almost nothing to the bf16 operand format.
__device__ __forceinline__ void split_bf16x8(const f32x16& x, int half, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float v = x[8 * half + t];
    const __bf16 hv = (__bf16)v;
    hi[t] = hv;
    lo[t] = (__bf16)(v - (float)hv);
  }
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
