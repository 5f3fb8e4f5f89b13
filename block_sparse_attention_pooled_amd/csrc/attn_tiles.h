// Tile staging and MFMA operand gathers shared by the attention kernels.
#pragma once

#include "spa_common.h"

namespace spa {

template <int D>
struct TileCfg {
  static constexpr int LDP = D + 8;                // LDS row pitch in bf16 elements
  static constexpr int TILE = kBlkK * LDP;         // elements per K or V tile
  static constexpr int CHUNKS = kBlkK * D / 8;     // 16-byte chunks per tile
};

// Stage a 64-row tile of a [N, D] bf16 matrix (rows >= N read as zero) into registers.
template <int D, int NT>
__device__ __forceinline__ void tile_load(uint4 (&r)[TileCfg<D>::CHUNKS / NT],
                                          const uint16_t* __restrict__ base, int row0, int N) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int u = 0; u < TileCfg<D>::CHUNKS / NT; ++u) {
    const int x = threadIdx.x + NT * u;
    const int row = x / CPR, cc = x % CPR;
    const int grow = row0 + row;
    r[u] = (unsigned)grow < (unsigned)N
               ? *reinterpret_cast<const uint4*>(base + (size_t)grow * D + cc * 8)
               : make_uint4(0, 0, 0, 0);
  }
}

template <int D, int NT>
__device__ __forceinline__ void tile_store(const uint4 (&r)[TileCfg<D>::CHUNKS / NT],
                                           uint16_t* lds) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int u = 0; u < TileCfg<D>::CHUNKS / NT; ++u) {
    const int x = threadIdx.x + NT * u;
    const int row = x / CPR, cc = x % CPR;
    *reinterpret_cast<uint4*>(lds + row * TileCfg<D>::LDP + cc * 8) = r[u];
  }
}

// A operand of S^T = X Q^T: 8 consecutive columns of LDS row perm32(c) of the 32-row
// slab starting at row r0.
template <int D>
__device__ __forceinline__ bf16x8 lds_rowfrag(const uint16_t* lds, int r0, int kk, int lane) {
  const int c = lane & 31, h = lane >> 5;
  return *reinterpret_cast<const bf16x8*>(lds + (r0 + perm32(c)) * TileCfg<D>::LDP + 16 * kk +
                                          8 * h);
}

// Operand holding X[r0 + 8h + t][c0 + lane%32] for t = 0..7 (X row-major in LDS),
// gathered with two transpose reads.
template <int D>
__device__ __forceinline__ bf16x8 lds_colfrag(const uint16_t* lds, int r0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = r0 + 8 * (g >> 1) + (s >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const uint16_t* p = lds + row * TileCfg<D>::LDP + col;
  const i16x4 lo = lds_read_tr16((const SPA_LDS void*)p);
  const i16x4 hi = lds_read_tr16((const SPA_LDS void*)(p + 4 * TileCfg<D>::LDP));
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
    const __bf16 h = (__bf16)v;
    hi[t] = h;
    lo[t] = (__bf16)(v - (float)h);
  }
}

}  // namespace spa
