// Shared device helpers for the gfx950 kernels: vector types, bf16 conversion,
// MFMA wrappers, LDS transpose reads and the row permutation used by the attention
// kernels.  Internal to libspa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;

constexpr int kWave = 64;
constexpr int kBlkK = 64;  // key block size
constexpr int kMaxBlocks = 2048;  // most key blocks per head (query blocks are never more)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#define SPA_LDS __attribute__((address_space(3)))

// ---- bf16 <-> fp32 ------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// round-to-nearest-even fp32 -> bf16 bits (inputs here are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---- MFMA ---------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16.  Lane l = c + 32*h supplies A[row=c][k=8h..8h+7] and
// B[k=8h..8h+7][col=c]; accumulator element i of lane l is D[8*(i/4) + 4*h + i%4][c].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The attention kernels load the 32 rows of an MFMA A operand in the order
// row r -> source row perm32(r), so that accumulator element i of lane c + 32*h holds
// source row 16*(i/8) + 8*h + i%8: each lane then owns runs of 8 consecutive source
// rows, which is exactly the k-slot layout of the next MFMA's operand.
__device__ __forceinline__ int perm32(int r) {
  const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// Source row held by accumulator element i of a lane in half h (after perm32 loading).
__device__ __forceinline__ int acc_row(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }

// ---- LDS transpose read (ds_read_b64_tr_b16) -------------------------------------------
// Within each group of 16 lanes, lane s supplies the address of 4 consecutive bf16 of a
// row-major LDS matrix X at X[r0 + s/4][c0 + 4*(s%4)]; lane j of the group receives
// X[r0 + e][c0 + j] for e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const SPA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SPA_LDS i16x4*)p);
}

__device__ __forceinline__ bf16x8 join_bf16x8(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---- wave reductions ----------------------------------------------------------------
__device__ __forceinline__ float swap_halves(float x) {  // value of lane l ^ 32
  return __shfl_xor(x, 32, 64);
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
