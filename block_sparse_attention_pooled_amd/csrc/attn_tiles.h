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

// Raw buffer resource over [base, base + bytes) in four scalar registers: loads beyond
// the range return zeros.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu);  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;
  return r;
}

// One buffer->LDS transfer of 16 bytes per lane: lane l's bytes land at LDS byte address
// lds_addr + 16*l, read from byte soff + voff of the resource.  The range check of a raw
// buffer load compares only the per-lane (VGPR) offset with the record count: the scalar
// offset soff is added after the check, so it may carry an offset only where every byte of
// the transfer is known to be in range.  Issued as inline assembly so that the compiler's
// wait-count tracking does not see it: it would otherwise make every LDS read wait for all
// transfers still in flight (it cannot tell which buffer they target), exposing the load
// latency each step.  The caller waits (wait_vmem) and synchronises before reading the
// data.  M0 is restored.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, uint32_t soff,
                                      uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
      : "memory");
}

// The same with the scalar offset 0: the whole offset is range-checked, so bytes at or
// beyond the end of the resource read as zeros.
__device__ __forceinline__ void dma16_checked(const u32x4& rsrc, uint32_t voff,
                                              uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

// 4 bytes per lane (lane l's word at lds_addr + 4*l), from byte soff + voff; the same rule
// for soff as dma16.
__device__ __forceinline__ void dma4(const u32x4& rsrc, uint32_t voff, uint32_t soff,
                                     uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// Per-lane byte offsets of a tile transfer within its tile (row-major [NROWS, D] bf16 in
// HBM; the LDS side is the swizzled Tile layout), computed once per workgroup.  The empty
// asm statements make the values opaque, so that the compiler keeps them in registers
// across the staging loops instead of recomputing them before every transfer.
template <int D, int NROWS, int NWAVES>
struct TileLanes {
  static constexpr int SEGS = NROWS * D * 2 / 1024;
  static constexpr int PER = SEGS / NWAVES;
  static constexpr int RPS = 1024 / (D * 2);
  static_assert(SEGS % NWAVES == 0, "segments must divide among the waves");
  uint32_t off[PER];
  __device__ __forceinline__ TileLanes() {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = (wv * PER + u) * RPS + lane / Tile<D>::CPR;
      const int cc = (lane % Tile<D>::CPR) ^ Tile<D>::swz(row);
      off[u] = (uint32_t)(row * D + cc * 8) * 2;
      asm volatile("" : "+v"(off[u]));
    }
  }
};

// Tile staging through a buffer resource over one head's [N, D] matrix: the tile's first
// row is added to the per-lane offsets, so the range check of the resource sees every
// byte offset and rows at or beyond N read as zeros.
template <int D, int NROWS, int NWAVES>
__device__ __forceinline__ void tile_load_lds_rsrc(const u32x4& rsrc, int row0, uint16_t* lds,
                                                   const TileLanes<D, NROWS, NWAVES>& tl) {
  constexpr int PER = TileLanes<D, NROWS, NWAVES>::PER;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t base = (uint32_t)row0 * D * 2;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    dma16_checked(rsrc, base + tl.off[u], lds_addr(lds + (wv * PER + u) * 512));
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone), issued through the builtin so that
// the compiler's own wait-count bookkeeping knows every vector memory load has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// Per-lane byte offsets, within a tile, of the two transpose reads that gather the
// operand X[8h + t][c0 + lane%32] (t = 0..7; lds_colfrag with r0 = 0) for each 32-column
// block c0 = 32 db.  With the row swizzle depending on a row's low four bits only, a read
// for r0 = 16 kk differs from them by the constant kk * 16 rows, so after one add of the
// tile's base the reads of every k-step use the instruction's immediate offset.  Computed
// once per workgroup; the empty asm statements keep the compiler from recomputing them.
template <int D>
struct ColFragLanes {
  static constexpr int DB = D / 32;
  uint32_t off[DB][2];
  __device__ __forceinline__ explicit ColFragLanes(int lane) {
    const int g = lane >> 4, s = lane & 15;
    const int row = 8 * (g >> 1) + (s >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);
      off[db][0] = (uint32_t)Tile<D>::off(row, col) * 2;
      off[db][1] = (uint32_t)Tile<D>::off(row + 4, col) * 2;
      asm volatile("" : "+v"(off[db][0]), "+v"(off[db][1]));
    }
  }
};

// lds_colfrag<D>(tile, 16 * kk, 32 * db, lane) through precomputed lane offsets: base[h] is
// the tile's LDS byte address plus off[db][h].
template <int D>
__device__ __forceinline__ bf16x8 lds_colfrag_at(uint32_t base_lo, uint32_t base_hi, int kk) {
  const uint32_t step = (uint32_t)kk * 16 * D * 2;
  const i16x4 lo = lds_read_tr16((const SPA_LDS void*)(uintptr_t)(base_lo + step));
  const i16x4 hi = lds_read_tr16((const SPA_LDS void*)(uintptr_t)(base_hi + step));
  return join_bf16x8(lo, hi);
}

// The per-lane read addresses of a tile whose rows r0 .. r0+31 are read (r0 uniform).
template <int D>
__device__ __forceinline__ void colfrag_bases(const uint16_t* tile, int r0,
                                              const ColFragLanes<D>& cf,
                                              uint32_t (&lo)[D / 32], uint32_t (&hi)[D / 32]) {
  const uint32_t b = lds_addr(tile) + (uint32_t)r0 * D * 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    lo[db] = b + cf.off[db][0];
    hi[db] = b + cf.off[db][1];
  }
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

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// v_mfma_f32_32x32x16_f16, same lane layout as the bf16 form
__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// round-to-nearest-even of a float pair into packed fp16
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v));
}

__device__ __forceinline__ f16x8 to_f16x8(const f32x16& x, int half) {
  uint32_t w[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = pk_f16(x[8 * half + 2 * t], x[8 * half + 2 * t + 1]);
  return __builtin_bit_cast(f16x8, w);
}

// Eight bf16 values (packed in a uint4) as fp16 bit patterns, round to nearest even.
// Exact for magnitudes from 2^-14 to below 65504 (fp16 has three more mantissa bits than
// bf16); below 2^-14 fp16 keeps an absolute 2^-25.
__device__ __forceinline__ uint4 bf16x8_bits_to_f16(const uint4& a) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = pk_f16(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xFFFF0000u));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Range classes of eight bf16 values (packed in a uint4) for an fp16 copy, OR-ed together:
//   kF16Over  a value fp16 cannot carry (|x| >= 65504, an infinity or a NaN);
//   kF16Big   a value of magnitude 2^-9 or more;
//   kF16Sub   a nonzero value below 2^-14 (an fp16 subnormal).
constexpr uint32_t kF16Over = 1u, kF16Big = 2u, kF16Sub = 4u;
// The classes of many values are read off two running extremes, kept two bf16 values at a
// time in packed 16-bit integer lanes: the largest magnitude and the smallest magnitude
// minus one, where a zero wraps to 0xFFFF and so never counts as the smallest.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
struct F16Range {
  u16x2 mx = {0, 0};
  u16x2 mn1 = {0xFFFF, 0xFFFF};
  __device__ __forceinline__ void add(const uint4& a) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u16x2 m = __builtin_bit_cast(u16x2, w[e] & 0x7FFF7FFFu);  // bf16 magnitude bits
      mx = __builtin_elementwise_max(mx, m);
      mn1 = __builtin_elementwise_min(mn1, m - (u16x2){1, 1});
    }
  }
  __device__ __forceinline__ uint32_t bits() const {
    const uint32_t hi = mx.x > mx.y ? mx.x : mx.y;
    const uint32_t lo1 = mn1.x < mn1.y ? mn1.x : mn1.y;
    return (hi >= 0x4780u ? kF16Over : 0u)     // 2^16: next bf16 above 65280
           | (hi >= 0x3B00u ? kF16Big : 0u)    // 2^-9
           | (lo1 < 0x387Fu ? kF16Sub : 0u);   // a nonzero magnitude below 2^-14
  }
};
__device__ __forceinline__ uint32_t f16_range_bits(const uint4& a) {
  F16Range r;
  r.add(a);
  return r.bits();
}

// A block of values goes through its fp16 copy when nothing is beyond fp16's range and
// either some value reaches 2^-9 or none is an fp16 subnormal: every value is then carried
// to within 2^-16 of the block's largest magnitude (2^-25 <= 2^-16 * 2^-9), as fine as a
// bf16 hi + lo pair.  Blocks of small values take the bf16 pair instead.
__device__ __forceinline__ bool f16_block_ok(uint32_t r) {
  return !(r & kF16Over) && ((r & kF16Big) || !(r & kF16Sub));
}

// The OR of bits 0-3 of `r` over the wavefront, as wave-uniform bits.
__device__ __forceinline__ uint32_t wave_or4(uint32_t r) {
  uint32_t o = 0;
  if (__ballot(r & 1u)) o |= 1u;
  if (__ballot(r & 2u)) o |= 2u;
  if (__ballot(r & 4u)) o |= 4u;
  if (__ballot(r & 8u)) o |= 8u;
  return o;
}


}  // namespace spa
