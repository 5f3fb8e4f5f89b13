// Block-sparse attention backward over the kept tiles only, mask held fixed (abstract
// page "SpargeAttention2: Trainable Sparse Attention via Hybrid Top-k+Top-p Masking and
// Distillation Fine-Tuning", contribution (ii); mindverse article, section "Effiziente
// Kernel-Implementierung und Modellanpassung").
//
// Launch sequence (one stream):
//   k_bitmap    the kept-tile bitmap, transposed: word w of query block i at [w][i];
//   k_collists  per key block j, the ascending list of query blocks that keep j, and the
//               dispatch order of the dK/dV workgroups (longest lists first within each
//               run of 32 neighbouring key blocks);
//   k_vflag     per key block, whether its V may be read through an fp16 copy in dK/dV;
//   k_dq        one workgroup per (b, h, query block): first D_t = <dO_t, O_t> in fp32
//               (O = o + o_lo when the forward pass supplied its rounding residual) and
//               lse_t * log2(e) for its rows, kept in registers and written out for the
//               next kernel; then walks its key-block list in ascending order and
//               accumulates dQ += dS K;
//   k_dkdv      one resident workgroup per compute unit, taking (b, h, key block) tiles
//               from work queues in the dispatch order; per tile it walks the query-block
//               list in ascending order, recomputes S and P (reading D and lse * log2(e)
//               that k_dq wrote), accumulates dV += P^T dO and dK += dS^T Q in registers
//               (fixed order, so which workgroup takes a tile never changes the result).
// All products are MFMA with fp32 accumulation.  dS (in dQ = dS K and dK = dS^T Q) enters
// as a bf16 hi + lo pair (about 16 bits): on peaked rows dS is a difference of nearly
// equal terms, and a single bf16 rounding would be visible in the gradients.  P (in
// dV = P^T dO, where a key that many queries attend to sums thousands of products) enters
// as one fp16 rounding (P <= 1) against an fp16 copy of dO that k_dq writes; a key block
// whose list holds a query block with dO beyond fp16's range, or whose V is beyond it,
// takes bf16 dO with P as a bf16 hi + lo pair.  dP = dO V^T runs on the same operand
// format as dO (V converted in registers; both conversions are exact).
#include "attn_tiles.h"
#include "spa_internal.h"

namespace spa {

// ------------------------------------------------------------------------------------
// column lists
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_bitmap(const int32_t* __restrict__ kv_idx,
                                               const int32_t* __restrict__ kv_cnt, int nqb,
                                               int nkb, int nw, uint32_t* __restrict__ bits) {
  __shared__ uint32_t words[64];
  const int bh = blockIdx.y, i = blockIdx.x, t = threadIdx.x;
  words[t] = 0u;
  __syncthreads();
  const size_t row = (size_t)bh * nqb + i;
  const int cnt = kv_cnt[row];
  const int32_t* list = kv_idx + row * nkb;
  for (int e = t; e < cnt; e += 64) {
    const int j = list[e];
    if ((unsigned)j < (unsigned)nkb) atomicOr(&words[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (t < nw) bits[((size_t)bh * nw + t) * nqb + i] = words[t];
}

// k_dkdv's work queues: eight per-XCD ticket counters, one for the remainder, and the
// count of workgroups that have finished.
constexpr int kDkdvCounters = 10;

// Column lists, 32 key blocks of one head per workgroup, and the dispatch order of their
// dK/dV workgroups: within these 32 neighbouring key blocks the longest lists go first
// (ranked by length, ties by position, so the order is deterministic).  The workgroups
// that start last on an XCD are then short ones, while the key blocks that run side by
// side stay neighbours that read the same Q and dO tiles from L2.  The order affects only
// scheduling, never results.
__global__ __launch_bounds__(256) void k_collists(const uint32_t* __restrict__ bits, int nqb,
                                                  int nkb, int nw, int32_t* __restrict__ q_idx,
                                                  int32_t* __restrict__ q_cnt,
                                                  int32_t* __restrict__ order,
                                                  int32_t* __restrict__ ctr) {
  extern __shared__ uint32_t colw[];  // [nqb]
  __shared__ int32_t lens[32];
  const int bh = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  if (w == 0 && bh == 0 && t < kDkdvCounters) ctr[t] = 0;  // k_dkdv's work queues
  const uint32_t* src = bits + ((size_t)bh * nw + w) * nqb;
  for (int x = t; x < nqb; x += 256) colw[x] = src[x];
  __syncthreads();
  const int lane = t & 63, wv = t >> 6;
  for (int bb = 0; bb < 8; ++bb) {
    const int b = wv * 8 + bb;
    const int j = w * 32 + b;
    if (j >= nkb) break;
    int32_t* out = q_idx + ((size_t)bh * nkb + j) * nqb;
    int base = 0;
    for (int i0 = 0; i0 < nqb; i0 += 64) {
      const int i = i0 + lane;
      const bool on = i < nqb && ((colw[min(i, nqb - 1)] >> b) & 1u);
      const unsigned long long ball = __ballot(on);
      const int before = __popcll(ball & ((1ull << lane) - 1ull));
      if (on) out[base + before] = i;
      base += __popcll(ball);
    }
    if (lane == 0) {
      q_cnt[(size_t)bh * nkb + j] = base;
      lens[b] = base;
    }
  }
  __syncthreads();
  const int nb = min(32, nkb - w * 32);
  if (t < nb) {
    int rank = 0;
    for (int y = 0; y < nb; ++y) rank += (lens[y] > lens[t] || (lens[y] == lens[t] && y < t)) ? 1 : 0;
    const size_t first = (size_t)bh * nkb + w * 32;
    order[first + rank] = (int32_t)(first + t);
  }
}

// The dK/dV pass's fp16 flag of each key block: 1 where its V is not to be read through an
// fp16 copy (f16_block_ok over the block's 64 rows), else 0; k_dq then also sets it where a
// listed query block's dO is not.  One workgroup per (b, h, key block), 16-byte loads.
template <int D>
__global__ __launch_bounds__(256) void k_vflag(const uint16_t* __restrict__ v, int N, int nkb,
                                               int32_t* __restrict__ kvflag) {
  __shared__ uint32_t wbits[4];
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int rows = min(kBlkK, N - j * kBlkK);
  const uint16_t* vb = v + ((size_t)bh * N + (size_t)j * kBlkK) * D;
  F16Range r;
#pragma unroll
  for (int u = 0; u < kBlkK * D / 8 / 256; ++u) {
    const int x = t + 256 * u;
    if (x * 8 < rows * D) r.add(*reinterpret_cast<const uint4*>(vb + 8 * (size_t)x));
  }
  const uint32_t wb = wave_or4(r.bits());
  if ((t & 63) == 0) wbits[t >> 6] = wb;
  __syncthreads();
  if (t == 0)
    kvflag[(size_t)bh * nkb + j] = f16_block_ok(wbits[0] | wbits[1] | wbits[2] | wbits[3]) ? 0 : 1;
}

// ------------------------------------------------------------------------------------
// dK, dV: one workgroup of 8 wavefronts per CU, resident for the whole launch: it takes
// key blocks from work queues (per-XCD contiguous ranges of the dispatch order) until all
// are done.  A launch of one workgroup per key block paid, per block, the hardware
// dispatcher's wait for a free CU on each shader engine in turn (1.5k to 8k cycles
// depending on the engine, measured with per-workgroup clock stamps).  Each key block's
// query-block list is walked in stages of 64 query rows; Q and dO of each stage stream
// into a ring of three LDS slots with direct buffer->LDS loads, one stage ahead.
//
// The 64 keys x 64 rows of a stage split into four units (32 keys x 32 rows).  Each
// unit has two wavefronts with different jobs, placed so that they share a SIMD:
//   producer (waves 0-3):  S = Q K^T (K fragments in registers), P = exp2(S c - lse2),
//                          P to LDS (fp32), dV += P^T dO (P in fp16, or a bf16 pair);
//   consumer (waves 4-7):  one stage behind: dP = dO V^T (V fragments in registers),
//                          P from LDS, dS = P (dP - D), dK += dS^T Q with dS as a bf16
//                          hi + lo pair.
// The two jobs of a SIMD interleave freely (one wavefront's exp and conversions run
// while the other's MFMAs execute).  Each wavefront's partial sums cover its 32-row
// slab of every stage; the two slabs are added at the end in a fixed order.
// ------------------------------------------------------------------------------------
struct DkdvSrc {
  u32x4 q, dout, lse2, dsum;
};

// Loads of stage st (64 query rows of query block qb) into one ring slot: the Q and dO
// tiles and the lse2 / D rows (one 4-byte transfer per lane, waves 2 and 3; the side
// arrays are padded to whole query blocks).  Q and dO rows at or beyond N read as zeros;
// their lse2 of +inf makes their P exactly 0.
template <int D, int BQ>
__device__ __forceinline__ void dkdv_load_stage(const DkdvSrc& src, int qb, int st, int w,
                                                int lane, uint16_t* tq, float* sd,
                                                const TileLanes<D, 64, 8>& tl) {
  constexpr int HR = 64, HPB = BQ / HR;
  const int row0 = qb * BQ + HR * (st % HPB);
  tile_load_lds_rsrc<D, HR, 8>(src.q, row0, tq, tl);
  tile_load_lds_rsrc<D, HR, 8>(src.dout, row0, tq + HR * D, tl);
  if (w == 2) dma4(src.lse2, lane * 4, row0 * 4, lds_addr(sd));
  if (w == 3) dma4(src.dsum, lane * 4, row0 * 4, lds_addr(sd + HR));
}

// Both jobs issue their LDS reads in batches ahead of the MFMAs that consume them
// (sched_barrier fences keep the compiler from interleaving each read with its MFMA, which
// would expose the LDS latency once per k-step).
#define SPA_FENCE() __builtin_amdgcn_sched_barrier(0)

// Producer, first half: S and P for the unit; P goes to LDS for the consumer.
template <int D, bool TAIL>
__device__ __forceinline__ void dkdv_scores(const uint16_t* tq, const float* sd, float* pw,
                                            const bf16x8 (&kf)[D / 16], int r0, int lane,
                                            float kmask, float scale_log2, f32x16& sacc,
                                            bf16x8 (&ob0)[D / 32]) {
  constexpr int KS = D / 16;
  const int h = lane >> 5;
  bf16x8 a[KS];
  float4 lv[4];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) a[kk] = lds_rowfrag<D>(tq, r0, kk, lane);
  // element e is query row r0 + acc_row(e, h): runs of 4 consecutive rows
#pragma unroll
  for (int g = 0; g < 4; ++g)
    lv[g] = *reinterpret_cast<const float4*>(sd + r0 + 16 * (g >> 1) + 8 * h + 4 * (g & 1));
  SPA_FENCE();
  sacc = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) sacc = mfma32(a[kk], kf[kk], sacc);
  // the dO^T fragments of the first half of dV += P^T dO do not depend on P: their
  // transpose reads are issued here and land while the exponentials run
#pragma unroll
  for (int db = 0; db < D / 32; ++db) ob0[db] = lds_colfrag<D>(tq + 64 * D, r0, 32 * db, lane);
  SPA_FENCE();
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    sacc[4 * g + 0] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 0], scale_log2, -lv[g].x));
    sacc[4 * g + 1] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 1], scale_log2, -lv[g].y));
    sacc[4 * g + 2] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 2], scale_log2, -lv[g].z));
    sacc[4 * g + 3] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * g + 3], scale_log2, -lv[g].w));
  }
  if constexpr (TAIL) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] *= kmask;
  }
  // lane-contiguous float4 groups: the consumer lane with the same index reads them back
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<float4*>(pw + (g * 64 + lane) * 4) =
        make_float4(sacc[4 * g], sacc[4 * g + 1], sacc[4 * g + 2], sacc[4 * g + 3]);
}

// Producer, second half: dV += P^T dO.
template <int D>
__device__ __forceinline__ void dkdv_dv(const uint16_t* tq, const f32x16& p, f32x16 (&acc)[D / 32],
                                        int r0, int lane, const bf16x8 (&ob0)[D / 32]) {
  constexpr int DB = D / 32, HR = 64;
  const uint16_t* dOb = tq + HR * D;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    bf16x8 ob[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
      ob[db] = kq == 0 ? ob0[db] : lds_colfrag<D>(dOb, r0 + 16 * kq, 32 * db, lane);
    bf16x8 ph, pl;
    split_bf16x8(p, kq, ph, pl);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma32(ph, ob[db], acc[db]);
      acc[db] = mfma32(pl, ob[db], acc[db]);
    }
  }
}

// Producer, second half, fp16 form: dV += P^T dO with P as one fp16 rounding (P <= 1)
// against the fp16 copy of dO held in the stage slot.
template <int D>
__device__ __forceinline__ void dkdv_dv16(const uint16_t* tq, const f32x16& p,
                                          f32x16 (&acc)[D / 32], int r0, int lane,
                                          const bf16x8 (&ob0)[D / 32]) {
  constexpr int DB = D / 32, HR = 64;
  const uint16_t* dOb = tq + HR * D;
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    bf16x8 ob[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
      ob[db] = kq == 0 ? ob0[db] : lds_colfrag<D>(dOb, r0 + 16 * kq, 32 * db, lane);
    const f16x8 ph = to_f16x8(p, kq);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      acc[db] = mfma32h(ph, __builtin_bit_cast(f16x8, ob[db]), acc[db]);
  }
}

template <int D>
__device__ __forceinline__ void dkdv_rowfrags(const uint16_t* tile, int r0, int lane,
                                              bf16x8 (&a)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) a[kk] = lds_rowfrag<D>(tile, r0, kk, lane);
}

// Consumer, first half: dP for the unit from dO row fragments read into registers.
template <int D>
__device__ __forceinline__ void dkdv_dp(const bf16x8 (&a)[D / 16], const bf16x8 (&vf)[D / 16],
                                        f32x16& dp) {
  constexpr int KS = D / 16;
  dp = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) dp = mfma32(a[kk], vf[kk], dp);
}

// The same with fp16 dO rows and fp16 V (both exact conversions of the bf16 data).
template <int D>
__device__ __forceinline__ void dkdv_dp16(const bf16x8 (&a)[D / 16], const bf16x8 (&vf)[D / 16],
                                          f32x16& dp) {
  constexpr int KS = D / 16;
  dp = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    dp = mfma32h(__builtin_bit_cast(f16x8, a[kk]), __builtin_bit_cast(f16x8, vf[kk]), dp);
}

// The consumer's per-row D values reach the accumulator elements by a row broadcast: lane
// l reads the value of slab row side_row(l), and element e of every lane in a 16-lane row
// takes lane e of that row (DPP row_newbcast, folded into the subtraction), one 4-byte LDS
// read per lane in place of 64 bytes.  Accumulator element e = 4g + i of the lanes with
// h = l / 32 holds query row 16 (g / 2) + 8 h + 4 (g % 2) + i of the slab (the order in which
// the row fragments are read).  The producer keeps its 64-byte lse reads: there the
// broadcast would cost a move per element, which measured slower than the reads.
__device__ __forceinline__ int side_row(int lane) {
  const int n = lane & 15;
  return 16 * (n >> 3) + 8 * (lane >> 5) + 4 * ((n >> 2) & 1) + (n & 3);
}

template <int E>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + E, 0xF, 0xF, false));
}

// dS = P (dP - D), element by element (the broadcast needs a constant lane index).
template <int E = 0>
__device__ __forceinline__ void dkdv_ds(f32x16& dp, const f32x4 (&pv)[4], float dl) {
  if constexpr (E < 16) {
    dp[E] = pv[E / 4][E % 4] * (dp[E] - row_bcast<E>(dl));
    dkdv_ds<E + 1>(dp, pv, dl);
  }
}

// Consumer, second half: dS = P (dP - D) with P from the producer, dK += dS^T Q.
template <int D>
__device__ __forceinline__ void dkdv_dk(const uint16_t* tq, const float* sd, const float* pr,
                                        f32x16& dp, f32x16 (&acc)[D / 32], int r0, int lane) {
  constexpr int DB = D / 32, HR = 64;
  f32x4 pv[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) pv[g] = *reinterpret_cast<const f32x4*>(pr + (g * 64 + lane) * 4);
  const float dl = sd[HR + r0 + side_row(lane)];
  bf16x8 qb[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) qb[db] = lds_colfrag<D>(tq, r0, 32 * db, lane);
  SPA_FENCE();
  dkdv_ds(dp, pv, dl);
  __builtin_amdgcn_s_setprio(0);  // the dK products issue at the producer's priority
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    if (kq == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db) qb[db] = lds_colfrag<D>(tq, r0 + 16, 32 * db, lane);
    }
    bf16x8 dh, dl;
    split_bf16x8(dp, kq, dh, dl);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma32(dh, qb[db], acc[db]);
      acc[db] = mfma32(dl, qb[db], acc[db]);
    }
  }
}

// Writes one wavefront's 32 x D block of dK or dV: element e of accumulator db goes to row
// 8*(e/4) + e%4 (relative to the lane's first row), column 32*db; rows from nrow on are
// past the end of the sequence.  The row check is taken only in the last key block
// (tail, uniform over the workgroup), the one block that can hold such rows.
template <int D, typename T>
__device__ __forceinline__ void dkdv_store(T* o, const f32x16 (&acc)[D / 32], bool tail,
                                           int nrow) {
  if (!tail) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[(8 * (e >> 2) + (e & 3)) * D + 32 * db] = (T)acc[db][e];
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (8 * (e >> 2) + (e & 3) < nrow) o[(8 * (e >> 2) + (e & 3)) * D + 32 * db] = (T)acc[db][e];
  }
}

template <int D, int BQ>
__global__ __launch_bounds__(512, 1) void k_dkdv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2p, const float* __restrict__ dsum,
    const int32_t* __restrict__ q_idx, const int32_t* __restrict__ q_cnt, int N, int npad,
    int nqb, int nkb, int total, float scale_log2, float scale, void* __restrict__ dk_out,
    void* __restrict__ dv_out, int grad_bf16, const uint16_t* __restrict__ do16,
    const int32_t* __restrict__ kvflag, const int32_t* __restrict__ order,
    int32_t* __restrict__ ctr) {
  constexpr int DB = D / 32;
  constexpr int KS = D / 16;
  constexpr int HR = 64;                 // query rows per stage
  constexpr int HPB = BQ / HR;           // stages per query block
  constexpr int SLOT = 2 * HR * D;       // Q | dO of one stage
  __shared__ __align__(16) uint16_t tiles[3][SLOT];
  __shared__ __align__(16) float side[3][2 * HR];     // [slot][lse2 | D]
  __shared__ __align__(16) float pbuf[2][4 * 1024];   // [stage parity][unit][32x32] fp32
  // the query-block list, staged once: reading it from LDS keeps scalar loads (which
  // complete out of order) out of the loop, so LDS waits can stay partial
  __shared__ int32_t lst[kMaxBlocks];
  static_assert(2 * DB * 16 * 64 * 4 <= SLOT * 2, "reduction buffer reuses a slot");
  // the next key block: {tile (b*h*nkb + j) or -1, list length, first query block, dO flag}
  __shared__ int32_t meta[4];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int role = w >> 2;               // 0 producer, 1 consumer
  const int unit = w & 3;
  const int kh = unit & 1, r0 = 32 * (unit >> 1);
  const TileLanes<D, 64, 8> tl;

  // Work queues, served by one lane (threadIdx 128: wavefront 2, idle while the first
  // slab's wavefronts write the results).  Position t of the dispatch order is ticket t;
  // queue x (x < 8) hands out the contiguous range [x * per, (x + 1) * per) of positions,
  // queue 8 the remainder.  A workgroup draws from queue blockIdx % 8 (workgroups are dealt
  // to the XCDs in turn, so each XCD walks one contiguous range, whose neighbouring key
  // blocks read the same Q and dO tiles), then from the others in turn, so every ticket is
  // taken once whichever workgroups run.
  constexpr int kQueueLane = 128;
  const int whole = total - total % 8, per = whole / 8;
  const int home = blockIdx.x & 7;
  int qo = 0;  // queues this workgroup has found empty
  auto queue = [&](int o) { return o < 8 ? (home + o) & 7 : 8; };
  // the next ticket's key block and what its prologue needs first, into meta
  auto fetch_next = [&]() {
    int raw = atomicAdd(ctr + queue(qo), 1), tix = -1;
    for (;;) {
      const int qi = queue(qo);
      if (raw >= 0 && raw < (qi < 8 ? per : total - whole)) {
        tix = (qi < 8 ? qi * per : whole) + raw;
        break;
      }
      if (++qo > 8) break;
      raw = atomicAdd(ctr + queue(qo), 1);
    }
    int tile = -1, n = 0, first = 0, flag = 0;
    if (tix >= 0) {
      tile = order[tix];
      n = q_cnt[tile];
      first = q_idx[(size_t)tile * nqb];
      flag = kvflag[tile];
    }
    meta[0] = tile;
    meta[1] = n;
    meta[2] = first;
    meta[3] = flag;
  };
  if (threadIdx.x == kQueueLane) fetch_next();
  __syncthreads();
  int tile_id = __builtin_amdgcn_readfirstlane(meta[0]);
  while (tile_id >= 0) {
  const int cnt = __builtin_amdgcn_readfirstlane(meta[1]);
  const int first = __builtin_amdgcn_readfirstlane(meta[2]);
  const bool do_flag = __builtin_amdgcn_readfirstlane(meta[3]) != 0;
  const int bh = tile_id / nkb;
  const int j = tile_id - bh * nkb;
  const size_t head = (size_t)bh * N * D;
  const int key = j * kBlkK + 32 * kh + c;  // this lane's key (B operand column)
  const bool tail = j * kBlkK + kBlkK > N;  // keys at or beyond N exist only here
  const float kmask = key < N ? 1.f : 0.f;

  const int nst = cnt * HPB;
  DkdvSrc src;
  src.q = make_rsrc(q + head, (uint32_t)N * D * 2);
  // dO is staged from its fp16 copy unless this key block's V or a listed query block's dO
  // is not to be read through fp16 (do_flag; f16_block_ok): then from bf16 dO, with P as a
  // bf16 pair
  src.dout = make_rsrc((do_flag ? dout : do16) + head, (uint32_t)N * D * 2);
  src.lse2 = make_rsrc(lse2p + (size_t)bh * npad, (uint32_t)npad * 4);
  src.dsum = make_rsrc(dsum + (size_t)bh * npad, (uint32_t)npad * 4);
  // every transfer of the block at once: stage 0, the list (64 entries per wavefront and
  // transfer; entries past the count read as zeros), and this key block's K and V rows,
  // each one contiguous 64-row block, into the slot that the loop fills only in its second
  // step, after the first step's barrier, by which every wavefront has read its rows
  // (rows at or beyond N read as zeros: their P is masked).  Gathering the operand rows
  // straight from memory, 32 bytes of each of 32 rows per load, took three times as long.
  if (nst > 0) dkdv_load_stage<D, BQ>(src, first, 0, w, lane, tiles[0], side[0], tl);
  {
    const u32x4 lrs = make_rsrc(q_idx + (size_t)tile_id * nqb, (uint32_t)cnt * 4);
    for (int ch = w; ch * 64 < cnt; ch += 8)
      dma4(lrs, (uint32_t)(ch * 64 + lane) * 4, 0, lds_addr(lst + ch * 64));
  }
  tile_load_lds_rsrc<D, 64, 8>(make_rsrc(k + head, (uint32_t)N * D * 2), j * kBlkK, tiles[2], tl);
  tile_load_lds_rsrc<D, 64, 8>(make_rsrc(v + head, (uint32_t)N * D * 2), j * kBlkK,
                               tiles[2] + 64 * D, tl);
  f32x16 acc[DB];  // producer: dV; consumer: dK (unscaled)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  wait_vmem();  // nothing vector-memory is pending inside the loop
  __syncthreads();
  auto list_at = [&](int st) {
    return __builtin_amdgcn_readfirstlane(lst[max(0, min(st / HPB, cnt - 1))]);
  };
  bf16x8 bf[KS];  // producer: K row of this lane's key; consumer: V row
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    bf[kk] = *reinterpret_cast<const bf16x8*>(tiles[2] + role * 64 * D +
                                              Tile<D>::off(32 * kh + c, 16 * kk + 8 * h));
  // the fp16 dV path, unless the key block's V (classified by k_collists) or a listed
  // query block's dO (flagged by k_dq) is not to be read through fp16
  const bool use16 = !do_flag;

  // One step: loads of stage st+1 into the next slot, producer on stage st, consumer on
  // stage st-1.  Each job runs its own copy of the loop (same barriers), so that neither
  // keeps the other's loop-invariant addresses alive.
// The query block of the next stage is read from LDS one step ahead and taken into a
// scalar register after the barrier, so that no step waits for that read.
#define SPA_DKDV_LOOP(...)                                                                   \
  {                                                                                        \
    int cur = 0, prev = 2;                                                                 \
    int qn = list_at(1);                                                                   \
    for (int st = 0; st <= nst; ++st) {                                                    \
      const int nxt = cur == 2 ? 0 : cur + 1;                                              \
      if (st + 1 < nst) dkdv_load_stage<D, BQ>(src, qn, st + 1, w, lane, tiles[nxt], side[nxt], tl); \
      const int qn_v = lst[max(0, min((st + 2) / HPB, cnt - 1))];                           \
      __VA_ARGS__;                                                                         \
      wait_vmem();                                                                         \
      __syncthreads();                                                                     \
      qn = __builtin_amdgcn_readfirstlane(qn_v);                                           \
      prev = cur;                                                                          \
      cur = nxt;                                                                           \
    }                                                                                      \
  }
  // Issue priority: the consumer's dP and dS phase goes first whenever both wavefronts of
  // a SIMD are ready (set at each consumer stage; its dK products and the producer's work
  // then share by age).  Clock stamps of the stage loop: with equal priority the producers
  // waited 35 % of the loop at the barrier and the consumers 5 %; with the whole consumer
  // stage first, 9 % and 25 %; this split is the fastest of the three.
  if (use16) {
    if (role == 0 && tail) {
      SPA_DKDV_LOOP(if (st < nst) {
        f32x16 p;
        bf16x8 ob0[DB];
        dkdv_scores<D, true>(tiles[cur], side[cur], pbuf[st & 1] + unit * 1024, bf, r0, lane,
                             kmask, scale_log2, p, ob0);
        dkdv_dv16<D>(tiles[cur], p, acc, r0, lane, ob0);
      })
    } else if (role == 0) {
      SPA_DKDV_LOOP(if (st < nst) {
        f32x16 p;
        bf16x8 ob0[DB];
        dkdv_scores<D, false>(tiles[cur], side[cur], pbuf[st & 1] + unit * 1024, bf, r0, lane,
                              kmask, scale_log2, p, ob0);
        dkdv_dv16<D>(tiles[cur], p, acc, r0, lane, ob0);
      })
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)  // V to fp16 (checked above)
        bf[kk] = __builtin_bit_cast(bf16x8, bf16x8_bits_to_f16(__builtin_bit_cast(uint4, bf[kk])));
      SPA_DKDV_LOOP(if (st >= 1) {
        __builtin_amdgcn_s_setprio(1);
        bf16x8 a[KS];
        dkdv_rowfrags<D>(tiles[prev] + HR * D, r0, lane, a);
        SPA_FENCE();
        f32x16 dp;
        dkdv_dp16<D>(a, bf, dp);
        dkdv_dk<D>(tiles[prev], side[prev], pbuf[(st - 1) & 1] + unit * 1024, dp, acc, r0,
                   lane);
      })
    }
  } else if (role == 0 && tail) {  // keys at or beyond N exist only in the last key block
    SPA_DKDV_LOOP(if (st < nst) {
      f32x16 p;
      bf16x8 ob0[DB];
      dkdv_scores<D, true>(tiles[cur], side[cur], pbuf[st & 1] + unit * 1024, bf, r0, lane,
                           kmask, scale_log2, p, ob0);
      dkdv_dv<D>(tiles[cur], p, acc, r0, lane, ob0);
    })
  } else if (role == 0) {
    SPA_DKDV_LOOP(if (st < nst) {
      f32x16 p;
      bf16x8 ob0[DB];
      dkdv_scores<D, false>(tiles[cur], side[cur], pbuf[st & 1] + unit * 1024, bf, r0, lane,
                            kmask, scale_log2, p, ob0);
      dkdv_dv<D>(tiles[cur], p, acc, r0, lane, ob0);
    })
  } else {
    SPA_DKDV_LOOP(if (st >= 1) {
      __builtin_amdgcn_s_setprio(1);
      bf16x8 a[KS];
      dkdv_rowfrags<D>(tiles[prev] + HR * D, r0, lane, a);
      SPA_FENCE();
      f32x16 dp;
      dkdv_dp<D>(a, bf, dp);
      dkdv_dk<D>(tiles[prev], side[prev], pbuf[(st - 1) & 1] + unit * 1024, dp, acc, r0, lane);
    })
  }
#undef SPA_DKDV_LOOP
  __builtin_amdgcn_s_setprio(0);

  // ---- add the two row slabs (fixed order) and write ------------------------------------
  // [role][DB*16][lane], lane-contiguous; key half 0 in slot 0, key half 1 in slot 1
  float* red = reinterpret_cast<float*>(tiles[kh]);
  const int rbase = role * (DB * 16);
  if (r0 != 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(rbase + db * 16 + e) * 64 + lane] = acc[db][e];
  }
  __syncthreads();
  // the next key block is fetched while the other slab's wavefronts add and write
  if (threadIdx.x == kQueueLane) fetch_next();
  if (r0 == 0) {
    const float f = role ? scale : 1.f;
    // every partial sum is read before the first store, so that the reads share one wait
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc[db][e] = (acc[db][e] + red[(rbase + db * 16 + e) * 64 + lane]) * f;
    // accumulator element e: key row 8*(e/4) + 4*h + e%4 of this unit's 32 keys, column c;
    // only the last key block has rows at or beyond N
    const int krow0 = j * kBlkK + 32 * kh + 4 * h;
    const size_t base = head + (size_t)krow0 * D + c;
    void* out = role ? dk_out : dv_out;
    if (grad_bf16)
      dkdv_store<D>(reinterpret_cast<__bf16*>(out) + base, acc, tail, N - krow0);
    else
      dkdv_store<D>(reinterpret_cast<float*>(out) + base, acc, tail, N - krow0);
  }
  __syncthreads();  // the slots and the list are refilled next; meta is written
  tile_id = __builtin_amdgcn_readfirstlane(meta[0]);
  }
  // the last workgroup to finish leaves the counters at zero for the next launch
  if (threadIdx.x == 0 && atomicAdd(ctr + 9, 1) == (int)gridDim.x - 1) {
#pragma unroll
    for (int x = 0; x < kDkdvCounters; ++x) ctr[x] = 0;
  }
}

// ------------------------------------------------------------------------------------
// dQ: one workgroup per query block (XCD-contiguous order), one wavefront per 32 rows;
// K and V tiles staged like the forward pass.
// ------------------------------------------------------------------------------------
// One kept tile for this wave's 32 query rows: per 32-key slab S and dP (K, V fragments
// read in batches of four k-steps), dS = P (dP - D), dQ += dS K with dS as a bf16 hi + lo
// pair.  K and V rows at or beyond N were staged as zeros; TAIL masks their dS.
template <int D, bool TAIL>
__device__ __forceinline__ void dq_tile(const uint16_t* Ks, const uint16_t* Vs, int key0, int N,
                                        const bf16x8 (&qf)[D / 16], const bf16x8 (&df)[D / 16],
                                        float lse2, float dq_sum, f32x16 (&acc)[D / 32],
                                        float scale_log2, int lane) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += 4) {
      bf16x8 ka[4], va[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ka[u] = lds_rowfrag<D>(Ks, 32 * kb, k0 + u, lane);
        va[u] = lds_rowfrag<D>(Vs, 32 * kb, k0 + u, lane);
      }
      SPA_FENCE();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s = mfma32(ka[u], qf[k0 + u], s);
        dp = mfma32(va[u], df[k0 + u], dp);
      }
    }
    // the K^T fragments of the first half of dQ += dS K do not depend on the softmax:
    // their transpose reads are issued first and land while the exponentials run
    bf16x8 kt0[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) kt0[db] = lds_colfrag<D>(Ks, 32 * kb, 32 * db, lane);
    SPA_FENCE();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, -lse2));
      dp[e] = pe * (dp[e] - dq_sum);
    }
    if constexpr (TAIL) {
      const int lim = N - key0 - 32 * kb - 8 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (16 * (e >> 3) + (e & 7) >= lim) dp[e] = 0.f;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 dh, dl;
      split_bf16x8(dp, half, dh, dl);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 kt =
            half == 0 ? kt0[db] : lds_colfrag<D>(Ks, 32 * kb + 16 * half, 32 * db, lane);
        acc[db] = mfma32(kt, dh, acc[db]);
        acc[db] = mfma32(kt, dl, acc[db]);
      }
    }
  }
}

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 2) void k_dq(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ o_lo, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ lse2p, float* __restrict__ dsum,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, int N, int npad,
    int nqb, int nkb, int total, float scale_log2, float scale, void* __restrict__ dq_out,
    int grad_bf16, uint16_t* __restrict__ do16, int32_t* __restrict__ kvflag) {
  constexpr int NT = BQ * 2;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __align__(16) uint16_t smem[2][2][Tile<D>::ELEMS];  // [buf][K|V]
  __shared__ int32_t lst[kMaxBlocks];  // the key-block list (keeps scalar loads out of the loop)
  __shared__ uint32_t wbits[NT / 64];  // fp16 range classes of dO, per wavefront
  __shared__ float dsh[BQ];            // D of each row of the block

  const int tile_id = xcd_remap(blockIdx.x, total);
  const int bh = tile_id / nqb;
  const int i = tile_id - bh * nqb;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const u32x4 krs = make_rsrc(k + head, (uint32_t)N * D * 2);
  const u32x4 vrs = make_rsrc(v + head, (uint32_t)N * D * 2);
  const int32_t* list = kv_idx + ((size_t)bh * nqb + i) * nkb;
  // the lists are trusted; the clamp only keeps a corrupt count inside the LDS list
  const int cnt = min(max(kv_cnt[(size_t)bh * nqb + i], 0), nkb);
  const int j0 = cnt > 0 ? list[0] : 0;
  const TileLanes<D, kBlkK, NT / 64> tl;
  // Everything the prologue reads is requested at once: the first K and V tiles, this
  // block's dO rows (by DMA into the second buffer, which the loop fills only after its
  // first step; rows at or beyond N read as zeros), the list, the Q rows of this lane, and
  // O (with its residual) in 16-byte chunks, a row to CPR consecutive lanes.  dO's operand
  // fragments, D = rowsum(dO * O), the fp16 copy of dO and its range classes then come
  // from the staged rows: gathering operand rows straight from memory (32 bytes of each
  // of 32 rows per load) made this prologue several times longer.
  if (cnt > 0) {
    tile_load_lds_rsrc<D, kBlkK, NT / 64>(krs, j0 * kBlkK, smem[0][0], tl);
    tile_load_lds_rsrc<D, kBlkK, NT / 64>(vrs, j0 * kBlkK, smem[0][1], tl);
  }
  uint16_t* dot = &smem[1][0][0];  // dO rows of this block, [BQ][D], Tile swizzle
  static_assert(BQ * D <= 2 * Tile<D>::ELEMS, "dO rows fit the second buffer");
  {
    const u32x4 drs = make_rsrc(dout + head, (uint32_t)N * D * 2);
#pragma unroll
    for (int hq = 0; hq < BQ / kBlkK; ++hq)
      tile_load_lds_rsrc<D, kBlkK, NT / 64>(drs, i * BQ + hq * kBlkK, dot + hq * Tile<D>::ELEMS,
                                            tl);
  }
  for (int x = threadIdx.x; x < cnt; x += NT) lst[x] = list[x];
  auto blk = [&](int t) { return __builtin_amdgcn_readfirstlane(lst[min(t, cnt - 1)]); };

  const int qrow = i * BQ + 32 * wv + c;
  const bool qvalid = qrow < N;
  const size_t qoff = head + (size_t)min(qrow, N - 1) * D + 8 * h;
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(q + qoff + 16 * kk);
  const float lse2 = qvalid ? lse[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPP = NT / CPR;  // rows per pass of the workgroup
  constexpr int NP = BQ / RPP;   // passes
  const int ch = threadIdx.x % CPR, rr = threadIdx.x / CPR;
  uint4 oc[NP], lc[NP];  // chunk ch of O and O_lo, rows rr + RPP * u
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const size_t off = head + (size_t)min(i * BQ + rr + RPP * u, N - 1) * D + 8 * ch;
    oc[u] = *reinterpret_cast<const uint4*>(o + off);
    lc[u] = o_lo ? *reinterpret_cast<const uint4*>(o_lo + off) : make_uint4(0u, 0u, 0u, 0u);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  wait_vmem();  // nothing vector-memory is pending inside the loop
  __syncthreads();  // dO rows and the list staged
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    df[kk] = *reinterpret_cast<const bf16x8*>(dot + Tile<D>::off(32 * wv + c, 16 * kk + 8 * h));
  // D in fp32 (O = o + o_lo when the forward pass supplied its residual), the fp16 copy
  // of dO for k_dkdv's dV = P^T dO, and the copy's range classes
  F16Range dr;
  float dpart[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int row = i * BQ + rr + RPP * u;
    const uint4 g = *reinterpret_cast<const uint4*>(dot + Tile<D>::off(rr + RPP * u, 8 * ch));
    const uint32_t wa[4] = {oc[u].x, oc[u].y, oc[u].z, oc[u].w};
    const uint32_t wl[4] = {lc[u].x, lc[u].y, lc[u].z, lc[u].w};
    const uint32_t wg[4] = {g.x, g.y, g.z, g.w};
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o0 = bf16_bits_to_f32(wa[e] & 0xFFFFu) + bf16_bits_to_f32(wl[e] & 0xFFFFu);
      const float o1 = bf16_bits_to_f32(wa[e] >> 16) + bf16_bits_to_f32(wl[e] >> 16);
      a = fmaf(o0, bf16_bits_to_f32(wg[e] & 0xFFFFu), a);
      a = fmaf(o1, bf16_bits_to_f32(wg[e] >> 16), a);
    }
    dpart[u] = row < N ? a : 0.f;
    if (row < N) {
      dr.add(g);
      *reinterpret_cast<uint4*>(do16 + head + (size_t)row * D + 8 * ch) = bf16x8_bits_to_f16(g);
    }
  }
  // each row's sum over its CPR chunks (lanes that differ in the low bits), a fixed tree
#pragma unroll
  for (int u = 0; u < NP; ++u)
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) dpart[u] += __shfl_xor(dpart[u], m, 64);
  if (ch == 0) {  // padded side arrays for k_dkdv; rows at or beyond N get D = 0
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      dsh[rr + RPP * u] = dpart[u];
      dsum[(size_t)bh * npad + i * BQ + rr + RPP * u] = dpart[u];
    }
  }
  if (h == 0) lse2p[(size_t)bh * npad + qrow] = lse2;  // +inf past N: P is exactly 0 there
  const uint32_t rbits = wave_or4(dr.bits());
  if (lane == 0) wbits[wv] = rbits;
  __syncthreads();  // D and the range classes staged; the second buffer is free again
  const float dq_sum = dsh[32 * wv + c];
  {
    uint32_t all = 0;
#pragma unroll
    for (int x = 0; x < NT / 64; ++x) all |= wbits[x];
    // a block of dO that its fp16 copy does not carry (f16_block_ok): every key block of
    // this list then takes bf16 dO in k_dkdv
    if (!f16_block_ok(all))
      for (int x = threadIdx.x; x < cnt; x += NT) kvflag[(size_t)bh * nkb + lst[x]] = 1;
  }
  // only the last key block of the list can be partial: it gets its own instantiation of
  // the tile body after the loop, so that the loop carries no per-element selects
  const bool tail_last = cnt > 0 && blk(cnt - 1) * kBlkK + kBlkK > N;
  const int cnt_main = cnt - (tail_last ? 1 : 0);
  // the block index of the next tile is read from LDS one tile ahead and taken into a
  // scalar register after the barrier, so that no step waits for that read; the loop is
  // unrolled over the two buffers, so that every LDS address in a tile is a loop-invariant
  // register plus a constant offset
  int jn = cnt > 1 ? blk(1) : 0;
#define SPA_DQ_STEP(BUF)                                                                     \
  {                                                                                        \
    if (t + 1 < cnt) { /* the next tile streams into the other buffer meanwhile */         \
      tile_load_lds_rsrc<D, kBlkK, NT / 64>(krs, jn * kBlkK, smem[(BUF) ^ 1][0], tl);      \
      tile_load_lds_rsrc<D, kBlkK, NT / 64>(vrs, jn * kBlkK, smem[(BUF) ^ 1][1], tl);      \
    }                                                                                      \
    const int jn_v = lst[min(t + 2, cnt - 1)];                                             \
    dq_tile<D, false>(smem[BUF][0], smem[BUF][1], 0 /* read by the tail form only */, N,   \
                      qf, df, lse2, dq_sum, acc, scale_log2, lane);                        \
    wait_vmem();                                                                           \
    __syncthreads();                                                                       \
    jn = __builtin_amdgcn_readfirstlane(jn_v);                                             \
  }
  for (int t = 0;;) {
    if (t >= cnt_main) break;
    SPA_DQ_STEP(0)
    if (++t >= cnt_main) break;
    SPA_DQ_STEP(1)
    ++t;
  }
#undef SPA_DQ_STEP
  if (tail_last) {
    const int buf = cnt_main & 1;
    dq_tile<D, true>(smem[buf][0], smem[buf][1], blk(cnt_main) * kBlkK, N, qf, df, lse2, dq_sum,
                     acc, scale_log2, lane);
  }
  if (qvalid) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        const size_t off = head + (size_t)qrow * D + d0;
        const float x0 = acc[db][4 * g + 0] * scale, x1 = acc[db][4 * g + 1] * scale;
        const float x2 = acc[db][4 * g + 2] * scale, x3 = acc[db][4 * g + 3] * scale;
        if (grad_bf16) {
          const bf16x4 pk = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
          *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(dq_out) + off) = pk;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(dq_out) + off) =
              make_float4(x0, x1, x2, x3);
        }
      }
  }
}

// ------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------
static int n_words(const Geometry& g) { return (g.nkb + 31) / 32; }

static size_t n_pad(const Geometry& g) { return (size_t)g.nqb * g.blk_q; }

size_t bwd_workspace_bytes(const Geometry& g) {
  const size_t bh = (size_t)g.bh();
  return 2 * align_up(bh * n_pad(g) * sizeof(float), 256) +
         align_up(bh * n_words(g) * g.nqb * sizeof(uint32_t), 256) +
         align_up(bh * g.nkb * g.nqb * sizeof(int32_t), 256) +
         align_up(bh * g.nkb * sizeof(int32_t), 256) +
         align_up(bh * (size_t)g.N * g.d * sizeof(uint16_t), 256) +
         align_up(bh * g.nkb * sizeof(int32_t), 256) +
         align_up(bh * g.nkb * sizeof(int32_t), 256) +
         align_up(kDkdvCounters * sizeof(int32_t), 256);
}

void bwd_workspace_carve(const Geometry& g, void* ws, BwdArgs* a) {
  const size_t bh = (size_t)g.bh();
  char* p = static_cast<char*>(ws);
  a->dsum = reinterpret_cast<float*>(p);
  p += align_up(bh * n_pad(g) * sizeof(float), 256);
  a->lse2 = reinterpret_cast<float*>(p);
  p += align_up(bh * n_pad(g) * sizeof(float), 256);
  a->bits = reinterpret_cast<uint32_t*>(p);
  p += align_up(bh * n_words(g) * g.nqb * sizeof(uint32_t), 256);
  a->q_idx = reinterpret_cast<int32_t*>(p);
  p += align_up(bh * g.nkb * g.nqb * sizeof(int32_t), 256);
  a->q_cnt = reinterpret_cast<int32_t*>(p);
  p += align_up(bh * g.nkb * sizeof(int32_t), 256);
  a->do16 = reinterpret_cast<uint16_t*>(p);
  p += align_up(bh * (size_t)g.N * g.d * sizeof(uint16_t), 256);
  a->kvflag = reinterpret_cast<int32_t*>(p);
  p += align_up(bh * g.nkb * sizeof(int32_t), 256);
  a->order = reinterpret_cast<int32_t*>(p);
  p += align_up(bh * g.nkb * sizeof(int32_t), 256);
  a->ctr = reinterpret_cast<int32_t*>(p);
}

// Compute units of the current device (one dK/dV workgroup fits on each), cached per device.
static int cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int D, int BQ>
static hipError_t launch_bwd_t(const BwdArgs& a, unsigned stages, hipStream_t s) {
  const Geometry& g = a.g;
  const float sl2 = a.scale * kLog2e;
  const int npad = (int)n_pad(g);
  if (stages & 1u) {
    const int nw = n_words(g);
    hipLaunchKernelGGL(k_bitmap, dim3(g.nqb, (unsigned)g.bh()), dim3(64), 0, s, a.kv_idx,
                       a.kv_cnt, g.nqb, g.nkb, nw, a.bits);
    hipLaunchKernelGGL(k_collists, dim3(nw, (unsigned)g.bh()), dim3(256),
                       g.nqb * sizeof(uint32_t), s, a.bits, g.nqb, g.nkb, nw, a.q_idx, a.q_cnt,
                       a.order, a.ctr);
    hipLaunchKernelGGL((k_vflag<D>), dim3(g.nkb, (unsigned)g.bh()), dim3(256), 0, s, a.v, g.N,
                       g.nkb, a.kvflag);
  }
  if (stages & 2u) {
    const int total = (int)(g.nqb * g.bh());
    hipLaunchKernelGGL((k_dq<D, BQ>), dim3(total), dim3(BQ * 2), 0, s, a.q, a.k, a.v, a.o,
                       a.o_lo, a.dout, a.lse, a.lse2, a.dsum, a.kv_idx, a.kv_cnt, g.N, npad,
                       g.nqb, g.nkb, total, sl2, a.scale, a.dq, a.grad_bf16, a.do16,
                       a.kvflag);
  }
  if (stages & 4u) {
    const int total = (int)(g.nkb * g.bh());
    // one resident workgroup per compute unit, a multiple of 8 so that every XCD holds
    // as many; each takes key blocks from the queues until all are done
    const int ncu = cu_count();
    int grid = ncu - ncu % 8;
    if (grid < 8) grid = 8;
    if (grid > total) grid = total;
    hipLaunchKernelGGL((k_dkdv<D, BQ>), dim3(grid), dim3(512), 0, s, a.q, a.k, a.v, a.dout,
                       a.lse2, a.dsum, a.q_idx, a.q_cnt, g.N, npad, g.nqb, g.nkb, total, sl2,
                       a.scale, a.dk, a.dv, a.grad_bf16, a.do16, a.kvflag, a.order, a.ctr);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, unsigned stages, hipStream_t s) {
  const int d = a.g.d, bq = a.g.blk_q;
  if (d == 128 && bq == 128) return launch_bwd_t<128, 128>(a, stages, s);
  if (d == 128 && bq == 64) return launch_bwd_t<128, 64>(a, stages, s);
  if (d == 64 && bq == 128) return launch_bwd_t<64, 128>(a, stages, s);
  return launch_bwd_t<64, 64>(a, stages, s);
}

}  // namespace spa
