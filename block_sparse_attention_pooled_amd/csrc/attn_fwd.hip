// Block-sparse attention forward over the kept tiles only (mindverse article on
// SpargeAttention2, sections "Block-dünnbesetzte Aufmerksamkeit" and "Effiziente
// Kernel-Implementierung und Modellanpassung": dropped tiles cost no matrix product and
// no softmax).
//
// One workgroup per (b, h, query block), one wavefront per 32 query rows, workgroups
// ordered so that each XCD works on a contiguous run of query blocks of one head.  For
// each listed key block (64 keys) the K and V tiles stream row-major into LDS with
// direct buffer->LDS loads (rows beyond N arrive as zeros), double buffered: the next
// tile is in flight while the current one is used.
// Per wavefront and tile:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16 (K rows read in perm32 order, Q in
//                 registers), so every lane holds 32 scores of a single query row;
//   online softmax in fp32 with exp2 against the exact running maximum, so that P <= 1
//                 and a row's dominant probability is exactly 1;
//   O^T += V^T P^T with V^T read by ds_read_b64_tr_b16.  P enters the MFMA as bf16, or,
//                 when the caller asks for the residual output o_lo (the backward pass
//                 needs D = <dO, O> to better than bf16), as one fp16 rounding against an
//                 fp16 copy of V: fp16 carries three more mantissa bits than bf16, so O
//                 is accurate to about 12 bits.  A workgroup whose list holds a key block of
//                 V that fp16 cannot carry (a value with |v| >= 65504, or only small values
//                 that fp16 would keep to less than 2^-16 of the block's largest) reads
//                 bf16 V for all its tiles instead, with P as a bf16 hi + lo pair (two
//                 MFMAs).
// The row log-sum-exp is saved for the backward pass.
//
// k_vconv writes the fp16 copy of V for the residual mode, one workgroup per (b, h, key
// block), with a per-block flag for blocks that are not to be read through it.
#include "attn_tiles.h"
#include "spa_internal.h"

namespace spa {


#define SPA_FENCE() __builtin_amdgcn_sched_barrier(0)

// fp16 copy of one key block of V (rows at or beyond N are not written).  flag[bh][j] = 1
// when the block is not to be read through the copy (a value beyond fp16's range, or
// small values that fp16 would carry to less than 2^-16 of the block's largest; see
// f16_block_ok), else 0: written on every call, so no clearing is needed.
template <int D>
__global__ __launch_bounds__(256) void k_vconv(const uint16_t* __restrict__ v,
                                               uint16_t* __restrict__ v16, int N, int nkb,
                                               int32_t* __restrict__ flag) {
  constexpr int PER = kBlkK * D / 8 / 256;  // 16-byte chunks per thread
  __shared__ uint32_t wbits[4];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int rows = min(kBlkK, N - j * kBlkK);
  const size_t base = ((size_t)bh * N + (size_t)j * kBlkK) * D;
  uint32_t r = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int chunk = threadIdx.x + 256 * u;
    if (chunk * 8 < rows * D) {
      const uint4 a = *reinterpret_cast<const uint4*>(v + base + (size_t)chunk * 8);
      r |= f16_range_bits(a);
      *reinterpret_cast<uint4*>(v16 + base + (size_t)chunk * 8) = bf16x8_bits_to_f16(a);
    }
  }
  const uint32_t wr = wave_or4(r);
  if ((threadIdx.x & 63) == 0) wbits[threadIdx.x >> 6] = wr;
  __syncthreads();
  if (threadIdx.x == 0)
    flag[(size_t)bh * nkb + j] = f16_block_ok(wbits[0] | wbits[1] | wbits[2] | wbits[3]) ? 0 : 1;
}

// One kept tile: S^T for this wave's 32 query rows, online softmax update, O^T += V^T P^T.
// K and V rows at or beyond N were staged as zeros; their scores are masked here.
template <int D, bool SPLIT, bool TAIL, bool V16>
__device__ __forceinline__ void fwd_tile(const uint16_t* Ks, const uint16_t* Vs, int key0, int N,
                                         const bf16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                         float& m_run, float& l_run, float scale_log2, int lane,
                                         const ColFragLanes<D>& cf) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int h = lane >> 5;
  // per-lane LDS byte addresses of this V tile's transpose reads (k-step 0; the other
  // k-steps are immediate offsets from them)
  uint32_t vlo[DB], vhi[DB];
  const uint32_t vbase = lds_addr(Vs);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    vlo[db] = vbase + cf.off[db][0];
    vhi[db] = vbase + cf.off[db][1];
  }
  // ---- S^T = K Q^T : two 32-key slabs, K fragments read in batches of four k-steps ------
  f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += 4) {
    bf16x8 a0[4], a1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a0[u] = lds_rowfrag<D>(Ks, 0, k0 + u, lane);
      a1[u] = lds_rowfrag<D>(Ks, 32, k0 + u, lane);
    }
    SPA_FENCE();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sc[0] = mfma32(a0[u], qf[k0 + u], sc[0]);
      sc[1] = mfma32(a1[u], qf[k0 + u], sc[1]);
    }
  }
  // keys at or beyond N exist only in the last key block (a separate instantiation, so
  // that the other tiles carry no per-element selects)
  if constexpr (TAIL) {
    const int lim = N - key0 - 8 * h;  // element e is valid iff acc_row(e,0) < lim
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 16 * (e >> 3) + (e & 7);
      if (r >= lim) sc[0][e] = -INFINITY;
      if (r + 32 >= lim) sc[1][e] = -INFINITY;
    }
  }
  // the V^T fragments of the first two k-steps of P*V do not depend on the softmax: their
  // transpose reads are issued first and land while the exponentials run
  bf16x8 va0[2][DB];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) va0[kk][db] = lds_colfrag_at<D>(vlo[db], vhi[db], kk);
  SPA_FENCE();
  // ---- online softmax (log2 domain, scale folded into the exponent) --------------------
  float mloc = sc[0][0];
#pragma unroll
  for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sc[0][e]);
#pragma unroll
  for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sc[1][e]);
  mloc = fmaxf(mloc, swap_halves(mloc)) * scale_log2;
  // the running maximum is exact: P <= 1, and the dominant probability of a peaked row is
  // exactly 1, which every operand format carries without error
  const bool raise = mloc > m_run;
  if (__ballot(raise)) {
    const float m_new = raise ? mloc : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
  }
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sc[0][e] = __builtin_amdgcn_exp2f(fmaf(sc[0][e], scale_log2, -m_run));
    sc[1][e] = __builtin_amdgcn_exp2f(fmaf(sc[1][e], scale_log2, -m_run));
    psum += sc[0][e] + sc[1][e];
  }
  l_run += psum;
  // ---- O^T += V^T P^T ---------------------------------------------------------------
  if constexpr (SPLIT && V16) {  // the V tile holds fp16 bits; P as one fp16 rounding
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f16x8 ph = to_f16x8(sc[kk >> 1], kk & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 va = kk < 2 ? va0[kk][db] : lds_colfrag_at<D>(vlo[db], vhi[db], kk);
        oacc[db] = mfma32h(__builtin_bit_cast(f16x8, va), ph, oacc[db]);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 ph, pl;
      if constexpr (SPLIT)
        split_bf16x8(sc[kk >> 1], kk & 1, ph, pl);
      else
        ph = to_bf16x8(sc[kk >> 1], kk & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 va = kk < 2 ? va0[kk][db] : lds_colfrag_at<D>(vlo[db], vhi[db], kk);
        oacc[db] = mfma32(va, ph, oacc[db]);
        if constexpr (SPLIT) oacc[db] = mfma32(va, pl, oacc[db]);
      }
    }
  }
}

template <int D, int BQ, bool SPLIT>
__global__ __launch_bounds__(BQ * 2, 2) void k_fwd(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  const uint16_t* __restrict__ v16,
                                                  const int32_t* __restrict__ vflag,
                                                  const int32_t* __restrict__ kv_idx,
                                                  const int32_t* __restrict__ kv_cnt, int N,
                                                  int nqb, int nkb, int total, float scale_log2,
                                                  uint16_t* __restrict__ o,
                                                  uint16_t* __restrict__ o_lo,
                                                  float* __restrict__ lse) {
  constexpr int NT = BQ * 2;
  constexpr int KS = D / 16;  // k-steps over the head dimension
  constexpr int DB = D / 32;  // 32-wide column blocks of O
  __shared__ __align__(16) uint16_t smem[2][2][Tile<D>::ELEMS];  // [buf][K|V]
  __shared__ int32_t lst[kMaxBlocks];  // the key-block list (keeps scalar loads out of the loop)

  const int tile_id = xcd_remap(blockIdx.x, total);
  const int bh = tile_id / nqb;
  const int i = tile_id - bh * nqb;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const u32x4 krs = make_rsrc(k + head, (uint32_t)N * D * 2);
  const u32x4 vrs = make_rsrc(v + head, (uint32_t)N * D * 2);
  const u32x4 v16rs = SPLIT ? make_rsrc(v16 + head, (uint32_t)N * D * 2) : vrs;
  const int32_t* list = kv_idx + ((size_t)bh * nqb + i) * nkb;
  // the lists are trusted; the clamp only keeps a corrupt count inside the LDS list
  const int cnt = min(max(kv_cnt[(size_t)bh * nqb + i], 0), nkb);
  const int j0 = cnt > 0 ? list[0] : 0;
  const TileLanes<D, kBlkK, NT / 64> tl;
  // the first K and V tiles (V from its fp16 copy unless found unusable below) and this
  // block's Q rows are requested before the list is staged: Q goes to the second buffer,
  // which the loop fills only after its first step.  Gathering the Q operand rows straight
  // from memory (32 bytes of each of 32 rows per load) was slower.  Rows at or beyond N
  // read as zeros and are never written.
  if (cnt > 0) {
    tile_load_lds_rsrc<D, kBlkK, NT / 64>(krs, j0 * kBlkK, smem[0][0], tl);
    tile_load_lds_rsrc<D, kBlkK, NT / 64>(v16rs, j0 * kBlkK, smem[0][1], tl);
  }
  {
    const u32x4 qrs = make_rsrc(q + head, (uint32_t)N * D * 2);
#pragma unroll
    for (int hq = 0; hq < BQ / kBlkK; ++hq)
      tile_load_lds_rsrc<D, kBlkK, NT / 64>(qrs, i * BQ + hq * kBlkK,
                                            &smem[1][0][0] + hq * Tile<D>::ELEMS, tl);
  }
  int bad16 = 0;
  for (int x = threadIdx.x; x < cnt; x += NT) {
    const int j = list[x];
    lst[x] = j;
    if (SPLIT) bad16 |= vflag[(size_t)bh * nkb + min(max(j, 0), nkb - 1)];
  }
  // one operand format for the whole workgroup: fp16 V unless a listed block cannot use it
  // (the list's loads were issued after the transfers above, so these have landed too)
  const bool use16 = SPLIT && !__syncthreads_or(bad16);
  if (SPLIT && !use16 && cnt > 0)  // the first V tile again, in bf16
    tile_load_lds_rsrc<D, kBlkK, NT / 64>(vrs, j0 * kBlkK, smem[0][1], tl);

  // this lane's query row (B operand of S^T = K Q^T)
  const int qrow = i * BQ + 32 * wv + c;
  const bool qvalid = qrow < N;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const ColFragLanes<D> cf(lane);
  auto blk = [&](int t) { return __builtin_amdgcn_readfirstlane(lst[min(t, cnt - 1)]); };
  const u32x4 vsrc = use16 ? v16rs : vrs;
  wait_vmem();  // nothing vector-memory is pending inside the loop
  __syncthreads();
  bf16x8 qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(&smem[1][0][0] +
                                              Tile<D>::off(32 * wv + c, 16 * kk + 8 * h));
  __syncthreads();  // Q is in registers before the loop refills its buffer
  const bool tail_last = cnt > 0 && blk(cnt - 1) * kBlkK + kBlkK > N;
  const int cnt_main = cnt - (tail_last ? 1 : 0);
  // the block index of the next tile is read from LDS one tile ahead and taken into a
  // scalar register after the barrier, so that no step waits for that read
// The loop is unrolled over the two buffers, so that every LDS address in a tile is a
// loop-invariant register plus a constant offset.
#define SPA_FWD_STEP(BUF, V16_)                                                              \
  {                                                                                        \
    if (t + 1 < cnt) {                                                                     \
      tile_load_lds_rsrc<D, kBlkK, NT / 64>(krs, jn * kBlkK, smem[(BUF) ^ 1][0], tl);      \
      tile_load_lds_rsrc<D, kBlkK, NT / 64>(vsrc, jn * kBlkK, smem[(BUF) ^ 1][1], tl);     \
    }                                                                                      \
    const int jn_v = lst[min(t + 2, cnt - 1)];                                             \
    /* key0 is read by the tail form only */                                              \
    fwd_tile<D, SPLIT, false, V16_>(smem[BUF][0], smem[BUF][1], 0, N, qf, oacc, m_run,     \
                                    l_run, scale_log2, lane, cf);                          \
    wait_vmem();                                                                           \
    __syncthreads();                                                                       \
    jn = __builtin_amdgcn_readfirstlane(jn_v);                                             \
  }
#define SPA_FWD_LOOP(V16_)                                                                   \
  {                                                                                        \
    int jn = cnt > 1 ? blk(1) : 0;                                                         \
    for (int t = 0;;) {                                                                    \
      if (t >= cnt_main) break;                                                            \
      SPA_FWD_STEP(0, V16_)                                                                \
      if (++t >= cnt_main) break;                                                          \
      SPA_FWD_STEP(1, V16_)                                                                \
      ++t;                                                                                 \
    }                                                                                      \
    if (tail_last) {                                                                       \
      const int buf = cnt_main & 1;                                                        \
      fwd_tile<D, SPLIT, true, V16_>(smem[buf][0], smem[buf][1], blk(cnt_main) * kBlkK, N, \
                                     qf, oacc, m_run, l_run, scale_log2, lane, cf);        \
    }                                                                                      \
  }
  // two copies of the loop, one per operand format, so that neither carries the other's
  // registers
  if (use16) SPA_FWD_LOOP(true) else SPA_FWD_LOOP(false)
#undef SPA_FWD_LOOP
#undef SPA_FWD_STEP

  // ---- epilogue ---------------------------------------------------------------------
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // O and its residual leave through LDS (row-major, Tile swizzle): in the accumulator
  // layout a store covers 8 bytes of each of 32 rows, while from the staged copy each
  // wavefront writes whole rows, 16 bytes per lane
  static_assert(2 * BQ * D <= 4 * Tile<D>::ELEMS, "the output tiles reuse the K and V buffers");
  const bool with_lo = SPLIT && o_lo != nullptr;
  uint16_t* ot = &smem[0][0][0];
  uint16_t* lt = ot + BQ * D;
  __syncthreads();  // every wavefront is done with the last K and V tiles
  {
    const int r = 32 * wv + c;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        bf16x4 hv, lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = oacc[db][4 * g + e] * inv;
          hv[e] = (__bf16)x;
          lv[e] = (__bf16)(x - (float)hv[e]);
        }
        *reinterpret_cast<bf16x4*>(ot + Tile<D>::off(r, d0)) = hv;
        if (with_lo) *reinterpret_cast<bf16x4*>(lt + Tile<D>::off(r, d0)) = lv;
      }
  }
  __syncthreads();
  {
    constexpr int CPR = Tile<D>::CPR;  // 16-byte chunks per row
    const int ch = lane % CPR;
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {  // this wavefront's 32 rows, 64 / CPR a pass
      const int r = 32 * wv + it * (64 / CPR) + lane / CPR;
      const int row = i * BQ + r;
      if (row < N) {
        const size_t off = head + (size_t)row * D + 8 * ch;
        *reinterpret_cast<uint4*>(o + off) = *reinterpret_cast<const uint4*>(ot + Tile<D>::off(r, 8 * ch));
        if (with_lo)
          *reinterpret_cast<uint4*>(o_lo + off) = *reinterpret_cast<const uint4*>(lt + Tile<D>::off(r, 8 * ch));
      }
    }
  }
  if (qvalid && h == 0)
    lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int BQ>
static hipError_t launch_fwd_t(const FwdArgs& a, unsigned stages, hipStream_t s) {
  const Geometry& g = a.g;
  const int total = (int)(g.nqb * g.bh());
  dim3 grid(total);
  if (a.o_lo) {
    if (stages & 1u)
      hipLaunchKernelGGL((k_vconv<D>), dim3(g.nkb, (unsigned)g.bh()), dim3(256), 0, s, a.v,
                         a.v16, g.N, g.nkb, a.vflag);
    if (stages & 2u)
      hipLaunchKernelGGL((k_fwd<D, BQ, true>), grid, dim3(BQ * 2), 0, s, a.q, a.k, a.v, a.v16,
                         a.vflag, a.kv_idx, a.kv_cnt, g.N, g.nqb, g.nkb, total,
                         a.scale * kLog2e, a.o, a.o_lo, a.lse);
  } else if (stages & 2u) {
    hipLaunchKernelGGL((k_fwd<D, BQ, false>), grid, dim3(BQ * 2), 0, s, a.q, a.k, a.v,
                       (const uint16_t*)nullptr, (const int32_t*)nullptr, a.kv_idx, a.kv_cnt,
                       g.N, g.nqb, g.nkb, total, a.scale * kLog2e, a.o, a.o_lo, a.lse);
  }
  return hipGetLastError();
}

size_t fwd_workspace_bytes(const Geometry& g) {
  return align_up((size_t)g.bh() * g.N * g.d * 2, 256) + align_up((size_t)g.bh() * g.nkb * 4, 256);
}

void fwd_workspace_carve(const Geometry& g, void* ws, FwdArgs* a) {
  char* p = static_cast<char*>(ws);
  a->v16 = reinterpret_cast<uint16_t*>(p);
  p += align_up((size_t)g.bh() * g.N * g.d * 2, 256);
  a->vflag = reinterpret_cast<int32_t*>(p);
}

hipError_t launch_fwd(const FwdArgs& a, unsigned stages, hipStream_t s) {
  const int d = a.g.d, bq = a.g.blk_q;
  if (d == 128 && bq == 128) return launch_fwd_t<128, 128>(a, stages, s);
  if (d == 128 && bq == 64) return launch_fwd_t<128, 64>(a, stages, s);
  if (d == 64 && bq == 128) return launch_fwd_t<64, 128>(a, stages, s);
  return launch_fwd_t<64, 64>(a, stages, s);
}

}  // namespace spa
