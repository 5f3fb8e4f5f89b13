// Block-sparse attention forward over the kept tiles only (mindverse article on
// SpargeAttention2, sections "Block-dünnbesetzte Aufmerksamkeit" and "Effiziente
// Kernel-Implementierung und Modellanpassung": dropped tiles cost no matrix product and
// no softmax).
//
// One workgroup per (b, h, query block); one wavefront per 32 query rows.  For each
// listed key block (64 keys) the K and V tiles are staged row-major in LDS (double
// buffered, the next tile's global loads in flight during the current tile's math).
// Per wavefront and tile:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16 (K rows read in perm32 order, Q in
//                 registers), so every lane holds 32 scores of a single query row;
//   online softmax in fp32 with exp2 (row max exchanged once with lane l^32);
//   O^T += V^T P^T with V^T read by ds_read_b64_tr_b16; P enters the MFMA as bf16,
//                 or, when the caller asks for the residual output o_lo, as a bf16
//                 hi + lo pair so that O is accurate to about 16 bits (the backward
//                 pass needs D = <dO, O> to that accuracy).
// The row log-sum-exp is saved for the backward pass.
#include "attn_tiles.h"
#include "spa_internal.h"

namespace spa {

template <int D, int BQ, bool SPLIT>
__global__ __launch_bounds__(BQ * 2) void k_fwd(const uint16_t* __restrict__ q,
                                               const uint16_t* __restrict__ k,
                                               const uint16_t* __restrict__ v,
                                               const int32_t* __restrict__ kv_idx,
                                               const int32_t* __restrict__ kv_cnt, int N,
                                               int nqb, int nkb, float scale_log2,
                                               uint16_t* __restrict__ o,
                                               uint16_t* __restrict__ o_lo,
                                               float* __restrict__ lse) {
  constexpr int NT = BQ * 2;
  constexpr int NCH = TileCfg<D>::CHUNKS / NT;
  constexpr int KS = D / 16;  // k-steps over the head dimension
  constexpr int DB = D / 32;  // 32-wide column blocks of O
  __shared__ __align__(16) uint16_t smem[2][2][TileCfg<D>::TILE];  // [buf][K|V]

  const int bh = blockIdx.y;
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* kh_ = k + head;
  const uint16_t* vh_ = v + head;
  const int32_t* list = kv_idx + ((size_t)bh * nqb + i) * nkb;
  const int cnt = kv_cnt[(size_t)bh * nqb + i];

  // this lane's query row and its Q fragments (B operand of S^T = K Q^T)
  const int qrow = i * BQ + 32 * wv + c;
  const bool qvalid = qrow < N;
  bf16x8 qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if (qvalid)
      qf[kk] = *reinterpret_cast<const bf16x8*>(q + head + (size_t)qrow * D + 16 * kk + 8 * h);
    else
      qf[kk] = bf16x8{};
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 kr[NCH], vr[NCH];
  if (cnt > 0) {
    const int j0 = list[0];
    tile_load<D, NT>(kr, kh_, j0 * kBlkK, N);
    tile_load<D, NT>(vr, vh_, j0 * kBlkK, N);
    tile_store<D, NT>(kr, smem[0][0]);
    tile_store<D, NT>(vr, smem[0][1]);
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int buf = t & 1;
    const int j = list[t];
    if (t + 1 < cnt) {
      const int jn = list[t + 1];
      tile_load<D, NT>(kr, kh_, jn * kBlkK, N);
      tile_load<D, NT>(vr, vh_, jn * kBlkK, N);
    }
    const uint16_t* Ks = smem[buf][0];
    const uint16_t* Vs = smem[buf][1];

    // ---- S^T = K Q^T : two 32-key slabs -------------------------------------------
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) s[kb] = mfma32(lds_rowfrag<D>(Ks, 32 * kb, kk, lane), qf[kk], s[kb]);
    }
    // ---- online softmax (log2 domain) ---------------------------------------------
    const int key0 = j * kBlkK;
    const bool tail = key0 + kBlkK > N;
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[kb][e] * scale_log2;
        if (tail && key0 + 32 * kb + acc_row(e, h) >= N) x = -INFINITY;
        s[kb][e] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, swap_halves(mloc));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(s[kb][e] - m_new);
        s[kb][e] = pe;
        psum += pe;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    // ---- O^T += V^T P^T ---------------------------------------------------------------
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 ph, pl;
      if constexpr (SPLIT)
        split_bf16x8(s[kk >> 1], kk & 1, ph, pl);
      else
        ph = to_bf16x8(s[kk >> 1], kk & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 va = lds_colfrag<D>(Vs, 16 * kk, 32 * db, lane);
        oacc[db] = mfma32(va, ph, oacc[db]);
        if constexpr (SPLIT) oacc[db] = mfma32(va, pl, oacc[db]);
      }
    }
    if (t + 1 < cnt) {
      tile_store<D, NT>(kr, smem[buf ^ 1][0]);
      tile_store<D, NT>(vr, smem[buf ^ 1][1]);
    }
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------------
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    uint16_t* orow = o + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        float x[4];
        uint32_t hb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = oacc[db][4 * g + e] * inv;
          hb[e] = f32_to_bf16_bits(x[e]);
        }
        *reinterpret_cast<uint2*>(orow + d0) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        if (SPLIT && o_lo) {
          uint32_t lb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) lb[e] = f32_to_bf16_bits(x[e] - bf16_bits_to_f32(hb[e]));
          *reinterpret_cast<uint2*>(o_lo + head + (size_t)qrow * D + d0) =
              make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
        }
      }
    if (h == 0)
      lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int BQ>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const Geometry& g = a.g;
  dim3 grid(g.nqb, (unsigned)g.bh());
  if (a.o_lo)
    hipLaunchKernelGGL((k_fwd<D, BQ, true>), grid, dim3(BQ * 2), 0, s, a.q, a.k, a.v, a.kv_idx,
                       a.kv_cnt, g.N, g.nqb, g.nkb, a.scale * kLog2e, a.o, a.o_lo, a.lse);
  else
    hipLaunchKernelGGL((k_fwd<D, BQ, false>), grid, dim3(BQ * 2), 0, s, a.q, a.k, a.v, a.kv_idx,
                       a.kv_cnt, g.N, g.nqb, g.nkb, a.scale * kLog2e, a.o, a.o_lo, a.lse);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  const int d = a.g.d, bq = a.g.blk_q;
  if (d == 128 && bq == 128) return launch_fwd_t<128, 128>(a, s);
  if (d == 128 && bq == 64) return launch_fwd_t<128, 64>(a, s);
  if (d == 64 && bq == 128) return launch_fwd_t<64, 128>(a, s);
  return launch_fwd_t<64, 64>(a, s);
}

}  // namespace spa
