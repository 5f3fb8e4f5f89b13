// Block-sparse attention backward over the kept tiles only, mask held fixed (abstract
// page "SpargeAttention2: Trainable Sparse Attention via Hybrid Top-k+Top-p Masking and
// Distillation Fine-Tuning", contribution (ii); mindverse article, section "Effiziente
// Kernel-Implementierung und Modellanpassung").
//
// Launch sequence (one stream):
//   k_dsum      D_t = <dO_t, O_t> in fp32, with O = o + o_lo when the forward pass
//               supplied its rounding residual;
//   k_bitmap    the kept-tile bitmap, transposed: word w of query block i at [w][i];
//   k_collists  per key block j, the ascending list of query blocks that keep j;
//   k_dkdv      one workgroup per (b, h, key block): walks its query-block list in
//               ascending order, recomputes S and P, accumulates dV += P^T dO and
//               dK += dS^T Q in registers (no atomics, fixed order);
//   k_dq        one workgroup per (b, h, query block): walks its key-block list in
//               ascending order and accumulates dQ += dS K.
// All products are bf16 MFMA with fp32 accumulation.  P (in dV = P^T dO) and dS (in
// dQ = dS K and dK = dS^T Q) enter as bf16 hi + lo pairs (about 16 bits): on peaked
// rows dS is a difference of nearly equal terms, and dV of a key that many queries
// attend to sums thousands of products, so a single bf16 rounding of either would be
// visible in the gradients.
#include "attn_tiles.h"
#include "spa_internal.h"

namespace spa {

// ------------------------------------------------------------------------------------
// D = rowsum(dO * O)
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_dsum(const uint16_t* __restrict__ o,
                                              const uint16_t* __restrict__ o_lo,
                                              const uint16_t* __restrict__ dout, long long rows,
                                              float* __restrict__ dsum) {
  constexpr int CPR = D / 8;         // lanes per row
  constexpr int RPB = 256 / CPR;     // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int cc = threadIdx.x % CPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + cc * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + cc * 8);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
    uint32_t wl[4] = {0u, 0u, 0u, 0u};
    if (o_lo) {
      const uint4 c = *reinterpret_cast<const uint4*>(o_lo + row * D + cc * 8);
      wl[0] = c.x;
      wl[1] = c.y;
      wl[2] = c.z;
      wl[3] = c.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o0 = bf16_bits_to_f32(wa[e] & 0xFFFFu) + bf16_bits_to_f32(wl[e] & 0xFFFFu);
      const float o1 = bf16_bits_to_f32(wa[e] >> 16) + bf16_bits_to_f32(wl[e] >> 16);
      acc = fmaf(o0, bf16_bits_to_f32(wb[e] & 0xFFFFu), acc);
      acc = fmaf(o1, bf16_bits_to_f32(wb[e] >> 16), acc);
    }
  }
#pragma unroll
  for (int off = CPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && cc == 0) dsum[row] = acc;
}

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

__global__ __launch_bounds__(256) void k_collists(const uint32_t* __restrict__ bits, int nqb,
                                                  int nkb, int nw, int32_t* __restrict__ q_idx,
                                                  int32_t* __restrict__ q_cnt) {
  extern __shared__ uint32_t colw[];  // [nqb]
  const int bh = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
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
    if (lane == 0) q_cnt[(size_t)bh * nkb + j] = base;
  }
}

// ------------------------------------------------------------------------------------
// dK, dV: one workgroup per key block (workgroups in XCD-contiguous order), 4 wavefronts,
// one workgroup per CU.  The key block's query-block list is walked one query block per
// stage; Q and dO of the next query block stream into the other LDS buffer with direct
// global->LDS loads while the current one is used.  Wavefront w owns keys
// 32*(w&1) .. +32 of the block and the 32-row slabs of parity w>>1 (two independent
// slabs per stage when the block has 128 rows); the two parities are summed at the end
// in a fixed order.
// ------------------------------------------------------------------------------------
// One 32-row query slab of a staged block against this wave's 32 keys.
// S = Q K^T and dP = dO V^T with lanes owning keys (K, V fragments in registers).
template <int D>
__device__ __forceinline__ void slab_scores(const uint16_t* Qb, const uint16_t* dOb, int r0,
                                            const bf16x8 (&kf)[D / 16],
                                            const bf16x8 (&vf)[D / 16], int lane, f32x16& s,
                                            f32x16& dp) {
  s = f32x16{};
  dp = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    s = mfma32(lds_rowfrag<D>(Qb, r0, kk, lane), kf[kk], s);
    dp = mfma32(lds_rowfrag<D>(dOb, r0, kk, lane), vf[kk], dp);
  }
}

// P = exp2(S*scale*log2e - lse2) and dS = P (dP - D), in place; element e belongs to
// query row r0 + acc_row(e, h) (two runs of 8 consecutive rows).
__device__ __forceinline__ void slab_probs(const float* lse2s, const float* dss, int r0, int h,
                                           float kmask, float scale_log2, f32x16& s,
                                           f32x16& dp) {
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int q0 = r0 + 16 * run + 8 * h;
    const float4 l0 = *reinterpret_cast<const float4*>(lse2s + q0);
    const float4 l1 = *reinterpret_cast<const float4*>(lse2s + q0 + 4);
    const float4 d0 = *reinterpret_cast<const float4*>(dss + q0);
    const float4 d1 = *reinterpret_cast<const float4*>(dss + q0 + 4);
    const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
    const float dv_[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = 8 * run + u;
      const float pe = kmask * __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, -lv[u]));
      s[e] = pe;
      dp[e] = pe * (dp[e] - dv_[u]);
    }
  }
}

// dV += P^T dO and dK += dS^T Q for the slab (P, dS as bf16 hi + lo pairs; dO^T, Q^T
// gathered with transpose reads).
template <int D>
__device__ __forceinline__ void slab_grads(const uint16_t* Qb, const uint16_t* dOb, int r0,
                                           int lane, const f32x16& p, const f32x16& ds,
                                           f32x16 (&dka)[D / 32], f32x16 (&dva)[D / 32]) {
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    bf16x8 ph, pl, dh, dl;
    split_bf16x8(p, kq, ph, pl);
    split_bf16x8(ds, kq, dh, dl);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x8 ob = lds_colfrag<D>(dOb, r0 + 16 * kq, 32 * db, lane);
      dva[db] = mfma32(ph, ob, dva[db]);
      dva[db] = mfma32(pl, ob, dva[db]);
      const bf16x8 qb = lds_colfrag<D>(Qb, r0 + 16 * kq, 32 * db, lane);
      dka[db] = mfma32(dh, qb, dka[db]);
      dka[db] = mfma32(dl, qb, dka[db]);
    }
  }
}

template <int D, int BQ>
__global__ __launch_bounds__(256, 1) void k_dkdv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dsum,
    const int32_t* __restrict__ q_idx, const int32_t* __restrict__ q_cnt, int N, int nqb,
    int nkb, int total, float scale_log2, float scale, void* __restrict__ dk_out,
    void* __restrict__ dv_out, int grad_bf16) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int SLABS = BQ / 32;          // 32-row slabs per query block
  constexpr int TILE = BQ * D;            // elements of one staged Q or dO tile
  constexpr int STAGE_BYTES = 2 * (2 * TILE * 2 + 2 * BQ * 4);  // 2 buffers: Q, dO, lse2, D
  constexpr int RED_BYTES = 2 * 2 * 64 * DB * 16 * 4;           // dK, dV partials
  constexpr int SMEM = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
  __shared__ __align__(16) unsigned char smem[SMEM];
  uint16_t* tiles = reinterpret_cast<uint16_t*>(smem);           // [buf][Q | dO][TILE]
  float* side = reinterpret_cast<float*>(smem + 2 * 2 * TILE * 2);  // [buf][lse2 | D][BQ], 16-byte aligned

  const int tile_id = xcd_remap(blockIdx.x, total);
  const int bh = tile_id / nkb;
  const int j = tile_id - bh * nkb;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int kh = wv & 1, par = wv >> 1;
  const size_t head = (size_t)bh * N * D;
  const int key = j * kBlkK + 32 * kh + c;  // this lane's key (B operand column)
  const float kmask = key < N ? 1.f : 0.f;  // keys beyond N compute on a copy and get P = 0

  bf16x8 kf[KS], vf[KS];
  {
    const size_t krow = head + (size_t)min(key, N - 1) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(k + krow + 16 * kk);
      vf[kk] = *reinterpret_cast<const bf16x8*>(v + krow + 16 * kk);
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  const int32_t* list = q_idx + ((size_t)bh * nkb + j) * nqb;
  const int cnt = q_cnt[(size_t)bh * nkb + j];
  float lse_r = 0.f, d_r = 0.f;  // side values of row t (t < BQ) of the staged block
  if (cnt > 0) {
    const int r0 = list[0] * BQ;
    tile_load_lds<D, BQ, 4>(q + head, r0, N, tiles);
    tile_load_lds<D, BQ, 4>(dout + head, r0, N, tiles + TILE);
    if (t < BQ) {
      const int grow = r0 + t;
      const size_t gi = (size_t)bh * N + min(grow, N - 1);
      side[t] = grow < N ? lse[gi] * kLog2e : INFINITY;  // rows beyond N get P = 0
      side[BQ + t] = grow < N ? dsum[gi] : 0.f;
    }
    wait_vmem();
  }
  __syncthreads();
  for (int it = 0; it < cnt; ++it) {
    const int b = it & 1;
    {  // next query block (the last iteration reloads its own block; the copy goes unused)
      const int r0 = list[min(it + 1, cnt - 1)] * BQ;
      uint16_t* nb = tiles + (b ^ 1) * 2 * TILE;
      tile_load_lds<D, BQ, 4>(q + head, r0, N, nb);
      tile_load_lds<D, BQ, 4>(dout + head, r0, N, nb + TILE);
      if (t < BQ) {
        const int grow = r0 + t;
        const size_t gi = (size_t)bh * N + min(grow, N - 1);
        lse_r = grow < N ? lse[gi] * kLog2e : INFINITY;
        d_r = grow < N ? dsum[gi] : 0.f;
      }
    }
    const uint16_t* Qb = tiles + b * 2 * TILE;
    const uint16_t* dOb = Qb + TILE;
    const float* lse2s = side + b * 2 * BQ;
    const float* dss = lse2s + BQ;
    if constexpr (SLABS == 4) {
      // two independent slabs per wave, software-pipelined: the MFMAs of one slab are
      // issued next to the VALU work of the other
      const int ra = 32 * par, rb = 32 * (par + 2);
      f32x16 sa, dpa, sb, dpb;
      slab_scores<D>(Qb, dOb, ra, kf, vf, lane, sa, dpa);
      slab_scores<D>(Qb, dOb, rb, kf, vf, lane, sb, dpb);
      slab_probs(lse2s, dss, ra, h, kmask, scale_log2, sa, dpa);
      slab_grads<D>(Qb, dOb, ra, lane, sa, dpa, dka, dva);
      slab_probs(lse2s, dss, rb, h, kmask, scale_log2, sb, dpb);
      slab_grads<D>(Qb, dOb, rb, lane, sb, dpb, dka, dva);
    } else {
      const int ra = 32 * par;
      f32x16 sa, dpa;
      slab_scores<D>(Qb, dOb, ra, kf, vf, lane, sa, dpa);
      slab_probs(lse2s, dss, ra, h, kmask, scale_log2, sa, dpa);
      slab_grads<D>(Qb, dOb, ra, lane, sa, dpa, dka, dva);
    }
    if (t < BQ) {
      side[(b ^ 1) * 2 * BQ + t] = lse_r;
      side[(b ^ 1) * 2 * BQ + BQ + t] = d_r;
    }
    wait_vmem();
    __syncthreads();
  }

  // ---- reduce the two slab parities and write ------------------------------------------
  float* red = reinterpret_cast<float*>(smem);  // [kh][K|V][DB*16][lane]: lane-contiguous
  auto slot = [&](int which, int idx) { return ((kh * 2 + which) * (DB * 16) + idx) * 64 + lane; };
  if (par == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[slot(0, db * 16 + e)] = dka[db][e];
        red[slot(1, db * 16 + e)] = dva[db][e];
      }
  }
  __syncthreads();
  if (par == 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float gk = (dka[db][e] + red[slot(0, db * 16 + e)]) * scale;
        const float gv = dva[db][e] + red[slot(1, db * 16 + e)];
        // accumulator element e: key row 8*(e/4) + 4*h + e%4 of this wave's 32 keys, column c
        const int krow = j * kBlkK + 32 * kh + 8 * (e >> 2) + 4 * h + (e & 3);
        if (krow < N) {
          const size_t off = head + (size_t)krow * D + 32 * db + c;
          if (grad_bf16) {
            reinterpret_cast<__bf16*>(dk_out)[off] = (__bf16)gk;
            reinterpret_cast<__bf16*>(dv_out)[off] = (__bf16)gv;
          } else {
            reinterpret_cast<float*>(dk_out)[off] = gk;
            reinterpret_cast<float*>(dv_out)[off] = gv;
          }
        }
      }
  }
}

// ------------------------------------------------------------------------------------
// dQ: one workgroup per query block (XCD-contiguous order), one wavefront per 32 rows;
// K and V tiles staged like the forward pass.
// ------------------------------------------------------------------------------------
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 2) void k_dq(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dsum,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, int N, int nqb,
    int nkb, int total, float scale_log2, float scale, void* __restrict__ dq_out,
    int grad_bf16) {
  constexpr int NT = BQ * 2;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __align__(16) uint16_t smem[2][2][Tile<D>::ELEMS];  // [buf][K|V]

  const int tile_id = xcd_remap(blockIdx.x, total);
  const int bh = tile_id / nqb;
  const int i = tile_id - bh * nqb;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* kh_ = k + head;
  const uint16_t* vh_ = v + head;
  const int32_t* list = kv_idx + ((size_t)bh * nqb + i) * nkb;
  const int cnt = kv_cnt[(size_t)bh * nqb + i];

  const int qrow = i * BQ + 32 * wv + c;
  const bool qvalid = qrow < N;
  const size_t qoff = head + (size_t)min(qrow, N - 1) * D + 8 * h;
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(q + qoff + 16 * kk);
    df[kk] = *reinterpret_cast<const bf16x8*>(dout + qoff + 16 * kk);
  }
  const size_t ri = (size_t)bh * N + min(qrow, N - 1);
  const float lse2 = lse[ri] * kLog2e;
  const float dq_sum = dsum[ri];

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  if (cnt > 0) {
    const int j0 = list[0];
    tile_load_lds<D, kBlkK, NT / 64>(kh_, j0 * kBlkK, N, smem[0][0]);
    tile_load_lds<D, kBlkK, NT / 64>(vh_, j0 * kBlkK, N, smem[0][1]);
    wait_vmem();
  }
  __syncthreads();
  for (int t = 0; t < cnt; ++t) {
    const int buf = t & 1;
    const int j = list[t];
    {  // next tile streams into the other buffer (the last iteration reloads its own
       // tile; the copy goes unused)
      const int jn = list[min(t + 1, cnt - 1)];
      tile_load_lds<D, kBlkK, NT / 64>(kh_, jn * kBlkK, N, smem[buf ^ 1][0]);
      tile_load_lds<D, kBlkK, NT / 64>(vh_, jn * kBlkK, N, smem[buf ^ 1][1]);
    }
    const uint16_t* Ks = smem[buf][0];
    const uint16_t* Vs = smem[buf][1];
    const int key0 = j * kBlkK;
    // one 32-key slab at a time: scores, dP, dS, then its two 16-key steps of dQ
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        s = mfma32(lds_rowfrag<D>(Ks, 32 * kb, kk, lane), qf[kk], s);
        dp = mfma32(lds_rowfrag<D>(Vs, 32 * kb, kk, lane), df[kk], dp);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, -lse2));
        dp[e] = pe * (dp[e] - dq_sum);
      }
      if (key0 + kBlkK > N) {  // keys at or beyond N exist only in the last key block
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
          const bf16x8 ka = lds_colfrag<D>(Ks, 32 * kb + 16 * half, 32 * db, lane);
          acc[db] = mfma32(ka, dh, acc[db]);
          acc[db] = mfma32(ka, dl, acc[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
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

size_t bwd_workspace_bytes(const Geometry& g) {
  const size_t bh = (size_t)g.bh();
  return align_up(bh * g.N * sizeof(float), 256) +
         align_up(bh * n_words(g) * g.nqb * sizeof(uint32_t), 256) +
         align_up(bh * g.nkb * g.nqb * sizeof(int32_t), 256) +
         align_up(bh * g.nkb * sizeof(int32_t), 256);
}

void bwd_workspace_carve(const Geometry& g, void* ws, BwdArgs* a) {
  const size_t bh = (size_t)g.bh();
  char* p = static_cast<char*>(ws);
  a->dsum = reinterpret_cast<float*>(p);
  p += align_up(bh * g.N * sizeof(float), 256);
  a->bits = reinterpret_cast<uint32_t*>(p);
  p += align_up(bh * n_words(g) * g.nqb * sizeof(uint32_t), 256);
  a->q_idx = reinterpret_cast<int32_t*>(p);
  p += align_up(bh * g.nkb * g.nqb * sizeof(int32_t), 256);
  a->q_cnt = reinterpret_cast<int32_t*>(p);
}

template <int D, int BQ>
static hipError_t launch_bwd_t(const BwdArgs& a, unsigned stages, hipStream_t s) {
  const Geometry& g = a.g;
  const float sl2 = a.scale * kLog2e;
  if (stages & 1u) {
    const long long rows = (long long)g.bh() * g.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((k_dsum<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s,
                       a.o, a.o_lo, a.dout, rows, a.dsum);
    const int nw = n_words(g);
    hipLaunchKernelGGL(k_bitmap, dim3(g.nqb, (unsigned)g.bh()), dim3(64), 0, s, a.kv_idx,
                       a.kv_cnt, g.nqb, g.nkb, nw, a.bits);
    hipLaunchKernelGGL(k_collists, dim3(nw, (unsigned)g.bh()), dim3(256),
                       g.nqb * sizeof(uint32_t), s, a.bits, g.nqb, g.nkb, nw, a.q_idx, a.q_cnt);
  }
  if (stages & 2u) {
    const int total = (int)(g.nkb * g.bh());
    hipLaunchKernelGGL((k_dkdv<D, BQ>), dim3(total), dim3(256), 0, s, a.q, a.k, a.v, a.dout,
                       a.lse, a.dsum, a.q_idx, a.q_cnt, g.N, g.nqb, g.nkb, total, sl2, a.scale,
                       a.dk, a.dv, a.grad_bf16);
  }
  if (stages & 4u) {
    const int total = (int)(g.nqb * g.bh());
    hipLaunchKernelGGL((k_dq<D, BQ>), dim3(total), dim3(BQ * 2), 0, s, a.q, a.k, a.v, a.dout,
                       a.lse, a.dsum, a.kv_idx, a.kv_cnt, g.N, g.nqb, g.nkb, total, sl2, a.scale,
                       a.dq, a.grad_bf16);
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
