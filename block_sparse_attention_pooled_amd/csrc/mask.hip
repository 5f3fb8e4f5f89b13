// Mask construction: block-mean pooling of Q and K, the pooled row softmax and the
// hybrid Top-k + Top-p selection per query block (mindverse article on SpargeAttention2,
// sections "Maskierungsstrategien: Top-k und Top-p" and "Hybride Top-k+Top-p Maskierung").
//
// k_pool    streams Q and K once from HBM (16-byte loads) and writes the block means in
//           fp64.  Sums of bf16 values are exact in fp64, so the means are the correctly
//           rounded means.  Workgroups run in XCD-contiguous order, so that the 8-byte
//           writes of neighbouring key blocks into one line of the transposed pooled K
//           meet in one L2.
// k_select  one workgroup per (b, h, 8 query blocks), XCD-contiguous: the pooled logits of
//           its 8 rows (fp64 FMA against the transposed pooled K), then one wavefront per row:
//           fp64 softmax, and a most-significant-digit radix select over the fp64 bit
//           patterns of the probabilities that finds the last element of the kept prefix.
//           The prefix condition "count >= Lk and cumulative probability >= p" is checked
//           on bucket totals; probabilities are summed as 62-bit fixed-point integers, so
//           every sum is exact and independent of order.  The kept blocks are written
//           in ascending order.
#include "spa_common.h"
#include "spa_internal.h"

namespace spa {

// ------------------------------------------------------------------------------------
// pooling
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_pool(const uint16_t* __restrict__ q,
                                              const uint16_t* __restrict__ k, int N, int blk_q,
                                              int nqb, int nkb, double* __restrict__ qbar,
                                              double* __restrict__ kbar_t) {
  constexpr int C = D / 8;    // 16-byte chunks per row
  constexpr int R = 256 / C;  // rows per pass
  __shared__ double part[R][D];
  const int per_head = nqb + nkb;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / per_head;
  const int x = tile - bh * per_head;
  const bool is_q = x < nqb;
  const int blk = is_q ? blk_q : kBlkK;
  const int b = is_q ? x : x - nqb;
  const int row0 = b * blk;
  const int nrows = min(blk, N - row0);
  const uint16_t* src = (is_q ? q : k) + ((size_t)bh * N + row0) * D;

  const int t = threadIdx.x, c = t % C, r = t / C;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  // all of this thread's loads of a 128-row block are issued before the first one is
  // used (rows at or beyond N are read as zeros and not counted)
  constexpr int PASSES = 128 / R;
  uint4 v[PASSES];
#pragma unroll
  for (int u = 0; u < PASSES; ++u) {
    const int rr = r + u * R;
    v[u] = rr < nrows ? *reinterpret_cast<const uint4*>(src + (size_t)rr * D + c * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < PASSES; ++u) {
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_bits_to_f32(w[e] & 0xFFFFu);
      acc[2 * e + 1] += (double)bf16_bits_to_f32(w[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r][c * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) s += part[rr][t];
    const double mean = s / (double)nrows;
    if (is_q)
      qbar[((size_t)bh * nqb + b) * D + t] = mean;
    else
      kbar_t[((size_t)bh * D + t) * nkb + b] = mean;
  }
}

// ------------------------------------------------------------------------------------
// wave helpers
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// inclusive prefix sum over lanes 0..63
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

template <typename T>
__device__ __forceinline__ T wave_suffix_excl(T x) {  // sum over lanes > this lane
  const int lane = threadIdx.x & 63;
  T incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T y = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += y;
  }
  return incl - x;
}

struct SelectResult {
  uint64_t tau;   // fp64 bit pattern of the last kept probability
  int take_ties;  // how many elements equal to tau (lowest indices first) are kept
  int len;        // kept length L
  int all;        // 1: keep every valid element
};

// Radix select over the wave's elements.  Element e of this lane: key[e] (fp64 bits of
// the probability, monotone as unsigned), w[e] (probability * 2^62, rounded), valid if
// e < nval.  Finds the smallest prefix length L of the order (key desc, index asc) with
// L >= lk and prefix mass >= wp.
template <int E>
__device__ SelectResult radix_select(const uint64_t (&key)[E], const uint64_t (&w)[E], int nval,
                                     int lk, uint64_t wp, uint32_t* cnt, unsigned long long* mass) {
  const int lane = threadIdx.x & 63;
  uint64_t prefix = 0, pmask = 0;
  int c_above = 0;
  uint64_t m_above = 0;
  SelectResult res;
  res.all = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      cnt[lane * 4 + b] = 0u;
      mass[lane * 4 + b] = 0ull;
    }
    wave_sync_lds();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e < nval && (key[e] & pmask) == prefix) {
        const int dgt = (int)((key[e] >> shift) & 255u);
        atomicAdd(&cnt[dgt], 1u);
        atomicAdd(&mass[dgt], (unsigned long long)w[e]);
      }
    }
    wave_sync_lds();
    uint32_t bc[4];
    uint64_t bm[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      bc[b] = cnt[lane * 4 + b];
      bm[b] = mass[lane * 4 + b];
    }
    wave_sync_lds();
    const int tc = (int)(bc[0] + bc[1] + bc[2] + bc[3]);
    const uint64_t tm = bm[0] + bm[1] + bm[2] + bm[3];
    const int sc = wave_suffix_excl<int>(tc);         // count in buckets of higher lanes
    const uint64_t sm = wave_suffix_excl<uint64_t>(tm);
    // cumulative (descending) count / mass including bucket 4*lane + b
    int best = -1;
    int cum_c = c_above + sc;
    uint64_t cum_m = m_above + sm;
    int above_c = 0;
    uint64_t above_m = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      const int prev_c = cum_c;
      const uint64_t prev_m = cum_m;
      cum_c += (int)bc[b];
      cum_m += bm[b];
      if (best < 0 && bc[b] > 0 && cum_c >= lk && cum_m >= wp) {
        best = lane * 4 + b;
        above_c = prev_c;
        above_m = prev_m;
      }
    }
    const unsigned long long ball = __ballot(best >= 0);
    if (ball == 0ull) {  // no prefix reaches the targets: keep every element
      res.all = 1;
      res.len = nval;  // per-lane count; the caller keeps everything
      res.tau = 0;
      res.take_ties = 0;
      return res;
    }
    const int src = 63 - __builtin_clzll(ball);  // highest lane holding a hit
    const int bsel = __shfl(best, src, 64);
    c_above = __shfl(above_c, src, 64);
    m_above = __shfl(above_m, src, 64);
    const int ncand = (int)__shfl((int)bc[bsel & 3], src, 64);
    prefix |= (uint64_t)bsel << shift;
    pmask |= (uint64_t)255u << shift;
    if (ncand == 1 || shift == 0) {
      // the candidates now all equal prefix on the examined digits
      uint64_t tau = prefix;
      if (ncand == 1 && shift > 0) {
        uint64_t mine = 0;
        int have = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (e < nval && (key[e] & pmask) == prefix) {
            mine = key[e];
            have = 1;
          }
        const unsigned long long hb = __ballot(have);
        tau = __shfl(mine, __builtin_ctzll(hb), 64);
      }
      // elements equal to tau: ncand of them (all with the same mass)
      int take = 1;
      if (ncand > 1) {
        const double p = __longlong_as_double((long long)tau);
        const uint64_t wt = (uint64_t)__double2ull_rn(p * 0x1p62);
        int need_c = lk - c_above;
        int need_m = 1;
        if (m_above < wp) {
          if (wt == 0)
            need_m = ncand;
          else
            need_m = (int)((wp - m_above + wt - 1) / wt);
        }
        take = max(1, max(need_c, need_m));
        take = min(take, ncand);
      }
      res.tau = tau;
      res.take_ties = take;
      res.len = c_above + take;
      return res;
    }
  }
  return res;  // not reached
}

// ------------------------------------------------------------------------------------
// selection
// ------------------------------------------------------------------------------------
constexpr int kSelRows = 8;      // query blocks per workgroup (one wavefront each)
constexpr int kSelThreads = 512;

template <int D, int E>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const double* __restrict__ qbar, const double* __restrict__ kbar_t, int nqb, int nkb,
    double pscale, int lk, int p_all, uint64_t wp, int32_t* __restrict__ kv_idx,
    int32_t* __restrict__ kv_cnt, int32_t* __restrict__ rule_len) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* qs = reinterpret_cast<double*>(smem);                 // [8][D]
  double* srow = qs + kSelRows * D;                             // [8][nkb]
  unsigned long long* hmass =
      reinterpret_cast<unsigned long long*>(srow + (size_t)kSelRows * nkb);  // [8][256]
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(hmass + kSelRows * 256);      // [8][256]

  // workgroups in XCD-contiguous order: the 8 query-block groups of one head read the
  // same pooled K, which then stays in that XCD's L2
  const int ngroups = (nqb + kSelRows - 1) / kSelRows;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / ngroups;
  const int i0 = (tile - bh * ngroups) * kSelRows;
  const int t = threadIdx.x;
  for (int x = t; x < kSelRows * D; x += kSelThreads) {
    const int g = x / D, c = x % D;
    qs[x] = (i0 + g < nqb) ? qbar[((size_t)bh * nqb + i0 + g) * D + c] : 0.0;
  }
  __syncthreads();
  const double* kt = kbar_t + (size_t)bh * D * nkb;
  for (int j = t; j < nkb; j += kSelThreads) {
    double acc[kSelRows];
#pragma unroll
    for (int g = 0; g < kSelRows; ++g) acc[g] = 0.0;
    for (int c = 0; c < D; ++c) {
      const double kv = kt[(size_t)c * nkb + j];
#pragma unroll
      for (int g = 0; g < kSelRows; ++g) acc[g] = fma(qs[g * D + c], kv, acc[g]);
    }
#pragma unroll
    for (int g = 0; g < kSelRows; ++g) srow[(size_t)g * nkb + j] = pscale * acc[g];
  }
  __syncthreads();

  const int wv = t >> 6, lane = t & 63;
  const int i = i0 + wv;
  if (i >= nqb) return;
  const double* row = srow + (size_t)wv * nkb;
  const int j0 = lane * E;
  const int nval = max(0, min(E, nkb - j0));
  double s[E];
  double mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s[e] = (e < nval) ? row[j0 + e] : -INFINITY;
    mx = fmax(mx, s[e]);
  }
  mx = wave_max_f64(mx);
  double z = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s[e] = (e < nval) ? exp(s[e] - mx) : 0.0;
    z += s[e];
  }
  z = wave_sum_f64(z);
  uint64_t key[E], w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double p = s[e] / z;
    key[e] = (uint64_t)__double_as_longlong(p);
    w[e] = (uint64_t)__double2ull_rn(p * 0x1p62);
  }
  uint32_t* cnt = hcnt + wv * 256;
  unsigned long long* mass = hmass + wv * 256;

  SelectResult sel;
  if (p_all) {
    sel.all = 1;
  } else {
    sel = radix_select<E>(key, w, nval, lk, wp, cnt, mass);
  }
  int L;
  // kept flags and emission in ascending block order
  int tie_local = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) tie_local += (!sel.all && e < nval && key[e] == sel.tau) ? 1 : 0;
  const int tie_before = wave_incl_scan(tie_local) - tie_local;
  bool kept[E];
  int kc = 0, tr = tie_before;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bool k_ = false;
    if (e < nval) {
      if (sel.all) {
        k_ = true;
      } else if (key[e] > sel.tau) {
        k_ = true;
      } else if (key[e] == sel.tau) {
        k_ = tr < sel.take_ties;
        ++tr;
      }
    }
    kept[e] = k_;
    kc += k_ ? 1 : 0;
  }
  const int incl = wave_incl_scan(kc);
  L = __shfl(incl, 63, 64);
  int pos = incl - kc;
  int32_t* out = kv_idx + ((size_t)bh * nqb + i) * nkb;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (kept[e]) out[pos++] = j0 + e;
  if (lane == 0) kv_cnt[(size_t)bh * nqb + i] = L;

  if (rule_len) {
    int lp;
    if (p_all)
      lp = nkb;
    else if (L > lk)
      lp = L;
    else if (wp == 0)
      lp = 1;
    else {
      const SelectResult sp = radix_select<E>(key, w, nval, 1, wp, cnt, mass);
      lp = sp.all ? nkb : sp.len;
    }
    if (lane == 0) {
      rule_len[((size_t)bh * nqb + i) * 2 + 0] = lk;
      rule_len[((size_t)bh * nqb + i) * 2 + 1] = lp;
    }
  }
}

// ------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------
size_t mask_workspace_bytes(const Geometry& g) {
  const size_t a = align_up((size_t)g.bh() * g.nqb * g.d * sizeof(double), 256);
  const size_t b = align_up((size_t)g.bh() * g.d * g.nkb * sizeof(double), 256);
  return a + b;
}

void mask_workspace_carve(const Geometry& g, void* ws, double** qbar, double** kbar_t) {
  char* p = static_cast<char*>(ws);
  *qbar = reinterpret_cast<double*>(p);
  p += align_up((size_t)g.bh() * g.nqb * g.d * sizeof(double), 256);
  *kbar_t = reinterpret_cast<double*>(p);
}

template <int D, int E>
static hipError_t launch_select_t(const MaskArgs& a, hipStream_t s) {
  const Geometry& g = a.g;
  const size_t shm = (size_t)kSelRows * D * sizeof(double) +
                     (size_t)kSelRows * g.nkb * sizeof(double) +
                     (size_t)kSelRows * 256 * (sizeof(unsigned long long) + sizeof(uint32_t));
  if (shm > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)k_select<D, E>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(((g.nqb + kSelRows - 1) / kSelRows) * g.bh()));
  hipLaunchKernelGGL((k_select<D, E>), grid, dim3(kSelThreads), shm, s, a.qbar, a.kbar_t, g.nqb,
                     g.nkb, a.pooled_scale, a.lk, a.p_all, a.wp, a.kv_idx, a.kv_cnt, a.rule_len);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mask_d(const MaskArgs& a, unsigned stages, hipStream_t s) {
  const Geometry& g = a.g;
  if (stages & 1u) {
    dim3 grid((unsigned)((g.nqb + g.nkb) * g.bh()));
    hipLaunchKernelGGL((k_pool<D>), grid, dim3(256), 0, s, a.q, a.k, g.N, g.blk_q, g.nqb, g.nkb,
                       a.qbar, a.kbar_t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & 2u)) return hipSuccess;
  const int per_lane = (g.nkb + 63) / 64;
  if (per_lane <= 8) return launch_select_t<D, 8>(a, s);
  if (per_lane <= 16) return launch_select_t<D, 16>(a, s);
  return launch_select_t<D, 32>(a, s);
}

hipError_t launch_mask(const MaskArgs& a, unsigned stages, hipStream_t s) {
  return a.g.d == 64 ? launch_mask_d<64>(a, stages, s) : launch_mask_d<128>(a, stages, s);
}

}  // namespace spa
