// Internal launch interface between the C ABI (spa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spa {

struct Geometry {
  int B, H, N, d, blk_q, blk_k;
  int nqb, nkb;  // ceil(N / blk_q), ceil(N / blk_k)
  long long bh() const { return (long long)B * H; }
};

// ---- mask ----------------------------------------------------------------------------
struct MaskArgs {
  Geometry g;
  const uint16_t* q;
  const uint16_t* k;
  double pooled_scale;
  int lk;             // Top-k length, already clamped to [1, nkb]
  int p_all;          // p >= 1: keep every block
  uint64_t wp;        // Top-p target mass in units of 2^-62
  int32_t* kv_idx;
  int32_t* kv_cnt;
  int32_t* rule_len;  // may be null
  double* qbar;       // workspace [BH][nqb][d]
  double* kbar_t;     // workspace [BH][d][nkb]
};
size_t mask_workspace_bytes(const Geometry& g);
void mask_workspace_carve(const Geometry& g, void* ws, double** qbar, double** kbar_t);
// stage bits: 1 = pooling, 2 = selection
hipError_t launch_mask(const MaskArgs& a, unsigned stages, hipStream_t s);

// ---- forward ------------------------------------------------------------------------
struct FwdArgs {
  Geometry g;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  float scale;
  uint16_t* o;
  uint16_t* o_lo;  // may be null
  float* lse;
  uint16_t* v16;   // workspace (with o_lo): fp16 copy of V [BH][N][d]
  int32_t* vflag;  // workspace (with o_lo): [BH][Nkb], 1 where fp16 cannot carry the block
};
size_t fwd_workspace_bytes(const Geometry& g);
void fwd_workspace_carve(const Geometry& g, void* ws, FwdArgs* a);
// stage bits: 1 = the fp16 copy of V (with o_lo only), 2 = the attention
hipError_t launch_fwd(const FwdArgs& a, unsigned stages, hipStream_t s);

// ---- backward -----------------------------------------------------------------------
struct BwdArgs {
  Geometry g;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* o_lo;  // may be null
  const uint16_t* dout;
  const float* lse;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  float scale;
  void* dq;
  void* dk;
  void* dv;
  int grad_bf16;
  // workspace sections
  float* dsum;      // [BH][nqb * blk_q]: D = rowsum(dO * O), 0 on padding rows (k_dq writes)
  float* lse2;      // [BH][nqb * blk_q]: lse * log2(e), +inf on padding rows (k_dq writes)
  uint32_t* bits;   // [BH][ceil(nkb/32)][nqb]
  int32_t* q_idx;   // [BH][nkb][nqb]
  int32_t* q_cnt;   // [BH][nkb]
  uint16_t* do16;   // [BH][N][d]: fp16 copy of dO (k_dq writes)
  int32_t* kvflag;  // [BH][nkb]: 1 where the key block's V or a listed query block's dO is
                    // not read through fp16 (k_vflag writes V's, k_dq sets dO's)
  int32_t* order;   // [BH * nkb]: dK/dV workgroup dispatch order (k_collists writes)
  int32_t* ctr;     // [kDkdvCounters]: dK/dV work-queue tickets (k_collists zeroes them)
};
size_t bwd_workspace_bytes(const Geometry& g);
void bwd_workspace_carve(const Geometry& g, void* ws, BwdArgs* a);
// stage bits: 1 = the column lists and the dK/dV order, 2 = dQ (also D, lse2 and the fp16
// copy of dO), 4 = dK/dV
hipError_t launch_bwd(const BwdArgs& a, unsigned stages, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- mask without a caller workspace ------------------------------------------------------
// Size of the fixed device scratch (SPA_NOALLOC_SCRATCH_BYTES in spa.h).
constexpr size_t kNoallocScratchBytes = size_t(96) << 20;
// The current device's address of the fixed scratch (queried once per device).  Fails if
// `stream` (non-null) belongs to another device.
hipError_t noalloc_scratch(hipStream_t stream, void** out);

}  // namespace spa
