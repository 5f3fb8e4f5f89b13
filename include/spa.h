/*
 * spa.h -- hybrid Top-k + Top-p block-sparse attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libspa.so.  Three operations, as the method is built from them
 * (mindverse article "Optimierung der Effizienz von Video-Diffusionsmodellen durch
 * SpargeAttention2", section "Effiziente Kernel-Implementierung und Modellanpassung":
 * mask construction, and the forward and backward passes of block-sparse attention
 * that skip the masked tiles' matrix products and softmax):
 *
 *   spa_build_mask       block-mean pooling of Q and K, the pooled row softmax, and per
 *                        query block the union of the Top-k and Top-p key-block sets
 *                        (same article, sections "Maskierungsstrategien: Top-k und Top-p"
 *                        and "Hybride Top-k+Top-p Maskierung");
 *   spa_sparse_attn_fwd  softmax attention over the kept tiles only, with the row
 *                        log-sum-exp saved (section "Block-dünnbesetzte Aufmerksamkeit":
 *                        a tile is kept whole or dropped);
 *   spa_sparse_attn_bwd  dQ, dK, dV over the same kept tiles with the mask held fixed
 *                        (abstract page "SpargeAttention2: Trainable Sparse Attention via
 *                        Hybrid Top-k+Top-p Masking and Distillation Fine-Tuning",
 *                        contribution (ii): trainable sparse attention).
 *
 * Conventions for every entry point
 *   - Tensors are dense, contiguous, row-major [B, H, N, d] in device memory that the
 *     caller owns (allocated with hipMalloc or by a framework on the same device).
 *     Q, K, V, O and dO are bf16 (IEEE bfloat16 bit patterns).
 *   - Blocks: query block i covers tokens [i*blk_q, min(N, (i+1)*blk_q)), key block j
 *     covers [j*blk_k, min(N, (j+1)*blk_k)); Nqb = ceil(N/blk_q), Nkb = ceil(N/blk_k).
 *     The last block of each kind may be partial.
 *   - Supported: d in {64, 128}; blk_q in {64, 128}; blk_k == 64; B, H, N >= 1;
 *     B*H*N*d < 2^31; Nkb <= 2048.
 *   - All calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream).  None synchronises the host, allocates device memory or keeps
 *     state between calls; concurrent calls on different streams with disjoint outputs
 *     and workspaces are safe.
 *   - Invalid arguments are rejected before any launch with a negative status and no
 *     output is touched.  SPA_E_LAUNCH reports a failed kernel launch; outputs are then
 *     undefined.  Results are deterministic: the same inputs give bitwise-identical
 *     outputs on every run.
 */
#ifndef SPA_H
#define SPA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define SPA_API __attribute__((visibility("default")))
#else
#define SPA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPA_OK = 0,
  SPA_E_NULL = -1,        /* a required pointer is NULL                              */
  SPA_E_SHAPE = -2,       /* B, H or N < 1, or the tensor is too large               */
  SPA_E_PARAM = -3,       /* k_frac or p outside [0, 1] or NaN; scale NaN or inf     */
  SPA_E_UNSUPPORTED = -4, /* d, blk_q, blk_k or Nkb outside the supported set        */
  SPA_E_WORKSPACE = -5,   /* workspace smaller than the *_workspace_bytes figure     */
  SPA_E_LAUNCH = -6,      /* the HIP runtime reported an error at launch             */
  SPA_E_SCRATCH = -7      /* spa_build_mask_noalloc: the problem needs more than the
                             fixed scratch, or the scratch is not available            */
} spa_status;

typedef struct {
  int32_t B, H, N, d; /* tensor shape [B, H, N, d]                    */
  int32_t blk_q;      /* query block size (64 or 128)                 */
  int32_t blk_k;      /* key block size (64)                          */
} spa_dims;

/* Bytes of device workspace spa_build_mask needs (pooled Q and K in fp64, 256-byte
 * aligned sections).  Returns 0 for dims that spa_build_mask would reject. */
SPA_API size_t spa_mask_workspace_bytes(const spa_dims* dims);

/*
 * Builds the hybrid Top-k + Top-p block mask (mindverse article, sections
 * "Maskierungsstrategien: Top-k und Top-p" and "Hybride Top-k+Top-p Maskierung").
 * Per (b, h):
 *   qbar_i = mean of the valid rows of query block i, kbar_j likewise (fp64);
 *   P[i, :] = softmax_j(pooled_scale * <qbar_i, kbar_j>)   (fp64);
 *   order the row by P descending, ties by the lower block index;
 *   Lk = clamp(ceil(k_frac * Nkb - 1e-9), 1, Nkb);
 *   Lp = the shortest prefix of that order whose cumulative P is >= p
 *        (p >= 1 keeps every block; p <= 0 gives 1);
 *   the kept set is the prefix of length L = max(Lk, Lp): the union of both rules.
 * k_frac = 0 gives the pure Top-p rule and p = 0 the pure Top-k rule.
 *
 *   q, k          bf16 [B, H, N, d] device.
 *   k_frac, p     in [0, 1].
 *   pooled_scale  scale inside the pooled softmax; <= 0 selects 1/sqrt(d).
 *   kv_idx        int32 [B, H, Nqb, Nkb] device, out: row (b,h,i) holds its kept key
 *                 blocks in ascending order in its first kv_cnt[b,h,i] entries; the
 *                 remaining entries of the row are not written.
 *   kv_cnt        int32 [B, H, Nqb] device, out: L per row (1 <= L <= Nkb).
 *   rule_len      int32 [B, H, Nqb, 2] device, out, or NULL: (Lk, Lp) per row.
 *   ws, ws_bytes  device workspace of at least spa_mask_workspace_bytes(dims).
 */
SPA_API int spa_build_mask(const spa_dims* dims, const void* q, const void* k, double k_frac,
                   double p, double pooled_scale, int32_t* kv_idx, int32_t* kv_cnt,
                   int32_t* rule_len, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the fixed device scratch that spa_build_mask_noalloc uses. */
#define SPA_NOALLOC_SCRATCH_BYTES (96u << 20)

/*
 * spa_build_mask without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus ws, ws_bytes), results and
 * validation as spa_build_mask.  The pooled means live in a fixed device array of
 * SPA_NOALLOC_SCRATCH_BYTES (96 MiB) that every GPU the library runs on holds until the
 * process ends; a problem whose spa_mask_workspace_bytes exceeds it (B*H*N*d larger than
 * about 5e8, e.g. more than twice the B=1, H=40, N=75600, d=128 layer) returns
 * SPA_E_SCRATCH before any launch.  The first call on a device queries the array's address
 * there (hipGetSymbolAddress; no allocation).  `stream` must belong to the current device
 * (else SPA_E_SCRATCH).  All calls on one GPU share its array: calls that overlap on one
 * GPU (different streams, or threads) race and must be ordered by the caller; calls in
 * sequence on one stream are safe.
 */
SPA_API int spa_build_mask_noalloc(const spa_dims* dims, const void* q, const void* k,
                                   double k_frac, double p, double pooled_scale,
                                   int32_t* kv_idx, int32_t* kv_cnt, int32_t* rule_len,
                                   void* stream);

/*
 * Block-sparse attention forward (mindverse article, sections "Block-dünnbesetzte
 * Aufmerksamkeit" and "Effiziente Kernel-Implementierung und Modellanpassung").
 * For every token t of query block i, over the keys u of the listed key blocks with
 * u < N:  z_tu = scale * <q_t, k_u>;  O_t = sum_u softmax_u(z_t.) v_u;
 * LSE_t = ln sum_u exp(z_tu).  bf16 MFMA products, fp32 accumulation and softmax.
 *
 *   q, k, v       bf16 [B, H, N, d] device.
 *   kv_idx, kv_cnt  lists in spa_build_mask's layout; each list must be ascending,
 *                 unique, within [0, Nkb) and non-empty (they are trusted).
 *   scale         softmax scale; <= 0 selects 1/sqrt(d).
 *   o             bf16 [B, H, N, d] device, out: O rounded to nearest even.
 *   o_lo          bf16 [B, H, N, d] device, out, or NULL: the rounding residual of O.
 *                 Request it when a backward pass follows: the gradients depend on
 *                 D = <dO, O> to first order, and bf16 O alone leaves D off by about
 *                 2^-9 |dO| |O|.  With o_lo the probabilities enter P*V as one fp16
 *                 rounding against an fp16 copy of V (fp16 has three more mantissa bits
 *                 than bf16), so o + o_lo carries O to about 12 significant bits.  A query
 *                 block whose list holds a key block of V that the copy does not carry
 *                 to within 2^-16 of the block's largest magnitude (a value of magnitude
 *                 65504 or more, or only values below 2^-9 with some in fp16's subnormal
 *                 range) takes bf16 V with P as a bf16 hi + lo pair instead (about 16
 *                 bits).  Without o_lo, P enters as bf16.
 *   lse           fp32 [B, H, N] device, out (natural log).
 *   ws, ws_bytes  device workspace of at least spa_fwd_workspace_bytes(dims) when o_lo is
 *                 given (the fp16 copy of V and a flag per key block); ignored, and may be
 *                 NULL, without o_lo.
 */
SPA_API int spa_sparse_attn_fwd(const spa_dims* dims, const void* q, const void* k, const void* v,
                        const int32_t* kv_idx, const int32_t* kv_cnt, double scale, void* o,
                        void* o_lo, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace spa_sparse_attn_fwd needs with o_lo (an fp16 copy of V and
 * one int32 flag per key block, 256-byte aligned sections).  0 for rejected dims. */
SPA_API size_t spa_fwd_workspace_bytes(const spa_dims* dims);

/* Bytes of device workspace spa_sparse_attn_bwd needs (D = rowsum(dO*O) and lse*log2(e)
 * per row, padded to whole query blocks, the kept-tile bitmap, the per-key-block
 * query-block lists and their dispatch order, an fp16 copy of dO, one int32 flag per
 * key block (a listed query block's dO needs bf16) and ten int32 work-queue counters of
 * the dK/dV kernel; SPA_BWD_PREP zeroes the flags and the counters, and each dK/dV launch
 * leaves the counters at zero; 256-byte aligned sections).  0 for rejected dims. */
SPA_API size_t spa_bwd_workspace_bytes(const spa_dims* dims);

/*
 * Block-sparse attention backward with the mask held fixed (abstract page, contribution
 * (ii); mindverse article, section "Effiziente Kernel-Implementierung und
 * Modellanpassung").  With the loss sum_t <O_t, dO_t> and A the attention weights of
 * the forward pass:  D_t = <dO_t, O_t>;  dS_tu = A_tu (<dO_t, v_u> - D_t);
 * dQ_t = scale * sum_u dS_tu k_u;  dK_u = scale * sum_t dS_tu q_t;  dV_u = sum_t A_tu dO_t.
 * The accumulation order is fixed (ascending block index), so results are bitwise
 * reproducible.  dS enters dQ and dK as a bf16 hi + lo pair.  In dV = P^T dO, P enters as
 * one fp16 rounding against an fp16 copy of dO (P <= 1; the copy is exact from 2^-14 to
 * below 65504 in magnitude and keeps an absolute 2^-25 below 2^-14).  A key block whose
 * query-block list holds a query block of dO, or whose own V, that the copy does not
 * carry to within 2^-16 of the block's largest magnitude (a value beyond fp16's range, or
 * only values below 2^-9 with some in fp16's subnormal range) uses bf16 dO with P as a
 * bf16 hi + lo pair instead.
 *
 *   q, k, v, o, dout  bf16 [B, H, N, d] device (o and lse from spa_sparse_attn_fwd).
 *   o_lo          bf16 [B, H, N, d] device or NULL: the forward pass's residual; with it
 *                 D uses o + o_lo, without it o alone.
 *   lse           fp32 [B, H, N] device.
 *   kv_idx, kv_cnt  the lists given to the forward pass.
 *   scale         as in the forward pass.
 *   dq, dk, dv    [B, H, N, d] device, out: fp32 if grad_dtype == 0, bf16 if 1.
 *   ws, ws_bytes  device workspace of at least spa_bwd_workspace_bytes(dims).
 */
SPA_API int spa_sparse_attn_bwd(const spa_dims* dims, const void* q, const void* k, const void* v,
                        const void* o, const void* o_lo, const void* dout, const float* lse,
                        const int32_t* kv_idx, const int32_t* kv_cnt, double scale, void* dq,
                        void* dk, void* dv, int grad_dtype, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * Staged variants, for callers that schedule or time the phases separately (each stage
 * is one or more kernel launches on `stream`; running the stages in increasing bit order,
 * in one call or several with the same arguments and workspace, equals the unstaged
 * call).  Stage bits of spa_build_mask_stages: SPA_MASK_POOL (block means of Q and K
 * into the workspace), SPA_MASK_SELECT (pooled softmax and selection from the
 * workspace).  Stage bits of spa_sparse_attn_fwd_stages: SPA_FWD_PREP (with o_lo, the
 * fp16 copy of V and its per-block flags, into the workspace; it reads V only, so a caller
 * may run it on a second stream while the mask is built; without o_lo it launches
 * nothing), SPA_FWD_ATTN (the attention; with o_lo it reads what SPA_FWD_PREP wrote from
 * the same V).  Stage bits of spa_sparse_attn_bwd_stages: SPA_BWD_PREP (the
 * per-key-block query-block lists, the order in which their workgroups run and each key
 * block's fp16 flag of V, into the workspace; it reads kv_idx, kv_cnt and V only, so a
 * caller may run it on a second stream once the mask exists, e.g. during the forward),
 * SPA_BWD_DQ (dQ; also writes D and lse * log2(e) of every row and the fp16 copy of dO
 * into the workspace, and flags the key blocks of query blocks whose dO the copy does not
 * carry), SPA_BWD_DKDV
 * (dK, dV; reads what the other two wrote).  A zero or unknown stage mask gives
 * SPA_E_PARAM.
 */
enum {
  SPA_MASK_POOL = 1, SPA_MASK_SELECT = 2, SPA_MASK_ALL = 3,
  SPA_FWD_PREP = 1, SPA_FWD_ATTN = 2, SPA_FWD_ALL = 3,
  SPA_BWD_PREP = 1, SPA_BWD_DQ = 2, SPA_BWD_DKDV = 4, SPA_BWD_ALL = 7
};

SPA_API int spa_build_mask_stages(const spa_dims* dims, const void* q, const void* k,
                                  double k_frac, double p, double pooled_scale, int32_t* kv_idx,
                                  int32_t* kv_cnt, int32_t* rule_len, void* ws, size_t ws_bytes,
                                  unsigned stages, void* stream);

SPA_API int spa_sparse_attn_fwd_stages(const spa_dims* dims, const void* q, const void* k,
                                       const void* v, const int32_t* kv_idx,
                                       const int32_t* kv_cnt, double scale, void* o, void* o_lo,
                                       float* lse, void* ws, size_t ws_bytes, unsigned stages,
                                       void* stream);

SPA_API int spa_sparse_attn_bwd_stages(const spa_dims* dims, const void* q, const void* k,
                                       const void* v, const void* o, const void* o_lo,
                                       const void* dout, const float* lse, const int32_t* kv_idx,
                                       const int32_t* kv_cnt, double scale, void* dq, void* dk,
                                       void* dv, int grad_dtype, void* ws, size_t ws_bytes,
                                       unsigned stages, void* stream);

/* Static text for a status code. */
SPA_API const char* spa_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
SPA_API int spa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H */
