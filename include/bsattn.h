/*
 * bsattn.h - C ABI of the fused softmax-attention forward for AMD MI355X (gfx950).
 *
 * The library computes, for every (batch b, head h) and query row i,
 *
 *     O_i   = sum_j softmax_j(scale * q_i . k_j) v_j      over the allowed keys j
 *     LSE_i = ln sum_j exp(scale * q_i . k_j)             (natural log, fp32)
 *
 * without writing the N x N score or probability matrix to HBM: one
 * workgroup owns a query tile, streams key/value tiles past it and folds each
 * score tile into a running online-softmax state (max m, denominator l,
 * unnormalised accumulator A).  Sources of the operator:
 *   - "Exact Blocks, Rings, and Sparsity", section 1 (S = QK^T, P = softmax,
 *     O = PV), section 2 (online softmax state, merge invariant, saved LSE)
 *     and section 5 (block-sparse schedule over the active key-block set C_a);
 *   - "FlashAttention: Fast and Memory Efficient Exact Attention with IO
 *     Awareness" (notes), sections 5.1-5.2 (online softmax statistics,
 *     forward tiling) and 5.6 (block-sparse FlashAttention);
 *   - "block-sparse attention patterns", "Count active blocks and acknowledge
 *     the changed operator" (renormalisation over the sparse domain,
 *     triangular mask inside diagonal blocks, partial blocks, duplicates).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense and contiguous: Q, K, V, O are [B, H, N, d] with row
 *     stride d; LSE is [B, H, N] fp32.  Q, K, V, O have the same dtype.
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *     aligned to 16 bytes.  The caller owns every buffer, including any
 *     workspace an entry point takes; the library never allocates device
 *     memory and keeps no pointer after a call returns.
 *   - Calls are asynchronous on `stream` (0 = the null stream): the inputs
 *     must stay alive and unmodified until the stream has run the work.
 *   - Allowed pairs: causal keeps j <= i.  A query row with no allowed key
 *     gets O = 0 and LSE = -inf.
 *   - Status codes: every function returns ATTN_OK or a negative code, and
 *     validates all arguments before any launch (nothing is launched on
 *     error).  No C++ exception crosses this interface.
 *   - Tuning override (not part of the interface contract): the environment
 *     variable ATTN_TILE, read once per process, forces the workgroup shape of
 *     the bf16 dense and causal forwards to "128" or "256" query rows; any
 *     other value, or none, keeps the automatic choice.  The results are the
 *     same in both shapes.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,       /* null pointer, bad size, bad flag, misaligned pointer, malformed metadata */
    ATTN_EUNSUPPORTED = -2, /* valid request outside what the kernels implement (d, dtype, block size) */
    ATTN_ECAPACITY = -3,    /* caller-provided output or workspace buffer too small */
    ATTN_EHIP = -4          /* the HIP runtime reported an error at launch */
};

enum { ATTN_F32 = 0, ATTN_BF16 = 1 };

/* Bits of the per-entry flags of canonical block-sparse metadata. */
enum {
    ATTN_FLAG_DIAGONAL = 1, /* causal and the tile straddles the diagonal: triangular element mask */
    ATTN_FLAG_PARTIAL = 2   /* key block is the last one and N % block != 0: keys j >= N are masked */
};

/* Static text for a status code (never NULL). */
const char* attn_status_string(int status);

/*
 * attn_fwd - dense or causal attention forward.
 *   q, k, v : device, [B,H,N,d] of `dtype` (ATTN_BF16 or ATTN_F32), read only.
 *   o       : device, [B,H,N,d] of `dtype`, written (O in the input dtype).
 *   lse     : device, [B,H,N] fp32, written; natural-log log-sum-exp of the
 *             scaled logits over the allowed keys.
 *   B, H, N : >= 1; d in {64, 128}.
 *   scale   : finite and > 0 (e.g. 1/sqrt(d)); logits are scale * q.k.
 *   causal  : 0 or 1 (1 keeps j <= i; tiles wholly in the future are skipped,
 *             the diagonal tile gets the triangular element mask).
 * One kernel launch, no workspace: K and V tiles are read in place.
 * Source: "Exact Blocks, Rings, and Sparsity", section 2, forward kernel
 * ("What the forward kernel keeps on chip"): the host wrapper takes q, k, v
 * and a causal flag and returns O and the per-row LSE.
 * Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, int dtype, float scale, int causal,
             hipStream_t stream);

/*
 * attn_blockmask_build - HOST-side canonicaliser of block-sparse metadata.
 *   raw_row_ptr : host, int32 [meta_heads * nqb + 1], nqb = ceil(N / block);
 *                 CSR offsets into raw_col: starts at 0, non-decreasing.
 *   raw_col     : host, int32 [raw_row_ptr[last]]; key-block indices per
 *                 query block, any order, repeats allowed, rows may be empty,
 *                 and under causal may name future blocks.  An index outside
 *                 [0, nqb) is an error (ATTN_EINVAL).
 *   meta_heads  : number of independent patterns (1: shared by every (b,h);
 *                 H: one per head, the same for every batch).
 *   N, block    : sequence length >= 1 and block size b >= 1.
 *   causal      : 0 or 1.
 * Outputs (host buffers owned by the caller):
 *   row_ptr [meta_heads*nqb + 1], col [capacity], flags [capacity]: canonical
 *     CSR: each row strictly increasing and unique; future blocks dropped when
 *     causal; flags per entry use ATTN_FLAG_*.
 *   capacity          : entries available in col/flags; raw nnz always suffices.
 *                       With capacity 0, col and flags may be NULL (a sizing
 *                       call: ATTN_ECAPACITY and nnz, or ATTN_OK if nothing is
 *                       listed); with capacity > 0 both are required.
 *   nnz               : entries written (or needed, with ATTN_ECAPACITY).
 *   allowed_pairs     : [meta_heads] logical (i, j) pairs with i, j < N allowed
 *                       by each pattern, per (b, h).
 *   executed_tile_pairs : [meta_heads] block x block tiles executed per (b, h).
 * Source: "Exact Blocks, Rings, and Sparsity", section 5, "Why the sparse
 * unit is usually a block" (active set C_a per query tile); "block-sparse
 * attention patterns" (duplicates count once, partial blocks, report logical
 * allowed pairs next to executed tile work).
 * Errors: ATTN_EINVAL, ATTN_ECAPACITY (row_ptr, nnz and the counts are still
 * written; col/flags hold only the first `capacity` entries).
 */
int attn_blockmask_build(const int32_t* raw_row_ptr, const int32_t* raw_col,
                         int64_t meta_heads, int64_t N, int64_t block, int causal,
                         int32_t* row_ptr, int32_t* col, uint8_t* flags, int64_t capacity,
                         int64_t* nnz, int64_t* allowed_pairs, int64_t* executed_tile_pairs);

/*
 * attn_fwd_blocksparse - block-sparse attention forward, renormalised over
 * the allowed pairs (drop-and-renormalize).
 *   q, k, v, o, lse, B, H, N, d, dtype, scale, causal: as for attn_fwd.
 *   block      : b in {64, 128}: query and key block size of the metadata.
 *   row_ptr    : DEVICE int32 [meta_heads * nqb + 1], canonical CSR offsets.
 *   col, flags : DEVICE int32 / uint8 [nnz]: canonical entries and their
 *                ATTN_FLAG_* bits, as written by attn_blockmask_build (sorted,
 *                unique: a duplicated entry would be counted twice).
 *   nnz        : number of entries in col/flags; offsets are clamped to it and
 *                entries outside [0, nqb) are skipped, so malformed metadata
 *                cannot make the kernel read out of bounds.
 *   meta_heads : 1 (one pattern for every (b,h)), H (pattern h for head h) or
 *                B*H (pattern b*H + h, as the device selector writes).
 * One kernel launch, no workspace.
 * Source: "Exact Blocks, Rings, and Sparsity", section 5 (the outer loop runs
 * over b in C_a; skipped tiles skip their loads and both products) and
 * section 6 (drop-and-renormalize); "block-sparse attention patterns"
 * (triangular element mask inside diagonal blocks, empty rows).
 * Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, int dtype, float scale,
                         int causal, int64_t block,
                         const int32_t* row_ptr, const int32_t* col, const uint8_t* flags,
                         int64_t nnz, int64_t meta_heads, hipStream_t stream);

/*
 * Two-step form of the bf16 path, for callers that run many forwards against
 * the same V: V is transposed once, and the fused kernel then reads V^T tiles
 * with plain 16-byte LDS reads instead of transposing LDS reads (about 1 %
 * less kernel time at B=1 H=32 N=8192 d=128).
 *
 * attn_prepared_v_bytes - bytes of the V^T buffer for these sizes:
 *   B*H*d*ceil(N/128)*128*2 (ATTN_BF16 only); -1 for sizes or a dtype the
 *   kernels do not accept.
 *
 * attn_prepare_v - write V transposed per head into `vt` (the layout the
 *   fused kernel reads: [B*H][d][ceil(N/128)*128] bf16, keys permuted inside
 *   each 16-key group, keys >= N zero).
 *   v : device [B,H,N,d] bf16.  vt : device, vt_bytes >=
 *   attn_prepared_v_bytes(...), 16-byte aligned, must not overlap v.
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED (dtype other than ATTN_BF16, d,
 *   or B*H > 65535: the transpose takes one grid row per head), ATTN_ECAPACITY,
 *   ATTN_EHIP.
 *
 * attn_fwd_prepared / attn_fwd_blocksparse_prepared - attn_fwd /
 *   attn_fwd_blocksparse without the V argument: V^T is read from `vt`, which
 *   attn_prepare_v filled for the same B, H, N, d (ATTN_BF16 only).  Results
 *   are bitwise equal to attn_fwd / attn_fwd_blocksparse (same arithmetic in
 *   the same order).
 * Source: as for attn_fwd and attn_fwd_blocksparse.
 */
int64_t attn_prepared_v_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

int attn_prepare_v(const void* v, int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                   void* vt, int64_t vt_bytes, hipStream_t stream);

int attn_fwd_prepared(const void* q, const void* k, void* o, float* lse,
                      int64_t B, int64_t H, int64_t N, int64_t d, int dtype, float scale, int causal,
                      const void* vt, int64_t vt_bytes, hipStream_t stream);

int attn_fwd_blocksparse_prepared(const void* q, const void* k, void* o, float* lse,
                                  int64_t B, int64_t H, int64_t N, int64_t d, int dtype, float scale,
                                  int causal, int64_t block,
                                  const int32_t* row_ptr, const int32_t* col, const uint8_t* flags,
                                  int64_t nnz, int64_t meta_heads, const void* vt,
                                  int64_t vt_bytes, hipStream_t stream);

/*
 * Backward pass (gradients of the forward above; ATTN_BF16 only).
 *
 * Given the forward's inputs, its outputs O and LSE, and the upstream
 * gradient dO, the library rebuilds P tile by tile from Q, K and LSE
 * (P_ij = exp(scale q_i.k_j - LSE_i) on allowed pairs), forms dP = dO V^T and
 * dS = P (dP - D) with D_i = dO_i . O_i, and accumulates dV = P^T dO,
 * dK = scale dS^T Q and dQ = scale dS K, never writing S, P, dP or dS to HBM.
 * Source: "Exact Blocks, Rings, and Sparsity", section 3 ("FlashAttention
 * Backward: recomputing P": the D_i preprocessing step, the LSE-based
 * reconstruction of P, the two traversals that own dK/dV and dQ); FlashAttention
 * notes, section 5.3 (backward recomputation).  Rows without allowed keys
 * (LSE = -inf) get dQ = 0 and contribute nothing.  The launch sequence is:
 * the row statistics (LSE in base 2 and D) into the workspace, the dK/dV
 * kernel, the dQ kernel, all on `stream`; results are deterministic (no
 * atomics).
 *
 * attn_bwd_workspace_bytes - device workspace attn_bwd needs (the row
 *   statistics): B*H*(ceil(N/128)*2 + 1)*512 bytes.  attn_bwd_gqa and the
 *   block-sparse backward size theirs with attn_bwd_gqa_workspace_bytes and
 *   attn_bwd_blocksparse_workspace_bytes.
 *   Returns -1 for sizes or a dtype the kernels do not accept.
 *
 * attn_bwd - gradients of attn_fwd.
 *   q, k, v  : device [B,H,N,d] bf16, the forward's inputs.
 *   o, lse   : device, the forward's outputs for the same q, k, v, scale and
 *              causal flag (O [B,H,N,d] bf16, LSE [B,H,N] fp32).
 *   dout     : device [B,H,N,d] bf16, the upstream gradient dO.
 *   dq, dk, dv : device [B,H,N,d] bf16, written (overwritten, not accumulated).
 *   B, H, N, d, scale, causal : as for attn_fwd; dtype must be ATTN_BF16.
 *   workspace : device, at least attn_bwd_workspace_bytes(...) bytes, aligned to
 *              256 bytes, overwritten, not overlapping any tensor argument.
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED (dtype, d), ATTN_ECAPACITY
 *   (workspace too small), ATTN_EHIP.
 */
int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, float scale,
             int causal, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * attn_bwd_noalloc - attn_bwd for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving or training loops, harnesses
 *   that forbid hipMalloc): the same gradients, bitwise, with no workspace
 *   argument.  The row statistics go to a fixed array of
 *   ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU the
 *   library runs on, held until the process ends; the call itself allocates
 *   nothing (no hipMalloc, no allocating library routine).
 *   Arguments, layouts and results as for attn_bwd (dense or causal,
 *   ATTN_BF16); the caller still owns q, k, v, o, lse, dout, dq, dk, dv.
 *   Limit: attn_bwd_workspace_bytes(B, H, N, d, dtype) must not exceed
 *   ATTN_NOALLOC_SCRATCH_BYTES (B*H*(2*ceil(N/128)+1)*512 bytes, e.g. B*H*N
 *   up to about 4.1M rows at N = 8192); larger sizes return ATTN_ECAPACITY
 *   before any launch.
 *   Calls on one GPU share its array and each overwrites it: calls that can
 *   overlap on one GPU (different streams, host threads) race and must be
 *   ordered by the caller.  Nothing in the array needs clearing between calls
 *   (the first kernel of a call writes every statistic the later ones read).
 *   The array is the current HIP device's (hipGetDevice); the stream and the
 *   tensors must be on that device.  The first call on a device looks up the
 *   array's address there (hipGetSymbolAddress, no allocation); a caller that
 *   captures graphs can make that first call before capturing.
 *   Errors: as for attn_bwd; ATTN_EHIP also when the array's device address
 *   cannot be obtained.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32LL << 20)

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                     int dtype, float scale, int causal, hipStream_t stream);

/*
 * attn_blockmask_transpose - HOST-side transpose of block-sparse metadata: for
 *   each key block, the query blocks whose lists name it, in increasing order
 *   (the dK/dV pass of the backward owns a key block and visits exactly these).
 *   row_ptr, col : host, CSR as written by attn_blockmask_build ([meta_heads *
 *                  nb + 1] offsets, nb = ceil(N / block); entries in [0, nb)).
 *   t_row_ptr    : host [meta_heads * nb + 1], written.
 *   t_col        : host [capacity], written (nnz = row_ptr[last] entries).
 *   Errors: ATTN_EINVAL (malformed CSR, null pointers), ATTN_ECAPACITY
 *   (t_row_ptr is still written).
 */
int attn_blockmask_transpose(const int32_t* row_ptr, const int32_t* col, int64_t meta_heads, int64_t N,
                             int64_t block, int32_t* t_row_ptr, int32_t* t_col, int64_t capacity);

/*
 * attn_bwd_blocksparse_workspace_bytes - device workspace attn_bwd_blocksparse
 *   and attn_bwd_blocksparse_gqa use for this metadata: the row statistics,
 *   the split plan, and fp32 partial dK, dV (2 * block * d * 4 bytes each) for
 *   the pieces of long key-block lists.  A key block whose transposed list
 *   holds more than 32 query tiles of 64 rows is processed by up to 8
 *   workgroups, one per piece of the list; their partial sums are added in
 *   piece order by a reduction pass (deterministic).
 *   t_row_ptr : HOST copy of attn_blockmask_transpose's offsets for the
 *               metadata ([meta_heads * ceil(N / block) + 1]), or NULL: then
 *               the minimum workspace (no list is split).  A workspace between
 *               the minimum and the returned size is accepted; the split is
 *               then turned off for the whole call.  A call uses at most 2^18
 *               partial slots; metadata that would need more gets the minimum
 *               (no split).
 *   Returns -1 for sizes, dtype, block or meta_heads the backward does not accept.
 *
 * attn_bwd_blocksparse - gradients of attn_fwd_blocksparse.
 *   Tensor and size arguments as for attn_bwd; block, row_ptr, col, flags,
 *   nnz, meta_heads as for attn_fwd_blocksparse (DEVICE copies of the
 *   canonical metadata); t_row_ptr, t_col: DEVICE copies of
 *   attn_blockmask_transpose's output for the same metadata (nnz entries).
 *   workspace : device, at least attn_bwd_blocksparse_workspace_bytes(..., NULL,
 *   ...) bytes, 256-byte aligned.  Offsets are clamped to nnz and out-of-range
 *   entries are skipped, as in the forward.  Source: as for attn_bwd, over the
 *   active key-block sets of "Exact Blocks, Rings, and Sparsity", section 5.
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ECAPACITY, ATTN_EHIP.
 */
int64_t attn_bwd_blocksparse_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype,
                                             int64_t block, const int32_t* t_row_ptr, int64_t meta_heads);

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                         int dtype, float scale, int causal, int64_t block,
                         const int32_t* row_ptr, const int32_t* col, const uint8_t* flags, int64_t nnz,
                         const int32_t* t_row_ptr, const int32_t* t_col, int64_t meta_heads,
                         void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Key splits and ring steps (ATTN_BF16): partial states and their merge.
 *
 * A partial state of a query row over a set of keys is (O_s, LSE_s): the
 * output normalised over those keys only, and the log-sum-exp of their scaled
 * logits (natural log; O_s = 0 and LSE_s = -inf when the row sees none of
 * them).  States over disjoint key sets merge exactly, in any order:
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * Source: "Exact Blocks, Rings, and Sparsity", section 2 (mergeable online
 * softmax state), section 4 (Ring Attention: device g keeps Q_g, meets one
 * KV block per step, merges; causal steps skip blocks wholly in the future and
 * mask the one crossing the diagonal).  Partial outputs are fp32.
 *
 * attn_fwd_splitkv - attn_fwd computed as num_splits key ranges in one
 *   launch (for shapes whose B*H*ceil(N/256) query tiles cannot fill the
 *   GPU), then merged: same arguments as attn_fwd plus num_splits in [1, 64]
 *   (key ranges of whole 64-key tiles; fewer ranges when N is small).
 *   workspace : at least attn_fwd_splitkv_workspace_bytes(...) bytes, aligned
 *   to 256 bytes (the fp32 partial states of every range).
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED (dtype, d), ATTN_ECAPACITY, ATTN_EHIP.
 */
int64_t attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                                         int64_t num_splits);

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t N, int64_t d, int dtype, float scale, int causal, int64_t num_splits,
                     void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * attn_fwd_block - one ring step: the partial state of query rows against one
 *   key/value block.
 *   q        : device [B,H,Nq,d] bf16; row i sits at global position q_offset + i.
 *   k, v     : device [B,H,Nk,d] bf16; key j sits at global position k_offset + j.
 *   o_part   : device [B,H,Nq,d] fp32, written: O_s of each row over this block.
 *   lse_part : device [B,H,Nq] fp32, written: LSE_s (-inf for rows that see no key).
 *   causal   : 1 keeps the pairs with k_offset + j <= q_offset + i.
 *   q_offset, k_offset : in [0, 2^40].
 *   One kernel launch, no workspace.
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_fwd_block(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int64_t B,
                   int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype, float scale, int causal,
                   int64_t q_offset, int64_t k_offset, hipStream_t stream);

/*
 * attn_merge - merge num_parts partial states over disjoint key sets.
 *   o_parts   : device fp32 [num_parts][B,H,N,d]; lse_parts : device fp32
 *               [num_parts][B,H,N] (num_parts in [1, 1024]).
 *   o, lse    : device, written: O [B,H,N,d] of out_dtype (ATTN_F32 or
 *               ATTN_BF16) and LSE [B,H,N] fp32.  With out_dtype ATTN_F32, o
 *               and lse may be exactly part 0 (merge in place, as a ring step
 *               folds its new block into the running state); no other overlap.
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED (d, out_dtype), ATTN_EHIP.
 */
int attn_merge(const float* o_parts, const float* lse_parts, int64_t num_parts, int64_t B, int64_t H,
               int64_t N, int64_t d, void* o, float* lse, int out_dtype, hipStream_t stream);

/*
 * Grouped-query attention: H query heads share Hkv key/value heads (H % Hkv ==
 * 0); query head h reads key/value head h / (H / Hkv).  Under block sparsity
 * the query heads of a group can share one key-block list (meta_heads == Hkv),
 * so the group loads one set of K/V blocks rather than the union of unrelated
 * sets.  Source: "Exact Blocks, Rings, and Sparsity", section 5 ("The selector
 * must cost less than the tiles it skips": GQA and the union of per-head
 * selections) and the NSA remarks on query heads sharing one KV cache.
 *
 *   q, o, dq, dout : [B,H,N,d];  k, v, dk, dv : [B,Hkv,N,d];  lse : [B,H,N].
 *   The other arguments are those of the non-grouped entry points; meta_heads
 *   may also be Hkv.  Each dK, dV head is the sum of the contributions of its
 *   group's query heads (one workgroup per key/value head sums them in a fixed
 *   order: deterministic).
 *   Workspaces: the forwards need none; the backward needs
 *   attn_bwd_gqa_workspace_bytes(B, H, Hkv, N, d, dtype).
 *   Errors: as for the non-grouped entry points; ATTN_EINVAL also when Hkv < 1,
 *   Hkv > H or H % Hkv != 0.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                 int64_t Hkv, int64_t N, int64_t d, int dtype, float scale, int causal, hipStream_t stream);

int attn_fwd_blocksparse_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                             int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype, float scale, int causal,
                             int64_t block, const int32_t* row_ptr, const int32_t* col, const uint8_t* flags,
                             int64_t nnz, int64_t meta_heads, hipStream_t stream);

int64_t attn_bwd_gqa_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype);

int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype,
                 float scale, int causal, void* workspace, int64_t workspace_bytes, hipStream_t stream);

int attn_bwd_blocksparse_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv,
                             int64_t N, int64_t d, int dtype, float scale, int causal, int64_t block,
                             const int32_t* row_ptr, const int32_t* col, const uint8_t* flags, int64_t nnz,
                             const int32_t* t_row_ptr, const int32_t* t_col, int64_t meta_heads,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Mean-pooled block selector: builds the active key-block sets C_a on the
 * device.  Source: "Exact Blocks, Rings, and Sparsity", section 5, "Fixed
 * pooling: a cheap proxy, not the true block mass" (a key block is
 * represented by the mean of its keys; ranking by the mean logit approximates
 * ranking by block mass when the block is homogeneous) and "The selector must
 * cost less than the tiles it skips" (GQA: heads of a group share one choice).
 *   score(a, b) = scale * mean(Q rows of query block a) . mean(K rows of key
 *   block b), the mean logit of the tile (means over the tokens a block holds);
 *   C_a = the topk highest-scoring candidates (every key block, or kb <= a when
 *   causal), ties to the lower index, written ascending.
 *   q : device [B,H,N,d], k : device [B,Hkv,N,d] (ATTN_BF16 or ATTN_F32).
 *   block in {64, 128}; topk in [1, 64]; ceil(N/block) <= 2048.
 *   share_groups : 1 averages the scores of each group's H/Hkv query heads and
 *                  gives every head of the group the same list; 0 selects per head.
 *   row_ptr : device int32 [B*H*nb + 1], col : device int32 [capacity],
 *   flags : device uint8 [capacity]: written; canonical metadata with one
 *           pattern per (batch, head), b-major (pass meta_heads = B*H to the
 *           block-sparse entry points).  nnz = attn_select_meanpool_nnz(...).
 *   workspace : device, attn_select_meanpool_workspace_bytes(...) bytes (the
 *               fp32 block means), 16-byte aligned.
 *   Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED (dtype, d, block, too many blocks,
 *   or nb * B * (H + Hkv) >= 2^24: the pooling launch takes one workgroup per
 *   head of Q or K and block), ATTN_ECAPACITY (capacity or workspace too
 *   small), ATTN_EHIP.
 */
int64_t attn_select_meanpool_nnz(int64_t B, int64_t H, int64_t N, int64_t block, int causal, int64_t topk);

int64_t attn_select_meanpool_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                             int64_t block);

int attn_select_meanpool(const void* q, const void* k, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                         int dtype, float scale, int causal, int64_t block, int64_t topk, int share_groups,
                         int32_t* row_ptr, int32_t* col, uint8_t* flags, int64_t capacity, void* workspace,
                         int64_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
