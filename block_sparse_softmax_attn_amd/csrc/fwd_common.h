// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

// Everything a forward launch needs; built and validated by the host layer.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t BH;          // B * H (query heads)
    int H;
    int Hkv;             // key/value heads per batch entry; H % Hkv == 0
    int N;
    int d;
    float scale_log2;    // scale * log2(e): logits are handled in base-2 units
    int causal;
    // block-sparse schedule (sparse launches only)
    const int32_t* row_ptr;
    const int32_t* col;
    const uint8_t* flags;
    int64_t nnz;
    int meta_heads;
    int block;
    // workspace: V transposed per head, [BH][d][npad] bf16 (bf16 path only)
    void* vt;
    int npad;            // keys rounded up to 128 (the V^T row length)
    // key-range launches (Mode::kRange): the queries meet keys [s*kv_chunk,
    // min(Nk, (s+1)*kv_chunk)) of a key/value block for split s, at global
    // positions q_off + i and k_off + j, and write normalised fp32 partials
    int Nk;              // keys per head in k and v
    int64_t q_off;
    int64_t k_off;
    int kv_chunk;        // keys per split, a multiple of 64
    int nsplit;
    float* o_part;       // [nsplit][BH][N][d]
    float* lse_part;     // [nsplit][BH][N]
    int fold_slots;      // causal: grid of this many resident workgroups (0: one per query tile)
};

enum class Mode : int { kDense = 0, kCausal = 1, kSparse = 2, kRange = 3 };

// Grouped-query attention: the H / Hkv query heads h of one group share key/value
// head h / (H / Hkv).  Index of the key/value head of query head bh = b*H + h.
__host__ __device__ inline int64_t kv_head_of(int64_t bh, int H, int Hkv) {
    return (bh / H) * Hkv + (bh % H) / (H / Hkv);
}

// Block-sparse pattern used by query head bh: one pattern for every head
// (meta_heads 1), one per query head (H), one per key/value head (Hkv: the
// query heads of a group share their key-block list), or one per (batch,
// head) (B*H).
__host__ __device__ inline int64_t meta_of(int64_t bh, int H, int Hkv, int meta_heads) {
    if (meta_heads == 1) return 0;
    if (meta_heads == H) return bh % H;
    if (meta_heads == Hkv) return (bh % H) / (H / Hkv);
    return bh;
}

// Mean-pooled block selector: block means of Q and K into qm, km (fp32
// workspace), then the canonical per-(batch, head) CSR of the top-k key blocks
// of every query block.  select_nnz gives its entry count.
hipError_t launch_select(const void* q, const void* k, bool bf16, int64_t B, int H, int Hkv, int N, int d,
                         float scale, int causal, int block, int topk, int share, int32_t* row_ptr, int32_t* col,
                         uint8_t* flags, float* qm, float* km, hipStream_t stream);
int64_t select_nnz(int64_t BH, int64_t nb, int64_t topk, int causal);
int64_t select_max_blocks();
int64_t select_max_topk();

// Merge nsplit normalised partial states (o_part, lse_part as in FwdArgs)
// into O (bf16 when out_bf16, else fp32) and LSE.
hipError_t launch_merge(const float* o_part, const float* lse_part, int nsplit, int64_t BH, int N, int d,
                        void* o, float* lse, bool out_bf16, hipStream_t stream);

// Everything a backward launch needs (bf16 path); built and validated by the
// host layer.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;       // forward output
    const void* dout;    // upstream gradient dO
    const float* lse;    // forward LSE (natural log)
    void* dq;
    void* dk;
    void* dv;
    int64_t BH;
    int H;
    int Hkv;
    int N;
    int d;
    float scale;
    float scale_log2;
    int causal;
    // block-sparse schedule: key blocks per query block (dQ) and, transposed,
    // query blocks per key block (dK, dV)
    const int32_t* row_ptr;
    const int32_t* col;
    const uint8_t* flags;
    int64_t nnz;
    const int32_t* t_row_ptr;
    const int32_t* t_col;
    int64_t t_nnz;
    int meta_heads;
    int block;
    // workspace: per-row statistics ([BH][npad/64 + 1][2][64] fp32: LSE in
    // base-2 units, then D = dO . O, per 64-row block)
    float* stats;
    int npad;
    // block-sparse dK/dV: a key block whose query-tile list is long is split
    // into up to `pieces` pieces of workgroups; plan[kvbh * nkt + kt] = (first
    // partial slot, pieces) and the pieces' fp32 partial dK, dV go to
    // part[slot][2][BKV][d] for an ordered reduction.
    // extra[slot] = (key tile, piece) for every used slot ((-1, -1) past them).
    // The dK/dV launch has part_slots + (key tiles) workgroups: the first run
    // the pieces >= 1 named by extra (piece-0 entries are skipped), the rest
    // piece 0 of every key tile; the reduction's workgroups sit on the piece-0
    // entries, the first slot of each split key tile.
    int2* plan;
    int2* extra;
    float* part;
    int64_t part_slots;   // partial slots the workspace holds (no split beyond them)
};

// Bytes of backward workspace for BH query heads of N rows (dense, causal).
int64_t bwd_workspace_bytes(int64_t BH, int64_t N);
// The block-sparse backward's workspace: the row statistics and the split
// plan (the minimum), then, per partial dK/dV slot of BKV = block keys, its
// fp32 partials and its entry of the extra-piece list (plus 256 bytes of
// alignment once).
int64_t bwd_sparse_workspace_base(int64_t BH, int64_t BHkv, int64_t N, int64_t block);
int64_t bwd_sparse_slot_bytes(int64_t block, int64_t d);

// Partial slots the split plan uses for host transposed offsets t_row_ptr
// ([meta_heads * ceil(N / block) + 1]); 0 when they would exceed the cap of
// 2^18 slots a call uses (the call then splits nothing).
int64_t bwd_sparse_slots(const int32_t* t_row_ptr, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t block,
                         int64_t meta_heads);
// Point the BwdArgs at their workspace pieces (a.BH, a.N set; for the sparse
// backward also a.H, a.Hkv, a.d, a.block, a.meta_heads, and ws_bytes given).
void bwd_workspace_carve(BwdArgs& a, void* ws);
void bwd_sparse_workspace_carve(BwdArgs& a, void* ws, int64_t ws_bytes);
// Row statistics, then the dK/dV and dQ kernels, all on `stream`.
hipError_t launch_bwd_bf16(const BwdArgs& a, Mode mode, hipStream_t stream);

// Launchers: return hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, Mode mode, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, Mode mode, hipStream_t stream);
// Forward with 64 query rows per wave (d = 128, V read in place, N a multiple
// of 64 and at least 128): dense or causal.
hipError_t launch_fwd_w64(const FwdArgs& a, bool causal, hipStream_t stream);
// Fill a.vt from a.v (bf16 path): V^T with the key order the forward kernel reads.
hipError_t launch_v_transpose(const FwdArgs& a, hipStream_t stream);
// Keys per head of the V^T workspace: N rounded up to 128.
int64_t vt_padded_keys(int64_t N);

// Workgroup index -> (tile order index) so that consecutive tile indices land
// on the same XCD: the dispatcher hands workgroup i to XCD i % 8, so XCD x
// receives the contiguous range [x*T/8, (x+1)*T/8) of the tile order and the
// query tiles of one head share that XCD's L2 while they stream its K/V.
__device__ __forceinline__ int64_t xcd_tile_order(int64_t wg, int64_t total) {
    constexpr int kXcds = 8;
    const int64_t per = total / kXcds;
    if (wg >= per * kXcds) return wg;  // ragged tail keeps its own index
    return (wg % kXcds) * per + wg / kXcds;
}

// Item order for launches whose items differ in cost (causal, block-sparse):
// `total` items are `per_head` tiles of each of several heads.  Each XCD still
// gets a contiguous range of whole heads (xcd_tile_order), but inside it the
// items are dispatched rank-major, head-minor, so the costliest tiles of every
// head of the XCD start first instead of one head at a time.  Returns the head
// and the tile's rank within it; when the ranges do not hold whole heads the
// order is head-major.
__device__ __forceinline__ void rank_major_order(int64_t wg, int64_t total, int per_head, int64_t& head,
                                                 int& rank) {
    constexpr int kXcds = 8;
    const int64_t per = total / kXcds;
    if (wg < per * kXcds && per % per_head == 0) {
        const int64_t hx = per / per_head;   // heads per XCD
        const int64_t x = wg % kXcds, local = wg / kXcds;
        head = x * hx + local % hx;
        rank = (int)(local / hx);
    } else {
        const int64_t ord = xcd_tile_order(wg, total);
        head = ord / per_head;
        rank = (int)(ord % per_head);
    }
}

}  // namespace bsattn
