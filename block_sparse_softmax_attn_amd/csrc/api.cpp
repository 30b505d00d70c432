// C ABI of the attention forward: argument validation and kernel dispatch.
// Every check happens before any launch; nothing here allocates device memory.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "bsattn.h"
#include "fwd_common.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 30;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                 int64_t N, int64_t d, int dtype, float scale, int causal) {
    if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
    if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    if (N > kMaxN || H > INT32_MAX) return ATTN_EINVAL;
    // element count and grid size must fit the kernels' 64-bit offsets and 32-bit grid
    if (B > (int64_t(1) << 62) / H) return ATTN_EINVAL;
    const int64_t bh = B * H;
    if (bh > (int64_t(1) << 62) / (N * d)) return ATTN_EINVAL;
    const int64_t tiles = ((N + 63) / 64) * bh;
    if (tiles > INT32_MAX) return ATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_EINVAL;
    return ATTN_OK;
}

bsattn::FwdArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                          int64_t H, int64_t N, int64_t d, float scale, int causal) {
    bsattn::FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.BH = B * H;
    a.H = static_cast<int>(H);
    a.Hkv = static_cast<int>(H);
    a.N = static_cast<int>(N);
    a.d = static_cast<int>(d);
    a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    a.causal = causal;
    return a;
}

bool valid_groups(int64_t H, int64_t Hkv) { return Hkv >= 1 && Hkv <= H && H % Hkv == 0; }

// V^T of B*H heads, as attn_prepare_v writes it
int64_t vt_bytes(int64_t B, int64_t H, int64_t N, int64_t d) { return B * H * d * bsattn::vt_padded_keys(N) * 2; }

int check_vt(const void* vt, int64_t given, int64_t B, int64_t H, int64_t N, int64_t d) {
    if (given < vt_bytes(B, H, N, d)) return ATTN_ECAPACITY;
    if (!vt || !aligned16(vt)) return ATTN_EINVAL;
    return ATTN_OK;
}

// One launch of the fused kernel on `stream`.  bf16 reads V in place, or V^T
// when the caller prepared it (vt != nullptr).
int run(bsattn::FwdArgs& a, int dtype, bsattn::Mode mode, const void* vt, hipStream_t stream) {
    hipError_t e = hipSuccess;
    if (dtype == ATTN_BF16) {
        a.vt = const_cast<void*>(vt);   // read only by the forward kernel
        a.npad = static_cast<int>(bsattn::vt_padded_keys(a.N));
        e = bsattn::launch_fwd_bf16(a, mode, stream);
    } else {
        e = bsattn::launch_fwd_f32(a, mode, stream);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

// v == nullptr: the prepared form, V^T in vt (vt_given bytes)
int fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Hkv,
              int64_t N, int64_t d, int dtype, float scale, int causal, const void* vt, int64_t vt_given,
              hipStream_t stream) {
    const bool prepared = v == nullptr;
    int st = check_common(q, k, prepared ? q : v, o, lse, B, H, N, d, dtype, scale, causal);
    if (st != ATTN_OK) return st;
    if (!valid_groups(H, Hkv)) return ATTN_EINVAL;
    if (prepared) {
        st = check_vt(vt, vt_given, B, Hkv, N, d);
        if (st != ATTN_OK) return st;
    }
    bsattn::FwdArgs a = make_args(q, k, v, o, lse, B, H, N, d, scale, causal);
    a.Hkv = static_cast<int>(Hkv);
    return run(a, dtype, causal ? bsattn::Mode::kCausal : bsattn::Mode::kDense, prepared ? vt : nullptr, stream);
}

int fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
               int64_t Hkv, int64_t N, int64_t d, int dtype, float scale, int causal, int64_t block,
               const int32_t* row_ptr, const int32_t* col, const uint8_t* flags, int64_t nnz, int64_t meta_heads,
               const void* vt, int64_t vt_given, hipStream_t stream) {
    // v == nullptr: the prepared form, V^T in vt (written by attn_prepare_v)
    const bool prepared = v == nullptr;
    int st = check_common(q, k, prepared ? q : v, o, lse, B, H, N, d, dtype, scale, causal);
    if (st != ATTN_OK) return st;
    if (block != 64 && block != 128) return ATTN_EUNSUPPORTED;
    if (!valid_groups(H, Hkv)) return ATTN_EINVAL;
    if (meta_heads != 1 && meta_heads != H && meta_heads != Hkv && meta_heads != B * H) return ATTN_EINVAL;
    if (!row_ptr || nnz < 0 || nnz > INT32_MAX) return ATTN_EINVAL;
    if (nnz > 0 && (!col || !flags)) return ATTN_EINVAL;
    if (prepared) {
        st = check_vt(vt, vt_given, B, Hkv, N, d);
        if (st != ATTN_OK) return st;
    }
    bsattn::FwdArgs a = make_args(q, k, v, o, lse, B, H, N, d, scale, causal);
    a.Hkv = static_cast<int>(Hkv);
    a.row_ptr = row_ptr;
    a.col = col;
    a.flags = flags;
    a.nnz = nnz;
    a.meta_heads = static_cast<int>(meta_heads);
    a.block = static_cast<int>(block);
    return run(a, dtype, bsattn::Mode::kSparse, prepared ? vt : nullptr, stream);
}

}  // namespace

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_EUNSUPPORTED: return "unsupported configuration";
        case ATTN_ECAPACITY: return "output capacity too small";
        case ATTN_EHIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

extern "C" int64_t attn_prepared_v_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || (d != 64 && d != 128) || dtype != ATTN_BF16) return -1;
    if (B > (int64_t(1) << 62) / H || B * H > (int64_t(1) << 62) / (2 * d * bsattn::vt_padded_keys(N))) return -1;
    return vt_bytes(B, H, N, d);
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                        int64_t N, int64_t d, int dtype, float scale, int causal, hipStream_t stream) {
    if (!v) return ATTN_EINVAL;
    return fwd_dense(q, k, v, o, lse, B, H, H, N, d, dtype, scale, causal, nullptr, 0, stream);
}

extern "C" int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                    int64_t H, int64_t N, int64_t d, int dtype, float scale, int causal,
                                    int64_t block, const int32_t* row_ptr, const int32_t* col,
                                    const uint8_t* flags, int64_t nnz, int64_t meta_heads, hipStream_t stream) {
    if (!v) return ATTN_EINVAL;
    return fwd_sparse(q, k, v, o, lse, B, H, H, N, d, dtype, scale, causal, block, row_ptr, col, flags, nnz,
                      meta_heads, nullptr, 0, stream);
}

extern "C" int attn_prepare_v(const void* v, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, void* vt,
                              int64_t vt_bytes_given, hipStream_t stream) {
    if (!v) return ATTN_EINVAL;
    if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    const int64_t need = attn_prepared_v_bytes(B, H, N, d, dtype);
    if (need < 0) return (d != 64 && d != 128) ? ATTN_EUNSUPPORTED : ATTN_EINVAL;
    if (!aligned16(v)) return ATTN_EINVAL;
    if (B * H > 65535) return ATTN_EUNSUPPORTED;   // the transpose launch puts the heads on the grid's rows
    const int st = check_vt(vt, vt_bytes_given, B, H, N, d);
    if (st != ATTN_OK) return st;
    bsattn::FwdArgs a{};
    a.v = v;
    a.vt = vt;
    a.BH = B * H;
    a.N = static_cast<int>(N);
    a.d = static_cast<int>(d);
    a.npad = static_cast<int>(bsattn::vt_padded_keys(N));
    return bsattn::launch_v_transpose(a, stream) == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" int attn_fwd_prepared(const void* q, const void* k, void* o, float* lse, int64_t B, int64_t H, int64_t N,
                                 int64_t d, int dtype, float scale, int causal, const void* vt,
                                 int64_t vt_bytes_given, hipStream_t stream) {
    if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    return fwd_dense(q, k, nullptr, o, lse, B, H, H, N, d, dtype, scale, causal, vt, vt_bytes_given, stream);
}

extern "C" int attn_fwd_blocksparse_prepared(const void* q, const void* k, void* o, float* lse, int64_t B, int64_t H,
                                             int64_t N, int64_t d, int dtype, float scale, int causal, int64_t block,
                                             const int32_t* row_ptr, const int32_t* col, const uint8_t* flags,
                                             int64_t nnz, int64_t meta_heads, const void* vt,
                                             int64_t vt_bytes_given, hipStream_t stream) {
    if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    return fwd_sparse(q, k, nullptr, o, lse, B, H, H, N, d, dtype, scale, causal, block, row_ptr, col, flags, nnz,
                      meta_heads, vt, vt_bytes_given, stream);
}

// ---------------------------------------------------------------------------
// backward (bf16)
// ---------------------------------------------------------------------------

namespace {

int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype,
              float scale, int causal, void* ws, int64_t ws_bytes, int64_t block = 0) {
    int st = check_common(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), B, H, N, d, dtype, scale, causal);
    if (st != ATTN_OK) return st;
    if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    if (!valid_groups(H, Hkv)) return ATTN_EINVAL;
    if (!dout || !dq || !dk || !dv) return ATTN_EINVAL;
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return ATTN_EINVAL;
    const int64_t need = block ? bsattn::bwd_sparse_workspace_base(B * H, B * Hkv, N, block)
                               : bsattn::bwd_workspace_bytes(B * H, N);
    if (ws_bytes < need) return ATTN_ECAPACITY;
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return ATTN_EINVAL;
    return ATTN_OK;
}

bsattn::BwdArgs make_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv,
                              int64_t N, int64_t d, float scale, int causal, void* ws) {
    bsattn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.BH = B * H;
    a.H = static_cast<int>(H);
    a.Hkv = static_cast<int>(Hkv);
    a.N = static_cast<int>(N);
    a.d = static_cast<int>(d);
    a.scale = scale;
    a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    a.causal = causal;
    bsattn::bwd_workspace_carve(a, ws);
    return a;
}

}  // namespace

namespace {

int64_t bwd_ws(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || (d != 64 && d != 128) || dtype != ATTN_BF16) return -1;
    if (!valid_groups(H, Hkv)) return -1;
    if (B > (int64_t(1) << 62) / H || B * H > (int64_t(1) << 58) / (8 * d * bsattn::vt_padded_keys(N))) return -1;
    return bsattn::bwd_workspace_bytes(B * H, N);
}

int bwd_dense(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype,
              float scale, int causal, void* workspace, int64_t ws_bytes, hipStream_t stream) {
    const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, dtype, scale, causal, workspace,
                             ws_bytes);
    if (st != ATTN_OK) return st;
    bsattn::BwdArgs a = make_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace);
    const hipError_t e =
        bsattn::launch_bwd_bf16(a, causal ? bsattn::Mode::kCausal : bsattn::Mode::kDense, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

int bwd_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype,
               float scale, int causal, int64_t block, const int32_t* row_ptr, const int32_t* col,
               const uint8_t* flags, int64_t nnz, const int32_t* t_row_ptr, const int32_t* t_col,
               int64_t meta_heads, void* workspace, int64_t ws_bytes, hipStream_t stream) {
    if (block != 64 && block != 128) {
        const int st0 = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, dtype, scale, causal,
                                  workspace, ws_bytes);
        return st0 != ATTN_OK ? st0 : ATTN_EUNSUPPORTED;
    }
    int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, dtype, scale, causal, workspace,
                       ws_bytes, block);
    if (st != ATTN_OK) return st;
    if (meta_heads != 1 && meta_heads != H && meta_heads != Hkv && meta_heads != B * H) return ATTN_EINVAL;
    if (!row_ptr || !t_row_ptr || nnz < 0 || nnz > INT32_MAX) return ATTN_EINVAL;
    if (nnz > 0 && (!col || !flags || !t_col)) return ATTN_EINVAL;
    bsattn::BwdArgs a = make_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace);
    a.row_ptr = row_ptr;
    a.col = col;
    a.flags = flags;
    a.nnz = nnz;
    a.t_row_ptr = t_row_ptr;
    a.t_col = t_col;
    a.t_nnz = nnz;
    a.meta_heads = static_cast<int>(meta_heads);
    a.block = static_cast<int>(block);
    bsattn::bwd_sparse_workspace_carve(a, workspace, ws_bytes);
    const hipError_t e = bsattn::launch_bwd_bf16(a, bsattn::Mode::kSparse, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // namespace

extern "C" int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
    return bwd_ws(B, H, H, N, d, dtype);
}

extern "C" int64_t attn_bwd_blocksparse_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                                        int dtype, int64_t block, const int32_t* t_row_ptr,
                                                        int64_t meta_heads) {
    if (bwd_ws(B, H, Hkv, N, d, dtype) < 0 || (block != 64 && block != 128)) return -1;
    if (meta_heads != 1 && meta_heads != H && meta_heads != Hkv && meta_heads != B * H) return -1;
    const int64_t base = bsattn::bwd_sparse_workspace_base(B * H, B * Hkv, N, block);
    if (!t_row_ptr) return base;
    const int64_t slots = bsattn::bwd_sparse_slots(t_row_ptr, B, H, Hkv, N, block, meta_heads);
    if (slots == 0) return base;
    const int64_t per_slot = bsattn::bwd_sparse_slot_bytes(block, d) + 8;   // partials + extra-list entry
    if (slots > (int64_t(1) << 40) / per_slot) return -1;
    return base + 256 + slots * per_slot;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                        int dtype, float scale, int causal, void* workspace, int64_t workspace_bytes_given,
                        hipStream_t stream) {
    return bwd_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, d, dtype, scale, causal, workspace,
                     workspace_bytes_given, stream);
}

// ---- the backward without a caller workspace ----
//
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): attn_bwd_noalloc keeps the row
// statistics in a fixed array of the library's code object instead of a
// caller workspace.  Every GPU the library runs on holds its own copy of the
// array until the process ends; its device address is looked up once per
// device and kept.  In host code the array's name is only a host-side stand-in
// for the symbol, never a device address: host code uses scratch_base().
namespace {

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on error).
void* scratch_base() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                                int64_t d, int dtype, float scale, int causal, hipStream_t stream) {
    // every argument check of attn_bwd, with the scratch standing in for the
    // workspace; sizes whose statistics exceed it are refused before any HIP call
    const int64_t need = bwd_ws(B, H, H, N, d, dtype);
    if (need > ATTN_NOALLOC_SCRATCH_BYTES) {
        const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, d, dtype, scale, causal,
                                 reinterpret_cast<void*>(uintptr_t(256)), need);
        return st != ATTN_OK ? st : ATTN_ECAPACITY;
    }
    const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, d, dtype, scale, causal,
                             reinterpret_cast<void*>(uintptr_t(256)), ATTN_NOALLOC_SCRATCH_BYTES);
    if (st != ATTN_OK) return st;
    void* ws = scratch_base();
    if (ws == nullptr) return ATTN_EHIP;
    return bwd_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, d, dtype, scale, causal, ws,
                     ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                    const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                                    int64_t N, int64_t d, int dtype, float scale, int causal, int64_t block,
                                    const int32_t* row_ptr, const int32_t* col, const uint8_t* flags, int64_t nnz,
                                    const int32_t* t_row_ptr, const int32_t* t_col, int64_t meta_heads,
                                    void* workspace, int64_t workspace_bytes_given, hipStream_t stream) {
    return bwd_sparse(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, d, dtype, scale, causal, block, row_ptr, col,
                      flags, nnz, t_row_ptr, t_col, meta_heads, workspace, workspace_bytes_given, stream);
}

// ---------------------------------------------------------------------------
// grouped-query attention: Hkv key/value heads shared by H query heads
// ---------------------------------------------------------------------------

extern "C" int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                            int64_t Hkv, int64_t N, int64_t d, int dtype, float scale, int causal,
                            hipStream_t stream) {
    if (!v) return ATTN_EINVAL;
    return fwd_dense(q, k, v, o, lse, B, H, Hkv, N, d, dtype, scale, causal, nullptr, 0, stream);
}

extern "C" int attn_fwd_blocksparse_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                        int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype, float scale,
                                        int causal, int64_t block, const int32_t* row_ptr, const int32_t* col,
                                        const uint8_t* flags, int64_t nnz, int64_t meta_heads, hipStream_t stream) {
    if (!v) return ATTN_EINVAL;
    return fwd_sparse(q, k, v, o, lse, B, H, Hkv, N, d, dtype, scale, causal, block, row_ptr, col, flags, nnz,
                      meta_heads, nullptr, 0, stream);
}

extern "C" int64_t attn_bwd_gqa_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                                int dtype) {
    return bwd_ws(B, H, Hkv, N, d, dtype);
}

extern "C" int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Hkv,
                            int64_t N, int64_t d, int dtype, float scale, int causal, void* workspace,
                            int64_t workspace_bytes_given, hipStream_t stream) {
    return bwd_dense(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, dtype, scale, causal, workspace,
                     workspace_bytes_given, stream);
}

extern "C" int attn_bwd_blocksparse_gqa(const void* q, const void* k, const void* v, const void* o,
                                        const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t B,
                                        int64_t H, int64_t Hkv, int64_t N, int64_t d, int dtype, float scale,
                                        int causal, int64_t block, const int32_t* row_ptr, const int32_t* col,
                                        const uint8_t* flags, int64_t nnz, const int32_t* t_row_ptr,
                                        const int32_t* t_col, int64_t meta_heads, void* workspace,
                                        int64_t workspace_bytes_given, hipStream_t stream) {
    return bwd_sparse(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, dtype, scale, causal, block, row_ptr, col,
                      flags, nnz, t_row_ptr, t_col, meta_heads, workspace, workspace_bytes_given, stream);
}

// ---------------------------------------------------------------------------
// key splits and ring steps (bf16): partial states and their merge
// ---------------------------------------------------------------------------

namespace {

constexpr int64_t kMaxSplits = 64;

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// keys per split: whole 64-key tiles, spread as evenly as the tiles allow
int64_t split_chunk(int64_t N, int64_t splits) {
    const int64_t tiles = (N + 63) / 64;
    return (tiles + splits - 1) / splits * 64;
}

int64_t partial_bytes(int64_t BH, int64_t N, int64_t d, int64_t splits) {
    return align256(splits * BH * N * d * 4) + align256(splits * BH * N * 4);
}

}  // namespace

extern "C" int64_t attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                                                    int64_t num_splits) {
    if (dtype != ATTN_BF16 || num_splits < 1 || num_splits > kMaxSplits) return -1;
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || (d != 64 && d != 128)) return -1;
    if (B > (int64_t(1) << 40) / H || B * H > (int64_t(1) << 56) / (N * (d + 1) * 4 * num_splits)) return -1;
    const int64_t splits = (N + split_chunk(N, num_splits) - 1) / split_chunk(N, num_splits);
    return partial_bytes(B * H, N, d, splits);
}

extern "C" int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t H, int64_t N, int64_t d, int dtype, float scale, int causal,
                                int64_t num_splits, void* workspace, int64_t workspace_bytes_given,
                                hipStream_t stream) {
    int st = check_common(q, k, v, o, lse, B, H, N, d, dtype, scale, causal);
    if (st != ATTN_OK) return st;
    if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    if (num_splits < 1 || num_splits > kMaxSplits) return ATTN_EINVAL;
    const int64_t need = attn_fwd_splitkv_workspace_bytes(B, H, N, d, dtype, num_splits);
    if (need < 0) return ATTN_EINVAL;
    if (workspace_bytes_given < need) return ATTN_ECAPACITY;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_EINVAL;
    const int64_t chunk = split_chunk(N, num_splits);
    const int64_t splits = (N + chunk - 1) / chunk;
    bsattn::FwdArgs a = make_args(q, k, v, o, lse, B, H, N, d, scale, causal);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    a.vt = nullptr;   // V read in place
    a.Nk = static_cast<int>(N);
    a.kv_chunk = static_cast<int>(chunk);
    a.nsplit = static_cast<int>(splits);
    a.o_part = reinterpret_cast<float*>(ws);
    a.lse_part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(a.o_part) + align256(splits * B * H * N * d * 4));
    if ((int64_t)((N + 255) / 256) * B * H * splits > INT32_MAX) return ATTN_EINVAL;
    hipError_t e = bsattn::launch_fwd_bf16(a, bsattn::Mode::kRange, stream);
    if (e == hipSuccess)
        e = bsattn::launch_merge(a.o_part, a.lse_part, a.nsplit, a.BH, a.N, a.d, o, lse, true, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" int attn_fwd_block(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype, float scale,
                              int causal, int64_t q_offset, int64_t k_offset, hipStream_t stream) {
    // shapes: Q [B,H,Nq,d]; K, V [B,H,Nk,d]; both sides pass the common checks
    int st = check_common(q, k, v, o_part, lse_part, B, H, Nq, d, dtype, scale, causal);
    if (st != ATTN_OK) return st;
    st = check_common(q, k, v, o_part, lse_part, B, H, Nk, d, dtype, scale, causal);
    if (st != ATTN_OK) return st;
    if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    if (q_offset < 0 || k_offset < 0 || q_offset > (int64_t(1) << 40) || k_offset > (int64_t(1) << 40))
        return ATTN_EINVAL;
    bsattn::FwdArgs a = make_args(q, k, v, o_part, lse_part, B, H, Nq, d, scale, causal);
    a.vt = nullptr;   // V read in place
    a.Nk = static_cast<int>(Nk);
    a.q_off = q_offset;
    a.k_off = k_offset;
    a.kv_chunk = static_cast<int>(bsattn::vt_padded_keys(Nk));   // one split covers every key
    a.nsplit = 1;
    a.o_part = o_part;
    a.lse_part = lse_part;
    const hipError_t e = bsattn::launch_fwd_bf16(a, bsattn::Mode::kRange, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" int attn_merge(const float* o_parts, const float* lse_parts, int64_t num_parts, int64_t B, int64_t H,
                          int64_t N, int64_t d, void* o, float* lse, int out_dtype, hipStream_t stream) {
    if (!o_parts || !lse_parts || !o || !lse) return ATTN_EINVAL;
    if (num_parts < 1 || num_parts > 1024 || B < 1 || H < 1 || N < 1 || N > kMaxN) return ATTN_EINVAL;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    if (B > (int64_t(1) << 40) / H || B * H * N > (int64_t(1) << 40) / (num_parts * d)) return ATTN_EINVAL;
    if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return ATTN_EINVAL;
    if ((B * H * N + 7) / 8 > INT32_MAX) return ATTN_EINVAL;
    const hipError_t e = bsattn::launch_merge(o_parts, lse_parts, static_cast<int>(num_parts), B * H,
                                              static_cast<int>(N), static_cast<int>(d), o, lse,
                                              out_dtype == ATTN_BF16, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

// ---------------------------------------------------------------------------
// mean-pooled block selector
// ---------------------------------------------------------------------------

extern "C" int64_t attn_select_meanpool_nnz(int64_t B, int64_t H, int64_t N, int64_t block, int causal,
                                            int64_t topk) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || (block != 64 && block != 128) || (causal != 0 && causal != 1))
        return -1;
    if (topk < 1 || topk > bsattn::select_max_topk()) return -1;
    const int64_t nb = (N + block - 1) / block;
    if (nb > bsattn::select_max_blocks() || B > (int64_t(1) << 40) / H) return -1;
    const int64_t n = bsattn::select_nnz(B * H, nb, topk, causal);
    return n > INT32_MAX ? -1 : n;
}

extern "C" int64_t attn_select_meanpool_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                                                        int64_t block) {
    if (B < 1 || H < 1 || N < 1 || N > kMaxN || (d != 64 && d != 128) || (block != 64 && block != 128)) return -1;
    if (!valid_groups(H, Hkv) || B > (int64_t(1) << 40) / H) return -1;
    const int64_t nb = (N + block - 1) / block;
    return (B * H + B * Hkv) * nb * d * 4;
}

extern "C" int attn_select_meanpool(const void* q, const void* k, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                    int64_t d, int dtype, float scale, int causal, int64_t block, int64_t topk,
                                    int share_groups, int32_t* row_ptr, int32_t* col, uint8_t* flags,
                                    int64_t capacity, void* workspace, int64_t workspace_bytes_given,
                                    hipStream_t stream) {
    if (!q || !k || !row_ptr || !col || !flags || !workspace) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    if (block != 64 && block != 128) return ATTN_EUNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_EINVAL;
    if (share_groups != 0 && share_groups != 1) return ATTN_EINVAL;
    if (topk < 1 || B < 1 || H < 1 || N < 1 || N > kMaxN || (causal != 0 && causal != 1)) return ATTN_EINVAL;
    if (topk > bsattn::select_max_topk() || (N + block - 1) / block > bsattn::select_max_blocks())
        return ATTN_EUNSUPPORTED;
    const int64_t nnz = attn_select_meanpool_nnz(B, H, N, block, causal, topk);
    if (nnz < 0) return ATTN_EINVAL;
    const int64_t need = attn_select_meanpool_workspace_bytes(B, H, Hkv, N, d, block);
    if (need < 0) return ATTN_EINVAL;
    if (capacity < nnz || workspace_bytes_given < need) return ATTN_ECAPACITY;
    if (!aligned16(q) || !aligned16(k) || !aligned16(workspace)) return ATTN_EINVAL;
    if (B * H * N > (int64_t(1) << 40) / d) return ATTN_EINVAL;
    const int64_t nb = (N + block - 1) / block;
    // one 256-thread workgroup per (head of Q or K, block) in a flat grid: keep
    // the grid's work-items under 2^32
    if (nb * B * (H + Hkv) >= (int64_t(1) << 24)) return ATTN_EUNSUPPORTED;
    float* qm = static_cast<float*>(workspace);
    float* km = qm + B * H * nb * d;
    const hipError_t e = bsattn::launch_select(q, k, dtype == ATTN_BF16, B, static_cast<int>(H),
                                               static_cast<int>(Hkv), static_cast<int>(N), static_cast<int>(d),
                                               scale, causal, static_cast<int>(block), static_cast<int>(topk),
                                               share_groups, row_ptr, col, flags, qm, km, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}
