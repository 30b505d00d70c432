// Mean-pooled block selector on the device, for gfx950.
//
// Source: "Exact Blocks, Rings, and Sparsity", section 5, "Fixed pooling": a
// key block is summarised by the mean of its keys, and the mean logit of a
// query over the block is scale q . k_bar.  The block-sparse kernel's unit is
// a query tile, so a (query block a, key block b) pair is scored by the mean
// logit of the whole tile, scale q_bar_a . k_bar_b (linearity), and C_a is the
// top-k key blocks of that score (ties to the lower index; causal candidates
// kb <= a).  With grouped-query attention the group's query heads can share
// one choice: their scores are averaged (by averaging q_bar, the same thing
// by linearity) and every head of the group gets the same list, so the group
// loads one set of K/V blocks.
//
// Two kernels, both far off the attention's critical cost (section 5: the
// selector must cost less than the tiles it skips):
//   pool:   block means of Q and K in fp32, one read of each, in one launch
//           (HBM-bound);
//   select: per head, 8 query blocks per workgroup; each thread scores the
//           key blocks it owns against the 8 pooled queries (k_bar is read
//           once per 8 query blocks), then one wave per query block finds the
//           k-th largest score by a radix select over order-preserving 32-bit
//           keys (one bit per pass, counted with wave ballots, stopping once
//           the keys that share the fixed bits are exactly the ones still
//           needed), and writes the canonical CSR row (ascending, unique) with
//           its flags, straight into the metadata the block-sparse kernels
//           read.  Equal scores go to the lower block index.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsattn.h"
#include "fwd_common.h"
#include "gfx950_util.h"

namespace bsattn {
namespace {

constexpr int kRowsPerWg = 8;          // query blocks per select workgroup
constexpr int kMaxBlocks = 2048;       // key blocks per head the select kernel holds
constexpr int kMaxTopk = 64;

// Order-preserving map of a score to an unsigned key: a larger score gives a
// larger key, -0 is folded into +0 (so equal scores give equal keys) and NaN
// ranks with -inf.  Every score maps to at least 0x007fffff, so 0 is free to
// mark a slot that holds no candidate.
__device__ __forceinline__ uint32_t score_key(float s) {
    s = s != s ? -__builtin_inff() : s + 0.0f;
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
    return (float)x;
}

// out[h][blk][c] = mean over the rows of block blk of x[h][row][c], for Q's
// heads then K's in one flat grid (workgroup = (head, block)).  Each thread
// owns one 16-byte chunk of a row (E values) and adds it over every RG-th row
// of the block, four rows' loads in flight at a time; the RG partial sums per
// column are then added in row-group order (deterministic).
template <int D, typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   float* __restrict__ qm, float* __restrict__ km, int64_t BHq,
                                                   int N, int block, int nb) {
    constexpr int E = 16 / (int)sizeof(T);   // values per 16-byte chunk
    constexpr int CPR = D / E;               // chunks per row
    constexpr int RG = 256 / CPR;            // row groups
    static_assert(CPR * E == D && RG * CPR == 256, "chunking must cover the row");
    __shared__ float part[RG][D];
    const int blk = (int)(blockIdx.x % (unsigned)nb);
    int64_t h = blockIdx.x / (unsigned)nb;
    const T* x = q;
    float* out = qm;
    if (h >= BHq) {
        h -= BHq;
        x = k;
        out = km;
    }
    const int ch = threadIdx.x % CPR, rg = threadIdx.x / CPR;
    const int r0 = blk * block, r1 = min(N, r0 + block);
    const T* src = x + h * (int64_t)N * D + ch * E;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    int r = r0 + rg;
    for (; r + 3 * RG < r1; r += 4 * RG) {
        uint4 raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const uint4*>(src + (int64_t)(r + u * RG) * D);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const T* vals = reinterpret_cast<const T*>(&raw[u]);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += to_f32(vals[e]);
        }
    }
    for (; r < r1; r += RG) {
        const uint4 raw = *reinterpret_cast<const uint4*>(src + (int64_t)r * D);
        const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += to_f32(vals[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) part[rg][ch * E + e] = acc[e];
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256) {
        float sum = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) sum += part[g][c];
        out[(h * nb + blk) * (int64_t)D + c] = sum / (float)(r1 - r0);
    }
}

struct SelArgs {
    const float* qm;     // [BH][nb][D]
    const float* km;     // [B*Hkv][nb][D]
    int32_t* row_ptr;    // [BH*nb + 1]
    int32_t* col;
    uint8_t* flags;
    int64_t BH;
    int H, Hkv, N, block, nb, topk, causal, share;
    float scale;
};

// entries of rows 0..qb-1 of one head
__device__ __forceinline__ int64_t row_start(int qb, int topk, int nb, int causal) {
    if (!causal) return (int64_t)qb * min(topk, nb);
    if (qb <= topk) return (int64_t)qb * (qb + 1) / 2;
    return (int64_t)topk * (topk + 1) / 2 + (int64_t)(qb - topk) * topk;
}

// MB: the key blocks per head this instance holds (nb <= MB); the score
// buffer is sized by it, so the smaller instance fits more workgroups per CU.
template <int D, int MB>
__global__ __launch_bounds__(256) void select_kernel(SelArgs a) {
    __shared__ float qs[kRowsPerWg][D];
    __shared__ float sc[kRowsPerWg][MB];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nwg_h = (a.nb + kRowsPerWg - 1) / kRowsPerWg;
    // each XCD takes a contiguous range of heads, so one head's pooled keys
    // stay in one L2; inside it the workgroups with the most (causal)
    // candidates start first
    int64_t bh;
    int rank;
    rank_major_order(blockIdx.x, (int64_t)nwg_h * a.BH, nwg_h, bh, rank);
    const int qb0 = (nwg_h - 1 - rank) * kRowsPerWg;
    const int64_t kvh = kv_head_of(bh, a.H, a.Hkv);
    const int group = a.H / a.Hkv;

    // pooled queries of this workgroup's query blocks (the group mean when shared)
    for (int i = tid; i < kRowsPerWg * D; i += 256) {
        const int rr = i / D, c = i % D, qb = qb0 + rr;
        float v = 0.f;
        if (qb < a.nb) {
            if (a.share) {
                const int64_t h0 = (bh / a.H) * a.H + ((bh % a.H) / group) * group;
                for (int g = 0; g < group; ++g) v += a.qm[((h0 + g) * a.nb + qb) * (int64_t)D + c];
                v /= (float)group;
            } else {
                v = a.qm[(bh * a.nb + qb) * (int64_t)D + c];
            }
        }
        qs[rr][c] = v * a.scale;
    }
    __syncthreads();
    // scores of every candidate key block against the pooled queries
    const int last = min(a.nb, qb0 + kRowsPerWg) - 1;
    const int ncand_max = a.causal ? last + 1 : a.nb;
    for (int kb = tid; kb < ncand_max; kb += 256) {
        const float* kr = a.km + (kvh * a.nb + kb) * (int64_t)D;
        float s[kRowsPerWg];
#pragma unroll
        for (int rr = 0; rr < kRowsPerWg; ++rr) s[rr] = 0.f;
#pragma unroll 4
        for (int c = 0; c < D; c += 4) {
            const float4 kv = *reinterpret_cast<const float4*>(kr + c);
#pragma unroll
            for (int rr = 0; rr < kRowsPerWg; ++rr)
                s[rr] += qs[rr][c] * kv.x + qs[rr][c + 1] * kv.y + qs[rr][c + 2] * kv.z + qs[rr][c + 3] * kv.w;
        }
#pragma unroll
        for (int rr = 0; rr < kRowsPerWg; ++rr) sc[rr][kb] = s[rr];
    }
    __syncthreads();

    // top-k per query block: one wave per row, candidates kb = lane + 64 j
    constexpr int J = MB / 64;
    const int64_t per_head = row_start(a.nb, a.topk, a.nb, a.causal);
    const uint64_t below = (1ull << lane) - 1ull;   // lanes under this one
    for (int rr = w; rr < kRowsPerWg; rr += 4) {
        const int qb = qb0 + rr;
        if (qb >= a.nb) break;
        const int ncand = a.causal ? qb + 1 : a.nb;
        const int kk = min(a.topk, ncand);
        const int jn = (ncand + 63) >> 6;   // 64-candidate slices that hold candidates
        uint32_t key[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = lane + 64 * j;
            key[j] = (j < jn && c < ncand) ? score_key(sc[rr][c]) : 0u;
        }
        // Radix select of the kk-th largest key T, from the top bit down:
        // 'prefix' holds T's bits fixed so far (the bits in 'mask'), 'match'
        // counts the candidates whose masked key equals it, and 'need' how
        // many of those belong to the top kk (every candidate with a larger
        // masked key does).  Once match == need they all do and the rest of
        // T's bits do not matter.
        uint32_t prefix = 0u, mask = 0u;
        int need = kk, match = ncand;
        for (int bit = 31; bit >= 0 && match != need; --bit) {
            const uint32_t m2 = mask | (1u << bit), p2 = prefix | (1u << bit);
            int cnt = 0;   // candidates that match and have this bit set
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (j < jn) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64((key[j] & m2) == p2));
            if (cnt >= need) {
                prefix = p2;
                match = cnt;
            } else {
                need -= cnt;
                match -= cnt;
            }
            mask = m2;
        }
        // write the row in ascending order: ballot per 64-candidate slice
        const int64_t start = bh * per_head + row_start(qb, a.topk, a.nb, a.causal);
        const int r = (int)(bh * a.nb + qb);
        if (lane == 0) a.row_ptr[r] = (int32_t)start;
        if (lane == 0 && r == a.BH * a.nb - 1) a.row_ptr[r + 1] = (int32_t)(start + kk);
        int written = 0, eq_left = need;   // keys equal to the prefix still to take, lowest index first
        const bool partial = (a.N % a.block) != 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (j >= jn) continue;
            const uint32_t km = key[j] & mask;
            const bool valid = lane + 64 * j < ncand;
            const uint64_t em = __builtin_amdgcn_ballot_w64(valid && km == prefix);
            const bool f =
                valid && (km > prefix || (km == prefix && __builtin_popcountll(em & below) < eq_left));
            eq_left -= min(eq_left, __builtin_popcountll(em));
            const uint64_t m = __builtin_amdgcn_ballot_w64(f);
            if (f) {
                const int c = lane + 64 * j;
                const int pos = written + __builtin_popcountll(m & below);
                a.col[start + pos] = c;
                uint8_t fl = 0;
                if (a.causal && c == qb && a.block > 1) fl |= ATTN_FLAG_DIAGONAL;
                if (partial && c == a.nb - 1) fl |= ATTN_FLAG_PARTIAL;
                a.flags[start + pos] = fl;
            }
            written += __builtin_popcountll(m);
        }
    }
}

}  // namespace

int64_t select_nnz(int64_t BH, int64_t nb, int64_t topk, int causal) {
    int64_t per;
    if (!causal) per = nb * (topk < nb ? topk : nb);
    else if (nb <= topk) per = nb * (nb + 1) / 2;
    else per = topk * (topk + 1) / 2 + (nb - topk) * topk;
    return BH * per;
}

int64_t select_max_blocks() { return kMaxBlocks; }
int64_t select_max_topk() { return kMaxTopk; }

hipError_t launch_select(const void* q, const void* k, bool bf16, int64_t B, int H, int Hkv, int N, int d,
                         float scale, int causal, int block, int topk, int share, int32_t* row_ptr, int32_t* col,
                         uint8_t* flags, float* qm, float* km, hipStream_t stream) {
    const int nb = (N + block - 1) / block;
    const int64_t BHq = B * H;
    const dim3 gp((unsigned)(nb * (BHq + B * Hkv)));
    if (d == 64) {
        if (bf16)
            hipLaunchKernelGGL((pool_kernel<64, __bf16>), gp, dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k,
                               qm, km, BHq, N, block, nb);
        else
            hipLaunchKernelGGL((pool_kernel<64, float>), gp, dim3(256), 0, stream, (const float*)q, (const float*)k, qm,
                               km, BHq, N, block, nb);
    } else {
        if (bf16)
            hipLaunchKernelGGL((pool_kernel<128, __bf16>), gp, dim3(256), 0, stream, (const __bf16*)q,
                               (const __bf16*)k, qm, km, BHq, N, block, nb);
        else
            hipLaunchKernelGGL((pool_kernel<128, float>), gp, dim3(256), 0, stream, (const float*)q, (const float*)k,
                               qm, km, BHq, N, block, nb);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SelArgs s;
    s.qm = qm;
    s.km = km;
    s.row_ptr = row_ptr;
    s.col = col;
    s.flags = flags;
    s.BH = B * H;
    s.H = H;
    s.Hkv = Hkv;
    s.N = N;
    s.block = block;
    s.nb = nb;
    s.topk = topk;
    s.causal = causal;
    s.share = share;
    s.scale = scale;
    const int64_t grid = (int64_t)((nb + kRowsPerWg - 1) / kRowsPerWg) * B * H;
    const dim3 gs((unsigned)grid);
    if (nb <= kMaxBlocks / 2) {
        if (d == 64) hipLaunchKernelGGL((select_kernel<64, kMaxBlocks / 2>), gs, dim3(256), 0, stream, s);
        else hipLaunchKernelGGL((select_kernel<128, kMaxBlocks / 2>), gs, dim3(256), 0, stream, s);
    } else {
        if (d == 64) hipLaunchKernelGGL((select_kernel<64, kMaxBlocks>), gs, dim3(256), 0, stream, s);
        else hipLaunchKernelGGL((select_kernel<128, kMaxBlocks>), gs, dim3(256), 0, stream, s);
    }
    return hipGetLastError();
}

}  // namespace bsattn
