// Merge of normalised partial attention states over disjoint key sets, for
// gfx950.
//
// Each partial s holds, per query row, the output O_s normalised over its own
// keys and LSE_s (natural log; -inf when the row saw none of them).  The merge
// is the online-softmax state merge in (O, LSE) form ("Exact Blocks, Rings, and
// Sparsity", section 2 merge invariant, section 4 associative ring merge):
//     LSE = m + ln sum_s exp(LSE_s - m),   m = max_s LSE_s
//     O   = sum_s exp(LSE_s - LSE) O_s
// with O = 0 and LSE = -inf when every part is empty.  Memory-bound: each row
// reads S * (d + 1) floats and writes d outputs plus one LSE.
//
// Layout: parts [S][BH][N][d] fp32 and [S][BH][N] fp32; outputs [BH][N][d]
// (bf16 or fp32) and [BH][N].  One row per d/4 consecutive lanes (one float4
// each), so a row never spans two waves: every lane of a row reads all of
// the row's partial LSEs before any lane of that wave writes, which makes an
// in-place merge into part 0 (fp32 output) safe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"
#include "gfx950_util.h"

namespace bsattn {
namespace {

// o and lse may be exactly part 0 of o_part and lse_part (an in-place merge),
// so the part pointers are not declared __restrict__.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_kernel(const float* o_part,
                                                    const float* lse_part, int nsplit, int64_t rows,
                                                    void* o, float* lse) {
    constexpr int TPR = D / 4;                    // lanes per row
    constexpr int RPB = 256 / TPR;                // rows per workgroup
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = (threadIdx.x % TPR) * 4;
    if (row >= rows) return;
    // one pass with a running max (the partial states are folded in split
    // order, each rescaled to the new max), unrolled so that several splits'
    // loads are in flight at once; empty states (LSE = -inf) are skipped
    float m = -__builtin_inff();
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) {
        const float ls = lse_part[(int64_t)s * rows + row];
        const float4 x = *reinterpret_cast<const float4*>(o_part + ((int64_t)s * rows + row) * D + c);
        if (ls > -__builtin_inff()) {
            const float mn = fmaxf(m, ls);
            const float keep = expf(m - mn);   // 0 while nothing is folded in yet
            const float wgt = expf(ls - mn);
            acc.x = acc.x * keep + wgt * x.x;
            acc.y = acc.y * keep + wgt * x.y;
            acc.z = acc.z * keep + wgt * x.z;
            acc.w = acc.w * keep + wgt * x.w;
            tot = tot * keep + wgt;
            m = mn;
        }
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
    if (OUT_BF16) {
        bf16x4 ov;
        ov[0] = (__bf16)(acc.x * inv);
        ov[1] = (__bf16)(acc.y * inv);
        ov[2] = (__bf16)(acc.z * inv);
        ov[3] = (__bf16)(acc.w * inv);
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(o) + row * D + c) = ov;
    } else {
        const float4 ov = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
        *reinterpret_cast<float4*>(static_cast<float*>(o) + row * D + c) = ov;
    }
    if (c == 0) lse[row] = tot > 0.f ? m + logf(tot) : -__builtin_inff();
}

template <int D>
hipError_t launch_d(const float* o_part, const float* lse_part, int nsplit, int64_t rows, void* o, float* lse,
                    bool out_bf16, hipStream_t stream) {
    constexpr int RPB = 256 / (D / 4);
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    if (out_bf16)
        hipLaunchKernelGGL((merge_kernel<D, true>), grid, dim3(256), 0, stream, o_part, lse_part, nsplit, rows, o, lse);
    else
        hipLaunchKernelGGL((merge_kernel<D, false>), grid, dim3(256), 0, stream, o_part, lse_part, nsplit, rows, o, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const float* o_part, const float* lse_part, int nsplit, int64_t BH, int N, int d, void* o,
                        float* lse, bool out_bf16, hipStream_t stream) {
    const int64_t rows = BH * N;
    if (d == 64) return launch_d<64>(o_part, lse_part, nsplit, rows, o, lse, out_bf16, stream);
    return launch_d<128>(o_part, lse_part, nsplit, rows, o, lse, out_bf16, stream);
}

}  // namespace bsattn
