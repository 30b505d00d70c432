// Fused attention forward, fp32 inputs and fp32 arithmetic throughout, for gfx950.
//
// Same schedule as the bf16 kernel ("Exact Blocks, Rings, and Sparsity",
// section 2; FlashAttention notes, section 5.2: query tile on chip, K/V tiles
// streamed, online softmax state, S and P never written out), with the fp32
// matrix core instruction v_mfma_f32_32x32x2_f32 for both contractions so no
// operand is rounded below fp32: P stays fp32 (rounding P to the input dtype
// is then a no-op).  This path serves fp32 inputs and is not tuned for speed.
//
//   * 4 waves x 32 query rows; S^T = K Q^T so a lane holds scores of one query
//     row; row max / sum need one exchange with lane l^32.
//   * O^T += V^T P^T in k-steps of 2 keys: the key of step (c, v) held by lane
//     half h is 32c + 8(v>>2) + 4h + (v&3), exactly the S^T register the lane
//     already owns, so P feeds the product without any data movement.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"

namespace bsattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 32;          // keys per tile step
constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int BM = 32 * NW;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float xor32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int MODE>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdArgs a) {
    constexpr int KS = D + 1;   // odd stride: lanes reading one column of 32 rows hit 32 banks
    constexpr int VS = D + 4;
    __shared__ float sK[BN * KS];
    __shared__ float sV[BN * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int N = a.N;
    const int bm = (MODE == (int)Mode::kSparse) ? a.block : BM;   // query rows per workgroup
    const int nqt = (N + bm - 1) / bm;
    const int64_t total = (int64_t)nqt * a.BH;
    const int64_t ord = xcd_tile_order(blockIdx.x, total);
    const int64_t bh = ord / nqt;
    int qt = (int)(ord % nqt);
    if (MODE != (int)Mode::kDense) qt = nqt - 1 - qt;
    const int q0 = qt * bm;
    const int q0w = q0 + 32 * w;
    const bool wave_rows_live = 32 * w < bm;   // block 64 uses 2 of the 4 waves

    const float* Qh = static_cast<const float*>(a.q) + bh * (int64_t)N * D;
    const int64_t kvh = kv_head_of(bh, a.H, a.Hkv);
    const float* Kh = static_cast<const float*>(a.k) + kvh * (int64_t)N * D;
    const float* Vh = static_cast<const float*>(a.v) + kvh * (int64_t)N * D;

    int ntiles = 0, e0 = 0, subs = 1, nqb_meta = 0;
    if (MODE == (int)Mode::kDense) {
        ntiles = (N + BN - 1) / BN;
    } else if (MODE == (int)Mode::kCausal) {
        ntiles = (min(N, q0 + bm) + BN - 1) / BN;
    } else {
        subs = a.block / BN;
        nqb_meta = (N + a.block - 1) / a.block;
        const int64_t r = meta_of(bh, a.H, a.Hkv, a.meta_heads) * nqb_meta + qt;
        int lo = a.row_ptr[r], hi_ = a.row_ptr[r + 1];
        lo = (int)min<int64_t>(max(lo, 0), a.nnz);
        hi_ = (int)min<int64_t>(max(hi_, lo), a.nnz);
        e0 = lo;
        ntiles = (hi_ - lo) * subs;
    }

    // Q fragments: B operand of S^T = K Q^T, lane holds Q[q0w + l32][2s + hi].
    float qf[D / 2];
    {
        const int qrow = min(q0w + l32, N - 1);
#pragma unroll
        for (int s = 0; s < D / 2; ++s) qf[s] = Qh[(int64_t)qrow * D + 2 * s + hi];
    }
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -__builtin_inff();
    float ell = 0.f;
    const float sl2 = a.scale_log2;
    const int qi = q0w + l32;

    for (int it = 0; it < ntiles; ++it) {
        int kb0, cmask, skip;
        if (MODE == (int)Mode::kSparse) {
            const int e = e0 + it / subs;
            const int kb = a.col[e];
            const bool valid = kb >= 0 && kb < nqb_meta;
            kb0 = valid ? kb * a.block + (it % subs) * BN : 0;
            cmask = ((a.flags[e] & 1) != 0) || (a.causal && kb0 + BN - 1 > q0);
            skip = !valid || kb0 >= N;
        } else {
            kb0 = it * BN;
            cmask = (MODE == (int)Mode::kCausal) && (kb0 + BN - 1 > q0);
            skip = 0;
        }
        __syncthreads();   // previous tile's readers are done
        for (int c = tid; c < BN * D / 4; c += NT) {
            const int row = c / (D / 4), ch = c % (D / 4);
            const int key = min(kb0 + row, N - 1);
            const f32x4 kv = *reinterpret_cast<const f32x4*>(Kh + (int64_t)key * D + 4 * ch);
            const f32x4 vv = *reinterpret_cast<const f32x4*>(Vh + (int64_t)key * D + 4 * ch);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sK[row * KS + 4 * ch + i] = kv[i];
                sV[row * VS + 4 * ch + i] = vv[i];
            }
        }
        __syncthreads();
        if (skip || !wave_rows_live || (cmask && kb0 > q0w + 31)) continue;

        f32x16 sacc = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 2; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[l32 * KS + 2 * s + hi], qf[s], sacc, 0, 0, 0);
        const bool need_n = kb0 + BN > N;
        const bool need_c = cmask && (kb0 + BN - 1 > q0w);
        if (need_n || need_c) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = kb0 + 8 * (v >> 2) + 4 * hi + (v & 3);
                const bool bad = (j >= N) || (need_c && j > qi);
                sacc[v] = bad ? -__builtin_inff() : sacc[v];
            }
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
        mx = xor32_max(mx);
        const float mt = mx * sl2;
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        const float mu = (m_run == -__builtin_inff()) ? 0.f : m_run;
        ell *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
        float p[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], sl2, -mu));
            ell += p[v];
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = 8 * (v >> 2) + 4 * hi + (v & 3);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[key * VS + 32 * db + l32], p[v], oacc[db], 0, 0, 0);
            }
    }

    const float l_tot = xor32_sum(ell);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (wave_rows_live && qi < N && qi < q0 + bm) {
        float* Oh = static_cast<float*>(a.o) + bh * (int64_t)N * D + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = oacc[db][4 * j + i] * inv;
                *reinterpret_cast<f32x4*>(Oh + 32 * db + 8 * j + 4 * hi) = ov;
            }
        if (hi == 0) a.lse[bh * (int64_t)N + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
    }
}

template <int D, int MODE>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int bm = (MODE == (int)Mode::kSparse) ? a.block : BM;
    const int64_t grid = (int64_t)((a.N + bm - 1) / bm) * a.BH;
    hipLaunchKernelGGL((fwd_f32_kernel<D, MODE>), dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, Mode mode, hipStream_t stream) {
    switch (mode) {
        case Mode::kDense: return launch<D, (int)Mode::kDense>(a, stream);
        case Mode::kCausal: return launch<D, (int)Mode::kCausal>(a, stream);
        case Mode::kSparse: return launch<D, (int)Mode::kSparse>(a, stream);
        case Mode::kRange: break;   // key-range launches are bf16 only
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, Mode mode, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, mode, stream);
    return launch_d<128>(a, mode, stream);
}

}  // namespace bsattn
