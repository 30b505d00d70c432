// Fused attention forward, bf16 inputs, fp32 accumulation, for gfx950 (CDNA4).
//
// The method ("Exact Blocks, Rings, and Sparsity", section 2, "What the forward
// kernel keeps on chip"; FlashAttention notes, section 5.2): one workgroup owns
// a query tile that stays in registers; key/value tiles stream through LDS; for
// each tile the score tile S = scale * Q K^T is folded into a per-row online
// softmax state (running max m, denominator l, unnormalised accumulator A) and
// discarded, so S and P never reach HBM.  The epilogue writes O = A / l and
// LSE = m + ln l.
//
// gfx950 mapping (ours, not the pages'):
//   * 4 waves x 32 query rows (BM = 128); each wave computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16, so a lane holds 16 scores of ONE query row per
//     32-key block: the row max and row sum stay inside the lane plus one
//     exchange with lane l^32 (v_permlane32_swap), no LDS reductions.
//   * The S^T accumulator converts in place to the B operand of O^T += V^T P^T;
//     the key order inside each 16-key step is permuted to match, and V is
//     stored transposed and permuted in LDS so its A operand is one
//     ds_read_b128 per lane.
//   * Logits are handled in base-2 units (scale * log2 e folded into one FMA
//     before v_exp_f32).  The running max is only raised when a row's new max
//     exceeds it by more than 8 (a factor 256): exact, since A and l share the
//     stale max, and it removes almost every rescale of the accumulator.
//   * K/V tiles are double-buffered in LDS; the next tile's global loads are
//     in flight while the current tile is computed.
//   * Causal: key tiles wholly in the future are never visited; the diagonal
//     tiles get the element mask.  Block-sparse: the tile loop runs over the
//     canonical list of active key blocks of the query block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_common.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;                 // keys per tile step
constexpr float kSlack = 8.0f;         // lazy-rescale headroom, base-2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int NW>
struct Geo {
    static constexpr int NT = 64 * NW;             // threads per workgroup
    static constexpr int BM = 32 * NW;             // query rows per workgroup
    static constexpr int KS = D + 8;               // K row stride in LDS (bf16)
    static constexpr int VS = BN + 8;              // V^T row stride in LDS (bf16)
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int K_CHUNKS = BN * D / 8;    // 16-byte chunks of a K tile
    static constexpr int K_PER_T = K_CHUNKS / NT;
    static constexpr int V_PAIRS = (BN / 4) * (D / 8);   // (4 keys x 8 dims) pieces of a V tile
    static constexpr int V_PER_T = (V_PAIRS + NT - 1) / NT;
    static_assert(K_CHUNKS % NT == 0, "K tile must split evenly");
};

// Position of key o (0..15) of a 16-key step inside the V^T LDS row: keys
// {4h..4h+3, 8+4h..8+4h+3} (the ones lane half h holds in its S^T registers)
// become the contiguous slots 8h..8h+7.
__device__ __forceinline__ int vt_pos_of_quad(int kq) {
    // first key of quad kq (keys 4kq..4kq+3) within a BN-key tile
    return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
}

__device__ __forceinline__ float xor32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Tile descriptor: first key of the 64-key tile and what to mask in it.
struct TileDesc {
    int kb0;
    int causal_mask;   // element mask j <= i needed somewhere in the tile
    int skip;          // no valid key at all (compute skipped, loads clamped)
};

template <int D, int NW>
__device__ __forceinline__ void load_tile(const __bf16* __restrict__ Kh, const __bf16* __restrict__ Vh, int kb0,
                                          int N, int tid, u32x4 (&kreg)[Geo<D, NW>::K_PER_T],
                                          u32x4 (&vreg)[Geo<D, NW>::V_PER_T][4]) {
    using G = Geo<D, NW>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < G::K_PER_T; ++u) {
        const int c = tid + u * G::NT;
        const int row = c / CPR, ch = c % CPR;
        const int key = min(kb0 + row, N - 1);
        kreg[u] = *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + ch * 8);
    }
#pragma unroll
    for (int u = 0; u < G::V_PER_T; ++u) {
        const int pr = tid + u * G::NT;
        if (pr < G::V_PAIRS) {
            const int kq = pr % (BN / 4), dq = pr / (BN / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = min(kb0 + 4 * kq + r, N - 1);
                vreg[u][r] = *reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D + dq * 8);
            }
        }
    }
}

template <int D, int NW>
__device__ __forceinline__ void store_tile(__bf16* sK, __bf16* sV, int tid, const u32x4 (&kreg)[Geo<D, NW>::K_PER_T],
                                           const u32x4 (&vreg)[Geo<D, NW>::V_PER_T][4]) {
    using G = Geo<D, NW>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < G::K_PER_T; ++u) {
        const int c = tid + u * G::NT;
        const int row = c / CPR, ch = c % CPR;
        *reinterpret_cast<u32x4*>(sK + row * G::KS + ch * 8) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < G::V_PER_T; ++u) {
        const int pr = tid + u * G::NT;
        if (pr < G::V_PAIRS) {
            const int kq = pr % (BN / 4), dq = pr / (BN / 4);
            const int pos = vt_pos_of_quad(kq);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                const int sh = (e & 1) * 16;
                const unsigned a0 = (vreg[u][0][w] >> sh) & 0xffffu, a1 = (vreg[u][1][w] >> sh) & 0xffffu;
                const unsigned a2 = (vreg[u][2][w] >> sh) & 0xffffu, a3 = (vreg[u][3][w] >> sh) & 0xffffu;
                u32x2 pk;
                pk[0] = a0 | (a1 << 16);
                pk[1] = a2 | (a3 << 16);
                *reinterpret_cast<u32x2*>(sV + (dq * 8 + e) * G::VS + pos) = pk;
            }
        }
    }
}

template <int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(FwdArgs a) {
    using G = Geo<D, NW>;
    __shared__ __attribute__((aligned(16))) __bf16 smem[2 * G::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int N = a.N;
    const int nqt = (N + G::BM - 1) / G::BM;
    const int64_t total = (int64_t)nqt * a.BH;
    const int64_t ord = xcd_tile_order(blockIdx.x, total);
    const int64_t bh = ord / nqt;
    int qt = (int)(ord % nqt);
    if (MODE != (int)Mode::kDense) qt = nqt - 1 - qt;   // heaviest query tiles first
    const int q0 = qt * G::BM;
    const int q0w = q0 + 32 * w;

    const __bf16* Qh = static_cast<const __bf16*>(a.q) + bh * (int64_t)N * D;
    const __bf16* Kh = static_cast<const __bf16*>(a.k) + bh * (int64_t)N * D;
    const __bf16* Vh = static_cast<const __bf16*>(a.v) + bh * (int64_t)N * D;

    // Tile schedule.
    int ntiles = 0;
    int e0 = 0;
    int subs = 1;
    int nqb_meta = 0;
    if (MODE == (int)Mode::kDense) {
        ntiles = (N + BN - 1) / BN;
    } else if (MODE == (int)Mode::kCausal) {
        ntiles = (min(N, q0 + G::BM) + BN - 1) / BN;
    } else {
        subs = a.block / BN;
        nqb_meta = (N + a.block - 1) / a.block;
        const int h = (int)(bh % a.H);
        const int mh = a.meta_heads == 1 ? 0 : h;
        const int r = mh * nqb_meta + qt;            // BM == block for sparse launches
        int lo = a.row_ptr[r], hi_ = a.row_ptr[r + 1];
        lo = (int)min<int64_t>(max(lo, 0), a.nnz);
        hi_ = (int)min<int64_t>(max(hi_, lo), a.nnz);
        e0 = lo;
        ntiles = (hi_ - lo) * subs;
    }

    auto describe = [&](int it) -> TileDesc {
        TileDesc t;
        if (MODE == (int)Mode::kSparse) {
            const int e = e0 + it / subs;
            const int sub = it % subs;
            const int kb = a.col[e];
            const int f = a.flags[e];
            const bool valid = kb >= 0 && kb < nqb_meta;
            t.kb0 = valid ? kb * a.block + sub * BN : 0;
            // the flag comes from canonical metadata; the geometric test keeps a
            // causal launch correct even for lists that were not pruned
            t.causal_mask = ((f & 1) != 0) || (a.causal && t.kb0 + BN - 1 > q0);
            t.skip = !valid || t.kb0 >= N;
        } else {
            t.kb0 = it * BN;
            t.causal_mask = (MODE == (int)Mode::kCausal) && (t.kb0 + BN - 1 > q0);
            t.skip = 0;
        }
        return t;
    };

    // Query fragments (B operand of S^T = K Q^T): lane holds dims 16s+8hi..+7 of row q0w+l32.
    bf16x8 qf[D / 16];
    {
        const int qrow = min(q0w + l32, N - 1);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[s] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qrow * D + 16 * s + 8 * hi);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -__builtin_inff();   // running max, base-2 units (possibly stale by < kSlack)
    float ell = 0.f;           // this lane's share of the denominator
    const float sl2 = a.scale_log2;
    const int qi = q0w + l32;  // this lane's query row

    u32x4 kreg[G::K_PER_T];
    u32x4 vreg[G::V_PER_T][4];

    if (ntiles > 0) {
        TileDesc t0 = describe(0);
        load_tile<D, NW>(Kh, Vh, t0.kb0, N, tid, kreg, vreg);
        store_tile<D, NW>(smem, smem + G::K_ELEMS, tid, kreg, vreg);
        __syncthreads();
    }

    for (int it = 0; it < ntiles; ++it) {
        const TileDesc t = describe(it);
        const bool more = it + 1 < ntiles;
        if (more) {
            const TileDesc tn = describe(it + 1);
            load_tile<D, NW>(Kh, Vh, tn.kb0, N, tid, kreg, vreg);
        }
        const __bf16* sK = smem + (it & 1) * G::STAGE;
        const __bf16* sV = sK + G::K_ELEMS;

        const bool wave_dead = t.skip || (t.causal_mask && t.kb0 > q0w + 31);
        if (!wave_dead) {
            // ---- scores S^T (keys x queries) ----
            f32x16 sacc[BN / 32];
#pragma unroll
            for (int c = 0; c < BN / 32; ++c) {
                sacc[c] = f32x16{};
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (32 * c + l32) * G::KS + 16 * s + 8 * hi);
                    sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[c], 0, 0, 0);
                }
            }
            // ---- masks: keys past N, and j > i on diagonal tiles ----
            const bool need_n = t.kb0 + BN > N;
            const bool need_c = t.causal_mask && (t.kb0 + BN - 1 > q0w);
            if (need_n || need_c) {
#pragma unroll
                for (int c = 0; c < BN / 32; ++c)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int j = t.kb0 + 32 * c + 8 * (v >> 2) + 4 * hi + (v & 3);
                        const bool bad = (j >= N) || (need_c && j > qi);
                        sacc[c][v] = bad ? -__builtin_inff() : sacc[c][v];
                    }
            }
            // ---- online softmax ----
            float mx = -__builtin_inff();
#pragma unroll
            for (int c = 0; c < BN / 32; ++c)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[c][v]);
            mx = xor32_max(mx);
            const float mt = mx * sl2;
            const bool upd = mt > m_run + kSlack;
            if (__builtin_amdgcn_ballot_w64(upd) != 0) {
                const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
                m_run = upd ? mt : m_run;
                ell *= alpha;
#pragma unroll
                for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
            }
            const float mu = (m_run == -__builtin_inff()) ? 0.f : m_run;
            // P rounds to bf16 for the PV product; the denominator sums the fp32
            // values so LSE keeps fp32 accuracy even for rows with few keys.
            bf16x8 pf[BN / 16];
            float ts[8];
#pragma unroll
            for (int g = 0; g < BN / 16; ++g) {
                const int c = g >> 1, t8 = (g & 1) * 8;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[c][t8 + i], sl2, -mu));
                    ts[i] = g == 0 ? p : ts[i] + p;
                    pf[g][i] = (__bf16)p;
                }
            }
            ell += ((ts[0] + ts[1]) + (ts[2] + ts[3])) + ((ts[4] + ts[5]) + (ts[6] + ts[7]));
            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < BN / 16; ++g) {
                    const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + (32 * db + l32) * G::VS + 16 * g + 8 * hi);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[g], oacc[db], 0, 0, 0);
                }
        }

        if (more) {
            __bf16* nK = smem + ((it + 1) & 1) * G::STAGE;
            store_tile<D, NW>(nK, nK + G::K_ELEMS, tid, kreg, vreg);
        }
        __syncthreads();
    }

    // ---- epilogue: O = A / l, LSE = (m + log2 l) * ln 2 ----
    const float l_tot = xor32_sum(ell);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qi < N) {
        __bf16* Oh = static_cast<__bf16*>(a.o) + bh * (int64_t)N * D + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][4 * j + i] * inv);
                *reinterpret_cast<bf16x4*>(Oh + 32 * db + 8 * j + 4 * hi) = ov;
            }
        if (hi == 0) {
            a.lse[bh * (int64_t)N + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        }
    }
}

template <int D, int NW, int MODE>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    using G = Geo<D, NW>;
    const int64_t nqt = (a.N + G::BM - 1) / G::BM;
    const int64_t grid = nqt * a.BH;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, MODE>), dim3((unsigned)grid), dim3(G::NT), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, Mode mode, hipStream_t stream) {
    switch (mode) {
        case Mode::kDense: return launch<D, 4, (int)Mode::kDense>(a, stream);
        case Mode::kCausal: return launch<D, 4, (int)Mode::kCausal>(a, stream);
        case Mode::kSparse:
            if (a.block == 128) return launch<D, 4, (int)Mode::kSparse>(a, stream);
            return launch<D, 2, (int)Mode::kSparse>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, Mode mode, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, mode, stream);
    return launch_d<128>(a, mode, stream);
}

}  // namespace bsattn
