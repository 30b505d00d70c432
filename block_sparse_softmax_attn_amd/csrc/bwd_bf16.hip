// Attention backward, bf16 inputs, fp32 accumulation, for gfx950 (CDNA4).
//
// The method ("Exact Blocks, Rings, and Sparsity", section 3, "FlashAttention
// Backward: recomputing P"; FlashAttention notes, section 5.3): P is rebuilt
// tile by tile from Q, K and the saved LSE, dP = dO V^T, dS = P (dP - D) with
// the per-row scalar D = dO . O from a preprocessing pass, and each tile's
// contributions to dQ, dK and dV are accumulated on chip; S, P, dP and dS never
// reach HBM.  The two opposing reductions (dK, dV sum over queries; dQ sums over
// keys) are split over two kernels, without atomics, the two-traversal choice
// that section describes:
//   * dK/dV: a workgroup owns a block of keys (32 per wave, kept in registers
//     together with their V rows) and streams 64-query tiles of Q, dO and the
//     row statistics through LDS;
//   * dQ: a workgroup owns a block of queries (as in the forward) and streams
//     64-key tiles of K and V.
// Both recompute S and dP for their tiles.
//
// gfx950 mapping (ours, not the pages'):
//   * dK/dV computes S = Q K^T and dP = dO V^T with the keys as the MFMA
//     columns: a lane holds 16 queries of ONE key, and those registers (P and
//     dS rounded to bf16) are directly the B operand of dV^T += dO^T P and
//     dK^T += Q^T dS.  The dP product runs on -V and starts from D (read from
//     LDS straight into the accumulator), so it yields D - dP and dS costs one
//     multiply per element; the wave accumulates -dK, negated in the epilogue.  The A operands dO^T and Q^T come from the same
//     row-major dO and Q tiles through the transposing LDS load
//     (ds_read_b64_tr_b16), in the query order the P and dS registers hold.
//   * dQ computes S^T = K Q^T and dP^T = V dO^T (a lane holds keys of ONE query,
//     the forward's layout): LSE_i and D_i are lane scalars, and dS^T is the B
//     operand of dQ^T += K^T dS^T, whose A operand K^T is read transposed from
//     the K tile.
//   * Every tile goes from global memory straight into LDS
//     (global_load_lds_dwordx4), XOR-swizzled so that both the plain and the
//     transposing reads spread over the banks; two tiles in flight for dK/dV,
//     up to three for dQ.  No transposed copy of any input is made.
//   * Rows without allowed keys, and rows past N, get LSE = +inf in the row
//     statistics, so exp2(s - lse) = 0 and they contribute nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fwd_common.h"
#include "gfx950_util.h"

namespace bsattn {
namespace {

constexpr int BT = 64;   // tokens per streamed tile: queries (dK/dV) or keys (dQ)
constexpr float kLog2e = 1.4426950408889634f;

// Block-sparse dK/dV: a key block whose list holds more than kPieceTiles query
// tiles is split into up to kMaxPieces pieces, each a workgroup of its own
// (a globally listed key block would otherwise run its whole list in one
// workgroup while the rest of the GPU idles).
constexpr int kPieceTiles = 32;
constexpr int kMaxPieces = 8;
constexpr int64_t kMaxSlots = 1 << 18;   // partial slots a call uses at most

__host__ __device__ inline int pieces_of(int ntiles) {
    if (ntiles <= kPieceTiles) return 1;
    return min(kMaxPieces, (ntiles + kPieceTiles - 1) / kPieceTiles);
}

// Entry idx of the split plan, written by the plan launch (scalar loads).
__device__ inline int2 plan_at(const BwdArgs& a, int64_t idx) {
    const int32_t* p = reinterpret_cast<const int32_t*>(a.plan);
    return make_int2(ld_meta(p, 2 * idx), ld_meta(p, 2 * idx + 1));
}

// Query tiles the key tile kt of key/value head kvbh visits, over the query
// heads of its group, in a block-sparse launch (BKV == block).
__device__ inline int sparse_key_tiles(const BwdArgs& a, int64_t kvbh, int kt, int nqb_meta, int subs) {
    const int group = a.H / a.Hkv;
    const int64_t bh0 = (kvbh / a.Hkv) * a.H + (kvbh % a.Hkv) * group;
    int n = 0;
    for (int gi = 0; gi < group; ++gi) {
        const int64_t r = meta_of(bh0 + gi, a.H, a.Hkv, a.meta_heads) * nqb_meta + kt;
        int lo = ld_meta(a.t_row_ptr, r), hi_ = ld_meta(a.t_row_ptr, r + 1);
        lo = (int)min<int64_t>(max(lo, 0), a.t_nnz);
        hi_ = (int)min<int64_t>(max(hi_, lo), a.t_nnz);
        n += (hi_ - lo) * subs;
    }
    return n;
}

// The split plan, by one workgroup of 256 threads: for every (key/value head,
// key tile) in order, its number of pieces and the first of its partial slots
// (an exclusive scan over the split items; unsplit items get slot -1), then the
// extra-piece list. It runs as one more workgroup of the row-statistics launch,
// beside the statistics, so it costs no launch of its own.
__device__ void split_plan(const BwdArgs& a, int nkt, int64_t items) {
    __shared__ int warp_tot[4];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nqb_meta = (a.N + a.block - 1) / a.block, subs = a.block / BT;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < items; base += 256) {
        const int64_t it = base + tid;
        int np = 0;
        if (it < items) np = pieces_of(sparse_key_tiles(a, it / nkt, (int)(it % nkt), nqb_meta, subs));
        const int need = np > 1 ? np : 0;
        // inclusive scan inside the wave, then across the 4 waves
        int x = need;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) warp_tot[w] = x;
        __syncthreads();
        int before = carry;
        for (int i = 0; i < w; ++i) before += warp_tot[i];
        if (it < items) a.plan[it] = make_int2(need ? before + x - need : -1, max(np, 1));
        __syncthreads();
        if (tid == 255) carry = before + x;
        __syncthreads();
    }
    const int used = carry;
    __syncthreads();
    if (used > a.part_slots) {   // the workspace holds fewer slots: no key tile is split
        for (int64_t it = tid; it < items; it += 256) a.plan[it] = make_int2(-1, 1);
        for (int64_t w2 = tid; w2 < a.part_slots; w2 += 256) a.extra[w2] = make_int2(-1, -1);
        return;
    }
    // the extra-piece list, indexed by slot: slot base + p holds (item, p)
    for (int64_t w2 = used + tid; w2 < a.part_slots; w2 += 256) a.extra[w2] = make_int2(-1, -1);
    for (int64_t it = tid; it < items; it += 256) {
        const int2 pl = a.plan[it];
        for (int p = 0; p < pl.y && pl.x >= 0; ++p) a.extra[pl.x + p] = make_int2((int)it, p);
    }
}

// ---------------------------------------------------------------------------
// row statistics: one workgroup per 64-row block (plus one padding block)
// ---------------------------------------------------------------------------

// stats[bh][blk][0..63]   = LSE_i * log2 e  (+inf: row without keys, or i >= N)
// stats[bh][blk][64..127] = D_i = dO_i . O_i (0 for i >= N)
// PLAN: column nblk + 1 of the grid holds the split-plan workgroup (row 0) and
// nothing else.  Grid rows stride over the heads (the grid's second dimension
// is capped below B*H on large batches).
template <int D, bool PLAN>
__global__ __launch_bounds__(256) void bwd_stats_kernel(BwdArgs a, int nblk, int nkt, int64_t items) {
    const int blk = blockIdx.x;
    if (PLAN && blk == nblk + 1) {
        if (blockIdx.y == 0) split_plan(a, nkt, items);
        return;
    }
    const __bf16* __restrict__ o = static_cast<const __bf16*>(a.o);
    const __bf16* __restrict__ dout = static_cast<const __bf16*>(a.dout);
    const float* __restrict__ lse = a.lse;
    float* __restrict__ stats = a.stats;
    const int N = a.N;
    const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int i = blk * BT + r;
    for (int64_t bh = blockIdx.y; bh < a.BH; bh += gridDim.y) {
    float acc = 0.f;
    if (i < N) {
        const __bf16* orow = o + (bh * N + i) * (int64_t)D;
        const __bf16* drow = dout + (bh * N + i) * (int64_t)D;
#pragma unroll
        for (int c = part; c < D / 8; c += 4) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(orow + 8 * c);
            const bf16x8 y = *reinterpret_cast<const bf16x8*>(drow + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0) {
        float* st = stats + (bh * (nblk + 1) + blk) * 128;
        float l2 = __builtin_inff();
        if (i < N) {
            const float L = lse[bh * N + i];
            if (L > -__builtin_inff()) l2 = L * kLog2e;
        }
        st[r] = l2;
        st[64 + r] = acc;
    }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: key-stationary
// ---------------------------------------------------------------------------

template <int D, int NW, bool PAIRED>
struct DkdvGeo {
    static constexpr int NT = 64 * NW;
    static constexpr int PAIRS = PAIRED ? NW / 2 : NW;   // 32-key slices per workgroup
    static constexpr int BKV = 32 * PAIRS;               // keys per workgroup
    static constexpr int TB = BT * D * 2;            // bytes of a Q or dO tile
    static constexpr int PER_T = TB / 1024 / NW;     // 1 KiB direct-to-LDS loads per wave per tile
    static_assert((!PAIRED || NW % 2 == 0) && TB % (1024 * NW) == 0, "tile must split over waves");
    static_assert(2 * PER_T + 1 < 64, "vmcnt range");
};

// PAIRED (d = 128): two waves share each 32-key slice: the P wave (role 0)
// computes S = Q K^T, P and dV^T += dO^T P; the dS wave (role 1) computes
// dP = dO V^T, reads the rounded P from LDS, forms dS = P (dP - D) and
// dK^T += Q^T dS.  Each keeps one operand row set and one accumulator, so both
// fit two waves per SIMD and their MFMA and VALU phases overlap; the P
// hand-over costs one extra barrier per tile.  Single (d = 64, where one wave
// holding K, V, dK and dV already fits two waves per SIMD): each wave does all
// four products for its 32 keys.
template <int D, int NW, int MODE, bool PAIRED>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dkdv_kernel(BwdArgs a) {
    using G = DkdvGeo<D, NW, PAIRED>;
    // Q tiles of the two stages, then dO tiles: sQO + u TB (Q), sQO + (2 + u) TB (dO)
    __shared__ __attribute__((aligned(1024))) unsigned char sQO[4 * G::TB];
    unsigned char* const sQ0 = sQO;
    unsigned char* const sQ1 = sQO + G::TB;
    unsigned char* const sO0 = sQO + 2 * G::TB;
    unsigned char* const sO1 = sQO + 3 * G::TB;
    __shared__ __attribute__((aligned(1024))) float sS0[256], sS1[256];
    __shared__ __attribute__((aligned(16))) bf16x8 sP[PAIRED ? G::PAIRS : 1][2][2][64];   // [pair][block][step][lane]
    __shared__ __attribute__((aligned(16))) float sZ[64];   // zeros: the P wave's accumulator start

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int role = PAIRED ? w / G::PAIRS : 0, pw = PAIRED ? w % G::PAIRS : w;
    const TrLane<D> trl = tr_lane<D>(lane);   // transposing-read offsets of dO^T / Q^T
    const RtLane<D> rtl = rt_lane<D>(lane);   // plain fragment offsets of Q / dO
    const int N = a.N;
    const int nkt = (N + G::BKV - 1) / G::BKV;
    // one workgroup per (key/value head, key tile); it sums the contributions
    // of every query head of the key/value head's group
    const int group = a.H / a.Hkv;
    const int64_t BHkv = a.BH / group;
    int64_t kvbh;
    int kt;   // causal: the first key tiles see the most queries and start first
    // block-sparse: the first part_slots workgroups run the pieces >= 1 of
    // split key tiles from the plan's list (so the long lists start first),
    // the others piece 0 of every key tile
    int piece = 0;
    const int64_t nextra = MODE == (int)Mode::kSparse ? a.part_slots : 0;
    if (MODE == (int)Mode::kSparse && (int64_t)blockIdx.x < nextra) {
        const int32_t* ex = reinterpret_cast<const int32_t*>(a.extra);
        const int64_t item = ld_meta(ex, 2 * (int64_t)blockIdx.x);
        piece = ld_meta(ex, 2 * (int64_t)blockIdx.x + 1);
        if (item < 0 || piece < 1) return;   // uniform: before any barrier
        kvbh = item / nkt;
        kt = (int)(item % nkt);
    } else if (MODE == (int)Mode::kDense) {
        const int64_t ord = xcd_tile_order(blockIdx.x, (int64_t)nkt * BHkv);
        kvbh = ord / nkt;
        kt = (int)(ord % nkt);
    } else {
        rank_major_order(blockIdx.x - nextra, (int64_t)nkt * BHkv, nkt, kvbh, kt);
    }
    const int64_t bh0 = (kvbh / a.Hkv) * a.H + (kvbh % a.Hkv) * group;   // first query head of the group
    const int kb0 = kt * G::BKV;
    const int kw0 = kb0 + 32 * pw;     // this wave pair's first key
    const int kj = kw0 + l32;          // this lane's key
    const int nblk = a.npad / BT;
    const bool causal = MODE == (int)Mode::kCausal || (MODE == (int)Mode::kSparse && a.causal);

    const __bf16* Kh = static_cast<const __bf16*>(a.k) + kvbh * (int64_t)N * D;
    const __bf16* Vh = static_cast<const __bf16*>(a.v) + kvbh * (int64_t)N * D;

    // ---- schedule: 64-query tiles of each query head of the group ----
    int per = 0, first = 0, subs = 1, nqb_meta = 0;
    bool uniform = true;   // every query head of the group has the same tile list
    if (MODE == (int)Mode::kDense) {
        per = (N + BT - 1) / BT;
    } else if (MODE == (int)Mode::kCausal) {
        first = kb0 / BT;   // queries before the first key see none of these keys
        per = (N + BT - 1) / BT - first;
    } else {
        subs = a.block / BT;
        nqb_meta = (N + a.block - 1) / a.block;
        uniform = group == 1 || a.meta_heads == 1 || a.meta_heads == a.Hkv;
    }
    // entries [lo, hi) of the transposed list of query head bh0 + gi (BKV == block)
    auto list_of = [&](int gi, int& lo, int& hi_) {
        const int64_t r = meta_of(bh0 + gi, a.H, a.Hkv, a.meta_heads) * nqb_meta + kt;
        lo = ld_meta(a.t_row_ptr, r);
        hi_ = ld_meta(a.t_row_ptr, r + 1);
        lo = (int)min<int64_t>(max(lo, 0), a.t_nnz);
        hi_ = (int)min<int64_t>(max(hi_, lo), a.t_nnz);
    };
    int ntiles = 0;
    int lo_u = 0;   // first entry of a list every query head of the group shares
    if (MODE != (int)Mode::kSparse) {
        ntiles = per * group;
    } else if (uniform) {
        int lo, hi_;
        list_of(0, lo, hi_);
        per = (hi_ - lo) * subs;
        ntiles = per * group;
        lo_u = lo;
    } else {
        for (int gi = 0; gi < group; ++gi) {
            int lo, hi_;
            list_of(gi, lo, hi_);
            ntiles += (hi_ - lo) * subs;
        }
    }
    // this workgroup's piece of the tile list (the plan's choice: a split the
    // workspace cannot hold was turned off there)
    const int npieces = MODE == (int)Mode::kSparse ? plan_at(a, kvbh * nkt + kt).y : 1;
    if (piece >= npieces) return;   // uniform: before any barrier
    const int psize = (ntiles + npieces - 1) / npieces;
    const int t_lo = piece * psize, t_hi = min(ntiles, t_lo + psize);
    // Tile it: its query head and first query (-1 for an out-of-range entry).
    struct QTile {
        int64_t bhq;
        int q0;
    };
    auto locate = [&](int it) -> QTile {
        int gi = 0, loc = it;
        if (uniform) {
            gi = it / per;
            loc = it % per;
        } else {
            for (;;) {
                int lo, hi_;
                list_of(gi, lo, hi_);
                if (loc < (hi_ - lo) * subs) break;
                loc -= (hi_ - lo) * subs;
                ++gi;
            }
        }
        QTile t;
        t.bhq = bh0 + gi;
        if (MODE != (int)Mode::kSparse) {
            t.q0 = (first + loc) * BT;
        } else {
            // a shared list's start is known; per-head lists look theirs up
            int lo = lo_u, hi_;
            if (!uniform) list_of(gi, lo, hi_);
            const int qb = ld_meta(a.t_col, lo + loc / subs);
            t.q0 = (qb >= 0 && qb < nqb_meta) ? qb * a.block + (loc % subs) * BT : -1;
        }
        return t;
    };

    // Direct-to-LDS sources: load i of this wave fills bytes [1024 (w PER_T + i)
    // + 16 lane, +16) of a tile: row r, physical chunk p, holding logical chunk
    // rt_swz(r, p) of that row.
    int rm_row[G::PER_T], rm_col[G::PER_T];
#pragma unroll
    for (int i = 0; i < G::PER_T; ++i) {
        const int byte = (w * G::PER_T + i) * 1024 + lane * 16;
        const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
        rm_row[i] = r;
        rm_col[i] = rt_swz<D>(r, p) * 8;
    }
    // Loads from a tile base that moves in scalar registers plus fixed
    // per-lane byte offsets; a tile that reaches past row N - 1 clamps its
    // rows to it instead.
    unsigned rm_boff[G::PER_T];
#pragma unroll
    for (int i = 0; i < G::PER_T; ++i) rm_boff[i] = (unsigned)(2 * (rm_row[i] * D + rm_col[i]));
    const unsigned lq[2] = {lds_addr(sQ0), lds_addr(sQ1)}, lo[2] = {lds_addr(sO0), lds_addr(sO1)};
    const unsigned ls[2] = {lds_addr(sS0), lds_addr(sS1)};
    const unsigned wl = __builtin_amdgcn_readfirstlane(w * G::PER_T * 1024);   // this wave's part of a tile
    auto issue = [&](const QTile& t, int u) {
        const int q0 = max(t.q0, 0);
        const __bf16* Qh = static_cast<const __bf16*>(a.q) + t.bhq * (int64_t)N * D;
        const __bf16* dOh = static_cast<const __bf16*>(a.dout) + t.bhq * (int64_t)N * D;
        const float* Sh = a.stats + t.bhq * (int64_t)(nblk + 1) * 128;
        if (q0 + BT <= N) {
            const __bf16* qt = Qh + (int64_t)q0 * D;
            const __bf16* ot = dOh + (int64_t)q0 * D;
#pragma unroll
            for (int i = 0; i < G::PER_T; ++i) {
                dma16_at(qt, rm_boff[i], lq[u] + wl + i * 1024);
                dma16_at(ot, rm_boff[i], lo[u] + wl + i * 1024);
            }
        } else {
            const int rb = min(q0, N - 1);   // clamped rows stay at or after rb
            const __bf16* qt = Qh + (int64_t)rb * D;
            const __bf16* ot = dOh + (int64_t)rb * D;
#pragma unroll
            for (int i = 0; i < G::PER_T; ++i) {
                const unsigned off = (unsigned)(2 * ((min(q0 + rm_row[i], N - 1) - rb) * D + rm_col[i]));
                dma16_at(qt, off, lq[u] + wl + i * 1024);
                dma16_at(ot, off, lo[u] + wl + i * 1024);
            }
        }
        // row statistics of this block (lanes 0-31) and of the next (32-63)
        if (w == 0) dma16_at(Sh + (q0 / BT) * 128, (unsigned)(lane * 16), ls[u]);
    };

    // ---- operands, accumulators and one tile's math for each design ----
    bf16x8 kvf[D / 16];          // paired: K (P wave) or V (dS wave) rows
    f32x16 acc[D / 32];          // paired: dV^T (P wave) or dK^T (dS wave)
    bf16x8 kf[PAIRED ? 1 : D / 16], vf[PAIRED ? 1 : D / 16];
    f32x16 dkacc[PAIRED ? 1 : D / 32], dvacc[PAIRED ? 1 : D / 32];
    if constexpr (PAIRED) {
        // this lane's key row (P wave: B operand of S = Q K^T) or value row
        // (dS wave: B operand of dP = dO V^T)
        const int row = min(kj, N - 1);
        const __bf16* src = (role == 0 ? Kh : Vh) + (int64_t)row * D + 8 * hi;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) kvf[k] = *reinterpret_cast<const bf16x8*>(src + 16 * k);
        // the dS wave holds -V, so its product started from D gives D - dP
        const unsigned flip = role == 0 ? 0u : 0x80008000u;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
            u32x4 x = __builtin_bit_cast(u32x4, kvf[k]);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] ^= flip;
            kvf[k] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
    } else {
        // this lane's key and value rows: B operands of S = Q K^T and dP = dO V^T
        const int row = min(kj, N - 1);
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
            kf[k] = *reinterpret_cast<const bf16x8*>(Kh + (int64_t)row * D + 16 * k + 8 * hi);
            vf[k] = *reinterpret_cast<const bf16x8*>(Vh + (int64_t)row * D + 16 * k + 8 * hi);
            // -V: the product started from D gives D - dP
            u32x4 x = __builtin_bit_cast(u32x4, vf[k]);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] ^= 0x80008000u;
            vf[k] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            dkacc[i] = f32x16{};
            dvacc[i] = f32x16{};
        }
    }
    if (tid < 64) sZ[tid] = 0.f;
    wait_vmcnt<0>();
    const float sl2 = a.scale_log2;

    // One 64-query tile, as two 32-query blocks.  Phase 1: S (P wave) or dP
    // (dS wave) for both blocks; the P wave writes the rounded P to LDS.
    // Barrier.  Phase 2: dV (P wave, P still in registers) or dS and dK (dS
    // wave).  Every wave reaches the barrier, also when the causal mask leaves
    // it nothing to do.
    // Paired: the wave's phase-1 operand (Q for the P wave, dO for the dS wave)
    // and phase-2 operand (dO^T, Q^T) are at a role-dependent distance from
    // the stage's Q tile; folded into the lane offsets once, every read is a
    // register plus an immediate.
    int a_off[D / 16];
    TrLane<D> t_off = trl;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) a_off[k] = rtl.off[k] + (role == 0 ? 0 : 2 * G::TB);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) t_off.off[h][db] += role == 0 ? 2 * G::TB : 0;
    auto compute_paired = [&](int q0, int u) {
        const unsigned char* bQ = u ? sQ1 : sQ0;
        const float* st = u ? sS1 : sS0;
        bool live[2];
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) live[qc] = !(causal && q0 + 32 * qc + 31 < kw0);
        // ---- phase 1: queries as rows, lane (l32, hi) gets query
        // q0 + 32qc + 8(v>>2) + 4hi + (v&3) of key kj in element v ----
        f32x16 pr[2];
        bf16x8 pb[2][2];
        // accumulators start at 0 (P wave: S) or at D_q (dS wave: D - dP, the
        // wave's V rows being negated); lane (l32, hi) element 4 g4 + e is query
        // 32 qc + 8 g4 + 4 hi + e
        const float* ib = role == 0 ? sZ : st + 64;
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
            pr[qc] = f32x16{};
            if (!live[qc]) continue;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 d4 = *reinterpret_cast<const float4*>(ib + 32 * qc * role + 8 * g4 + 4 * hi);
                pr[qc][4 * g4 + 0] = d4.x;
                pr[qc][4 * g4 + 1] = d4.y;
                pr[qc][4 * g4 + 2] = d4.z;
                pr[qc][4 * g4 + 3] = d4.w;
            }
            bf16x8 fa[D / 16];
#pragma unroll
            for (int k = 0; k < D / 16; ++k)
                fa[k] = *reinterpret_cast<const bf16x8*>(bQ + a_off[k] + 32 * qc * (2 * D));
            __builtin_amdgcn_iglp_opt(0);
#pragma unroll
            for (int k = 0; k < D / 16; ++k) pr[qc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], kvf[k], pr[qc], 0, 0, 0);
        }
        if (role == 0) {
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                if (!live[qc]) continue;
                const int qb0 = q0 + 32 * qc;
                // causal: scores of keys after their query become -inf (P = 0)
                // in a block of their own, so unmasked tiles pay nothing for it
                if (causal && qb0 < kw0 + 31) {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (kj > qb0 + 8 * (v >> 2) + 4 * hi + (v & 3)) pr[qc][v] = -__builtin_inff();
                }
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const float4 l4 = *reinterpret_cast<const float4*>(st + 32 * qc + 8 * g4 + 4 * hi);
                    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 4 * g4 + e;
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(pr[qc][v], sl2, -lv[e]));
                        pb[qc][v >> 3][v & 7] = (__bf16)p;
                    }
                }
                sP[pw][qc][0][lane] = pb[qc][0];
                sP[pw][qc][1][lane] = pb[qc][1];
            }
        }
        barrier();
        // ---- phase 2 ----
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
            if (!live[qc]) continue;
            bf16x8 op[2];
            if (role == 0) {
                op[0] = pb[qc][0];
                op[1] = pb[qc][1];
            } else {
                // -dS = P (D - dP) from the rounded P, rounded to bf16 (the
                // epilogue negates dK)
                const bf16x8 p0 = sP[pw][qc][0][lane], p1 = sP[pw][qc][1][lane];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = (float)((v >> 3) ? p1[v & 7] : p0[v & 7]);
                    op[v >> 3][v & 7] = (__bf16)(p * pr[qc][v]);
                }
            }
            // dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave) over two 16-query steps
            bf16x8 ta[2][D / 32];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) ta[t][db] = tr_operand<D>(bQ, t_off, 2 * qc + t, db);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[t][db], op[t], acc[db], 0, 0, 0);
        }
    };



    // One 64-query tile for this wave, as two 32-query blocks.  Each phase
    // loads all of its LDS operands first, then issues its MFMAs, so the
    // matrix pipe is not stalled by one LDS round trip per product.
    auto compute_single = [&](int q0, int u) {
        const unsigned char* bQ = u ? sQ1 : sQ0;
        const unsigned char* bO = u ? sO1 : sO0;
        const float* st = u ? sS1 : sS0;
#pragma unroll
        for (int qc = 0; qc < BT / 32; ++qc) {
            const int qb0 = q0 + 32 * qc;
            if (causal && qb0 + 31 < kw0) continue;   // all 32 queries precede all keys of this wave
            // ---- S = Q K^T and dP = dO V^T, queries as rows: lane (l32, hi)
            // gets query qb0 + 8(v>>2) + 4hi + (v&3) of key kj in element v ----
            bf16x8 fa[D / 16], fb[D / 16];
#pragma unroll
            for (int k = 0; k < D / 16; ++k) {
                const int off = rtl.off[k] + 32 * qc * (2 * D);
                fa[k] = *reinterpret_cast<const bf16x8*>(bQ + off);
                fb[k] = *reinterpret_cast<const bf16x8*>(bO + off);
            }
            // dp starts at D (its B operand is -V): D - dP
            f32x16 s = f32x16{}, dp;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 d4 = *reinterpret_cast<const float4*>(st + 64 + 32 * qc + 8 * g4 + 4 * hi);
                dp[4 * g4 + 0] = d4.x;
                dp[4 * g4 + 1] = d4.y;
                dp[4 * g4 + 2] = d4.z;
                dp[4 * g4 + 3] = d4.w;
            }
            __builtin_amdgcn_iglp_opt(0);
#pragma unroll
            for (int k = 0; k < D / 16; ++k) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], kf[k], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[k], vf[k], dp, 0, 0, 0);
            }
            // operands of the dV and dK products, fetched while S and dP run
            bf16x8 ta[2][D / 32], tb[2][D / 32];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    ta[t][db] = tr_operand<D>(bO, trl, 2 * qc + t, db);
                    tb[t][db] = tr_operand<D>(bQ, trl, 2 * qc + t, db);
                }
            // causal: scores of keys after their query become -inf (P = 0), in
            // a block of their own
            if (causal && qb0 < kw0 + 31) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (kj > qb0 + 8 * (v >> 2) + 4 * hi + (v & 3)) s[v] = -__builtin_inff();
            }
            // ---- P = exp2(s * scale log2 e - lse2) and dS = P (dP - D), bf16 ----
            bf16x8 pb[2], dsb[2];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 l4 = *reinterpret_cast<const float4*>(st + 32 * qc + 8 * g4 + 4 * hi);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * g4 + e;
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], sl2, -lv[e]));
                    const __bf16 pr = (__bf16)p;
                    pb[v >> 3][v & 7] = pr;
                    dsb[v >> 3][v & 7] = (__bf16)((float)pr * dp[v]);   // -dS
                }
            }
            // ---- dV^T += dO^T P, dK^T += Q^T dS over the two 16-query steps ----
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[t][db], pb[t], dvacc[db], 0, 0, 0);
                    dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[t][db], dsb[t], dkacc[db], 0, 0, 0);
                }
        }
    };

    auto compute = [&](int q0, int u) {
        if constexpr (PAIRED) {
            compute_paired(q0, u);
        } else {
            if (causal && q0 + BT - 1 < kw0) return;   // the whole tile precedes this wave's keys
            compute_single(q0, u);
        }
    };

    // Tile it sits in buffer it & 1: wait for its loads, barrier (every wave's
    // loads have landed, every wave is done with tile it-1 and with its P),
    // refill the other buffer with tile it+1, compute.
    auto step = [&](int it, int u) {
        wait_vmcnt<0>();
        barrier();
        if (it + 1 < t_hi) issue(locate(it + 1), u ^ 1);
        const int q0 = locate(it).q0;
        if (q0 < 0 || q0 >= N) return;                  // the same for every wave
        if (causal && q0 + BT - 1 < kb0) return;         // the whole tile precedes every key of the workgroup
        compute(q0, u);
    };
    if (t_lo < t_hi) issue(locate(t_lo), 0);
    for (int base = t_lo; base < t_hi; base += 2) {
        step(base, 0);
        if (base + 1 < t_hi) step(base + 1, 1);
    }

    if (npieces > 1) {   // fp32 partial sums of this piece: reduced in piece order afterwards
        const int slot = plan_at(a, kvbh * nkt + kt).x + piece;
        float* pK = a.part + (int64_t)slot * (2 * G::BKV * D) + (int64_t)(kj - kb0) * D;
        float* pV = pK + G::BKV * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 32 * db + 8 * j + 4 * hi;
                if constexpr (PAIRED) {
                    const float4 x = {acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
                    *reinterpret_cast<float4*>((role == 0 ? pV : pK) + c) = x;
                } else {
                    const float4 xk = {dkacc[db][4 * j], dkacc[db][4 * j + 1], dkacc[db][4 * j + 2], dkacc[db][4 * j + 3]};
                    const float4 xv = {dvacc[db][4 * j], dvacc[db][4 * j + 1], dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]};
                    *reinterpret_cast<float4*>(pK + c) = xk;
                    *reinterpret_cast<float4*>(pV + c) = xv;
                }
            }
        return;
    }

    // ---- epilogue: dV = (dO^T P)^T, dK = scale * (Q^T dS)^T ----
    if (kj < N) {
        __bf16* dKr = static_cast<__bf16*>(a.dk) + (kvbh * N + kj) * (int64_t)D;
        __bf16* dVr = static_cast<__bf16*>(a.dv) + (kvbh * N + kj) * (int64_t)D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 32 * db + 8 * j + 4 * hi;
                bf16x4 kv, vv;
                if constexpr (PAIRED) {
                    const float f = role == 0 ? 1.0f : -a.scale;
#pragma unroll
                    for (int i = 0; i < 4; ++i) kv[i] = (__bf16)(acc[db][4 * j + i] * f);
                    *reinterpret_cast<bf16x4*>((role == 0 ? dVr : dKr) + c) = kv;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        kv[i] = (__bf16)(dkacc[db][4 * j + i] * -a.scale);
                        vv[i] = (__bf16)dvacc[db][4 * j + i];
                    }
                    *reinterpret_cast<bf16x4*>(dKr + c) = kv;
                    *reinterpret_cast<bf16x4*>(dVr + c) = vv;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary
// ---------------------------------------------------------------------------

template <int D, int NW, int NS, int KT = BT>
struct DqGeo {
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 32 * NW;               // queries per workgroup
    static constexpr int TB = KT * D * 2;            // bytes of a K or V tile (KT keys)
    static constexpr int PER_T = TB / 1024 / NW;
    static constexpr int PER_W = 2 * PER_T;
    static_assert(TB % (1024 * NW) == 0, "tile must split over waves");
    static_assert(NS == 2 || NS == 3, "2 or 3 stages");
    static_assert((NS - 2) * PER_W < 64, "vmcnt range");
};

struct KeyTile {
    int kb0;      // first key
    int nlim;     // keys j >= nlim are masked (N; 0 for an invalid metadata entry)
    int causal;   // element mask j <= i applies
    int masked;   // any element mask needed
};

template <int D, int NW, int NS, int MODE, int KT = BT>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(BwdArgs a) {
    using G = DqGeo<D, NW, NS, KT>;
    constexpr int T2 = NS > 2 ? G::TB : 16;
    __shared__ __attribute__((aligned(1024))) unsigned char sK0[G::TB], sK1[G::TB], sK2[T2];
    __shared__ __attribute__((aligned(1024))) unsigned char sV0[G::TB], sV1[G::TB], sV2[T2];
    unsigned char* const kbuf[3] = {sK0, sK1, sK2};
    unsigned char* const vbuf[3] = {sV0, sV1, sV2};

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const TrLane<D> trl = tr_lane<D>(lane);   // transposing-read offsets of K^T
    const RtLane<D> rtl = rt_lane<D>(lane);   // plain fragment offsets of K / V
    const int N = a.N;
    const int nqt = (N + G::BM - 1) / G::BM;
    int64_t bh;
    int qt;
    if (MODE == (int)Mode::kDense) {
        const int64_t ord = xcd_tile_order(blockIdx.x, (int64_t)nqt * a.BH);
        bh = ord / nqt;
        qt = (int)(ord % nqt);
    } else {
        rank_major_order(blockIdx.x, (int64_t)nqt * a.BH, nqt, bh, qt);
        qt = nqt - 1 - qt;   // heaviest query tiles first
    }
    const int q0 = qt * G::BM;
    const int q0w = q0 + 32 * w;
    const int qi = q0w + l32;
    const int nblk = a.npad / BT;

    const __bf16* Qh = static_cast<const __bf16*>(a.q) + bh * (int64_t)N * D;
    const __bf16* dOh = static_cast<const __bf16*>(a.dout) + bh * (int64_t)N * D;
    const int64_t kvh = kv_head_of(bh, a.H, a.Hkv);
    const __bf16* Kh = static_cast<const __bf16*>(a.k) + kvh * (int64_t)N * D;
    const __bf16* Vh = static_cast<const __bf16*>(a.v) + kvh * (int64_t)N * D;
    const float* Sh = a.stats + bh * (int64_t)(nblk + 1) * 128;

    // ---- schedule of 64-key tiles (the forward's) ----
    int ntiles = 0, e0 = 0, subs = 1, nqb_meta = 0;
    if (MODE == (int)Mode::kDense) {
        ntiles = (N + KT - 1) / KT;
    } else if (MODE == (int)Mode::kCausal) {
        ntiles = (min(N, q0 + G::BM) + KT - 1) / KT;
    } else {
        subs = a.block / KT;
        nqb_meta = (N + a.block - 1) / a.block;
        const int64_t r = meta_of(bh, a.H, a.Hkv, a.meta_heads) * nqb_meta + qt;   // BM == block for sparse launches
        int lo = ld_meta(a.row_ptr, r), hi_ = ld_meta(a.row_ptr, r + 1);
        lo = (int)min<int64_t>(max(lo, 0), a.nnz);
        hi_ = (int)min<int64_t>(max(hi_, lo), a.nnz);
        e0 = lo;
        ntiles = (hi_ - lo) * subs;
    }
    auto describe = [&](int it) -> KeyTile {
        KeyTile t;
        if (MODE == (int)Mode::kSparse) {
            const int e = e0 + it / subs;
            const int kb = ld_meta(a.col, e);
            const bool valid = kb >= 0 && kb < nqb_meta;
            t.kb0 = valid ? kb * a.block + (it % subs) * KT : 0;
            t.nlim = valid ? N : 0;
            t.causal = ((ld_meta_byte(a.flags, e) & 1) != 0) || (a.causal && t.kb0 + KT - 1 > q0);
        } else {
            t.kb0 = it * KT;
            t.nlim = N;
            t.causal = (MODE == (int)Mode::kCausal) && (t.kb0 + KT - 1 > q0);
        }
        t.masked = t.causal || (t.kb0 + KT > t.nlim);
        return t;
    };

    int k_row[G::PER_T], k_col[G::PER_T];
#pragma unroll
    for (int i = 0; i < G::PER_T; ++i) {
        const int byte = (w * G::PER_T + i) * 1024 + lane * 16;
        const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
        k_row[i] = r;
        k_col[i] = rt_swz<D>(r, p) * 8;
    }
    // scalar tile base plus fixed per-lane offsets, as in the dK/dV kernel
    unsigned k_boff[G::PER_T];
#pragma unroll
    for (int i = 0; i < G::PER_T; ++i) k_boff[i] = (unsigned)(2 * (k_row[i] * D + k_col[i]));
    const unsigned kl[3] = {lds_addr(sK0), lds_addr(sK1), lds_addr(sK2)};
    const unsigned vl[3] = {lds_addr(sV0), lds_addr(sV1), lds_addr(sV2)};
    const unsigned wl = __builtin_amdgcn_readfirstlane(w * G::PER_T * 1024);
    auto issue = [&](int kb0, int u) {
        if (kb0 + KT <= N) {
            const __bf16* kt = Kh + (int64_t)kb0 * D;
            const __bf16* vt = Vh + (int64_t)kb0 * D;
#pragma unroll
            for (int i = 0; i < G::PER_T; ++i) {
                dma16_at(kt, k_boff[i], kl[u] + wl + i * 1024);
                dma16_at(vt, k_boff[i], vl[u] + wl + i * 1024);
            }
        } else {
            const int rb = min(kb0, N - 1);   // clamped rows stay at or after rb
            const __bf16* kt = Kh + (int64_t)rb * D;
            const __bf16* vt = Vh + (int64_t)rb * D;
#pragma unroll
            for (int i = 0; i < G::PER_T; ++i) {
                const unsigned off = (unsigned)(2 * ((min(kb0 + k_row[i], N - 1) - rb) * D + k_col[i]));
                dma16_at(kt, off, kl[u] + wl + i * 1024);
                dma16_at(vt, off, vl[u] + wl + i * 1024);
            }
        }
    };

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};
    const float sl2 = a.scale_log2;

    if (ntiles > 0) {
        // this lane's query and dO rows: B operands of S^T = K Q^T, dP^T = V dO^T
        bf16x8 qf[D / 16], dof[D / 16];
        {
            const int row = min(qi, N - 1);
#pragma unroll
            for (int k = 0; k < D / 16; ++k) {
                qf[k] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)row * D + 16 * k + 8 * hi);
                dof[k] = *reinterpret_cast<const bf16x8*>(dOh + (int64_t)row * D + 16 * k + 8 * hi);
            }
        }
        float lse2 = __builtin_inff(), dval = 0.f;
        if (qi < N) {
            lse2 = Sh[(qi / BT) * 128 + (qi % BT)];
            dval = Sh[(qi / BT) * 128 + 64 + (qi % BT)];
        }
        wait_vmcnt<0>();
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < ntiles) issue(describe(s).kb0, s);

        auto compute = [&](const KeyTile& t, int u) {
            const unsigned char* bK = kbuf[u];
            const unsigned char* bV = vbuf[u];
#pragma unroll
            for (int c = 0; c < KT / 32; ++c) {
                // ---- S^T and dP^T: lane (l32, hi) gets key
                // kb0 + 32c + 8(v>>2) + 4hi + (v&3) of query qi in element v ----
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int k = 0; k < D / 16; ++k) {
                    const int off = rtl.off[k] + 32 * c * (2 * D);
                    const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(bK + off);
                    const bf16x8 vfr = *reinterpret_cast<const bf16x8*>(bV + off);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qf[k], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr, dof[k], dp, 0, 0, 0);
                }
                // masked scores become -inf (P = 0) in a block of their own, so
                // unmasked tiles pay nothing for it
                if (t.masked) {
                    // key j masked when j >= nlim or, causal, j > qi: one bound
                    const int lim = t.causal ? min(t.nlim - 1, qi) : t.nlim - 1;
                    const int r = lim - t.kb0 - 32 * c - 4 * hi;
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (8 * (v >> 2) + (v & 3) > r) s[v] = -__builtin_inff();
                }
                bf16x8 dsb[2];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[v], sl2, -lse2));
                    dsb[v >> 3][v & 7] = (__bf16)(p * (dp[v] - dval));
                }
                // ---- dQ^T += K^T dS^T over this block's two 16-key steps ----
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int g = 2 * c + tt;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const bf16x8 ka = tr_operand<D>(bK, trl, g, db);   // K^T, keys in dsb's order
                        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsb[tt], dqacc[db], 0, 0, 0);
                    }
                }
            }
        };

        auto tile = [&](int it, int u) {
            const int ahead = min(NS - 2, ntiles - 1 - it);
            if (ahead >= 1) wait_vmcnt<G::PER_W>();
            else wait_vmcnt<0>();
            barrier();
            const int un = (u + NS - 1) % NS;
            if (it + NS - 1 < ntiles) issue(describe(it + NS - 1).kb0, un);
            const KeyTile t = describe(it);
            if (!(t.causal && t.kb0 > q0w + 31)) compute(t, u);
        };
        for (int base = 0; base < ntiles; base += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u)
                if (base + u < ntiles) tile(base + u, u);
        }
    }

    // ---- epilogue: dQ = scale * (K^T dS^T)^T ----
    if (qi < N) {
        __bf16* dQr = static_cast<__bf16*>(a.dq) + (bh * N + qi) * (int64_t)D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 qv;
#pragma unroll
                for (int i = 0; i < 4; ++i) qv[i] = (__bf16)(dqacc[db][4 * j + i] * a.scale);
                *reinterpret_cast<bf16x4*>(dQr + 32 * db + 8 * j + 4 * hi) = qv;
            }
    }
}

// ---------------------------------------------------------------------------
// block-sparse dK/dV split: plan and ordered reduction
// ---------------------------------------------------------------------------

// The ordered reduction of split key tiles. A split key tile's partials sit in
// consecutive slots from its first; each of its RCH workgroups owns one chunk of
// the [dK | dV] block and adds the pieces' values in piece order (all loads
// issued first), so the result does not depend on scheduling. Workgroups are
// indexed by (slot, chunk); only a split tile's first slot (piece 0 in the
// extra list) does work.
template <int D, int BKV>
struct ReduceGeo {
    static constexpr int TILE = 2 * BKV * D;           // floats per slot: dK, then dV
    static constexpr int F = 2;                        // float4 per thread and piece
    static constexpr int RCH = TILE / (256 * 4 * F);   // workgroups per key tile
    static_assert(RCH * 256 * 4 * F == TILE, "chunking must cover the slot");
};

template <int D, int BKV>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a, int nkt) {
    using G = ReduceGeo<D, BKV>;
    const int64_t w = blockIdx.x / G::RCH;
    const int ch = blockIdx.x % G::RCH;
    const int32_t* ex = reinterpret_cast<const int32_t*>(a.extra);
    const int item0 = ld_meta(ex, 2 * w);
    if (item0 < 0 || ld_meta(ex, 2 * w + 1) != 0) return;
    const int64_t item = item0;
    const int np = plan_at(a, item).y;   // its first slot is w
    const int64_t kvbh = item / nkt;
    const int kb0 = (int)(item % nkt) * BKV;
    const float* base = a.part + w * G::TILE;
    float4 x[kMaxPieces][G::F];
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p)
#pragma unroll
        for (int i = 0; i < G::F; ++i) {
            const int e = ((ch * G::F + i) * 256 + threadIdx.x) * 4;
            x[p][i] = p < np ? *reinterpret_cast<const float4*>(base + (int64_t)p * G::TILE + e)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
    for (int i = 0; i < G::F; ++i) {
        float4 sum = x[0][i];
#pragma unroll
        for (int p = 1; p < kMaxPieces; ++p) {
            sum.x += x[p][i].x; sum.y += x[p][i].y; sum.z += x[p][i].z; sum.w += x[p][i].w;
        }
        const int e = ((ch * G::F + i) * 256 + threadIdx.x) * 4;
        const bool is_k = e < BKV * D;
        const int r = is_k ? e : e - BKV * D;
        const int key = r / D, c = r % D;
        if (kb0 + key >= a.N) continue;
        const float m = is_k ? -a.scale : 1.f;   // the partial dK sums hold -dK / scale
        const bf16x4 out = {(__bf16)(sum.x * m), (__bf16)(sum.y * m), (__bf16)(sum.z * m), (__bf16)(sum.w * m)};
        __bf16* dst = static_cast<__bf16*>(is_k ? a.dk : a.dv);
        *reinterpret_cast<bf16x4*>(dst + (kvbh * a.N + kb0 + key) * (int64_t)D + c) = out;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int D, int NW, int MODE, bool PAIRED = (D == 128)>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream) {
    const int64_t nkt = (a.N + DkdvGeo<D, NW, PAIRED>::BKV - 1) / DkdvGeo<D, NW, PAIRED>::BKV;
    const int64_t bhkv = a.BH / (a.H / a.Hkv);
    const int64_t extra = MODE == (int)Mode::kSparse ? a.part_slots : 0;   // workgroups for the extra pieces
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, MODE, PAIRED>), dim3((unsigned)(extra + nkt * bhkv)), dim3(64 * NW), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int NW, int NS, int MODE, int KT = BT>
hipError_t launch_dq(const BwdArgs& a, hipStream_t stream) {
    const int64_t nqt = (a.N + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, NS, MODE, KT>), dim3((unsigned)(nqt * a.BH)), dim3(64 * NW), 0, stream,
                       a);
    return hipGetLastError();
}

template <int D, int BKV>
hipError_t launch_reduce(const BwdArgs& a, int nkt, hipStream_t stream) {
    if (a.part_slots == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_reduce_kernel<D, BKV>), dim3((unsigned)(a.part_slots * ReduceGeo<D, BKV>::RCH)), dim3(256),
                       0, stream, a, nkt);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, Mode mode, hipStream_t stream) {
    const int nblk = a.npad / BT;
    // block-sparse: the split plan rides in the statistics launch (one more
    // grid column whose row 0 computes it)
    const int nkt_sparse = mode == Mode::kSparse ? (a.N + a.block - 1) / a.block : 0;
    const int64_t items = (int64_t)nkt_sparse * (a.BH / (a.H / a.Hkv));
    const unsigned rows = (unsigned)(a.BH < 65535 ? a.BH : 65535);   // grid rows stride over the heads
    if (mode == Mode::kSparse)
        hipLaunchKernelGGL((bwd_stats_kernel<D, true>), dim3((unsigned)(nblk + 2), rows), dim3(256), 0,
                           stream, a, nblk, nkt_sparse, items);
    else
        hipLaunchKernelGGL((bwd_stats_kernel<D, false>), dim3((unsigned)(nblk + 1), rows), dim3(256), 0,
                           stream, a, nblk, 0, (int64_t)0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dK/dV: 128 keys per workgroup (one key block of a sparse pattern; 64 for
    // 64-key blocks): 4 wave pairs for d = 128, 4 single waves for d = 64;
    // dQ: the forward's shapes (8 waves and 3 stages dense/causal,
    // one query block and 2 stages block-sparse).
    switch (mode) {
        case Mode::kDense:
            e = launch_dkdv<D, D == 64 ? 4 : 8, (int)Mode::kDense>(a, stream);
            return e != hipSuccess ? e : launch_dq<D, 8, 3, (int)Mode::kDense>(a, stream);
        case Mode::kCausal:
            e = launch_dkdv<D, D == 64 ? 4 : 8, (int)Mode::kCausal>(a, stream);
            return e != hipSuccess ? e : launch_dq<D, 8, 3, (int)Mode::kCausal>(a, stream);
        case Mode::kSparse: {
            // dK/dV (pieces of long key-tile lists write partials), the ordered
            // reduction of split key tiles, dQ
            if (a.block == 128) {
                e = launch_dkdv<D, D == 64 ? 4 : 8, (int)Mode::kSparse>(a, stream);
                if (e == hipSuccess) e = launch_reduce<D, 128>(a, nkt_sparse, stream);
                return e != hipSuccess ? e : launch_dq<D, 4, 2, (int)Mode::kSparse>(a, stream);
            }
            e = launch_dkdv<D, D == 64 ? 2 : 4, (int)Mode::kSparse>(a, stream);
            if (e == hipSuccess) e = launch_reduce<D, 64>(a, nkt_sparse, stream);
            // dQ of 64-key blocks at d = 128 in 32-key steps: 32 KiB of LDS per
            // workgroup, so two waves per SIMD fit (64-key steps: one)
            return e != hipSuccess ? e : launch_dq<D, 2, 2, (int)Mode::kSparse, D == 128 ? 32 : BT>(a, stream);
        }
        case Mode::kRange: break;   // no backward for key-range launches
    }
    return hipErrorInvalidValue;
}

}  // namespace

int64_t bwd_workspace_bytes(int64_t BH, int64_t N) {
    const int64_t npad = vt_padded_keys(N);
    return BH * (npad / BT + 1) * 128 * 4;   // row statistics
}

void bwd_workspace_carve(BwdArgs& a, void* ws) {
    a.npad = (int)vt_padded_keys(a.N);
    a.stats = static_cast<float*>(ws);
}

namespace {
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
}  // namespace

int64_t bwd_sparse_workspace_base(int64_t BH, int64_t BHkv, int64_t N, int64_t block) {
    const int64_t nkt = (N + block - 1) / block;
    return align256(bwd_workspace_bytes(BH, N)) + align256(BHkv * nkt * (int64_t)sizeof(int2));
}

int64_t bwd_sparse_slot_bytes(int64_t block, int64_t d) { return 2 * block * d * 4; }

int64_t bwd_sparse_slots(const int32_t* t_row_ptr, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t block,
                         int64_t meta_heads) {
    const int64_t nkt = (N + block - 1) / block, group = H / Hkv, subs = block / BT;
    const int64_t nnz = t_row_ptr[meta_heads * nkt];
    int64_t slots = 0;
    for (int64_t kvbh = 0; kvbh < B * Hkv; ++kvbh) {
        const int64_t bh0 = (kvbh / Hkv) * H + (kvbh % Hkv) * group;
        for (int64_t kt = 0; kt < nkt; ++kt) {
            int64_t tiles = 0;
            for (int64_t gi = 0; gi < group; ++gi) {
                const int64_t r = meta_of(bh0 + gi, (int)H, (int)Hkv, (int)meta_heads) * nkt + kt;
                int64_t lo = std::min<int64_t>(std::max<int64_t>(t_row_ptr[r], 0), nnz);
                int64_t hi = std::min<int64_t>(std::max<int64_t>(t_row_ptr[r + 1], lo), nnz);
                tiles += (hi - lo) * subs;
            }
            const int np = pieces_of((int)std::min<int64_t>(tiles, INT32_MAX));
            if (np > 1) slots += np;
        }
    }
    return slots > kMaxSlots ? 0 : slots;   // beyond the cap the call splits nothing
}

void bwd_sparse_workspace_carve(BwdArgs& a, void* ws, int64_t ws_bytes) {
    bwd_workspace_carve(a, ws);
    const int64_t group = a.H / a.Hkv, BHkv = a.BH / group;
    unsigned char* p = static_cast<unsigned char*>(ws);
    a.plan = reinterpret_cast<int2*>(p + align256(bwd_workspace_bytes(a.BH, a.N)));
    const int64_t base = bwd_sparse_workspace_base(a.BH, BHkv, a.N, a.block);
    const int64_t per_slot = bwd_sparse_slot_bytes(a.block, a.d) + (int64_t)sizeof(int2);
    // no more slots than key tiles times pieces, and at most kMaxSlots, so the
    // dK/dV grid (slots plus key tiles) and the reduction grid (slots times its
    // chunks) stay far inside 32-bit work-item counts
    const int64_t items = (a.N + a.block - 1) / a.block * BHkv;
    a.part_slots = std::max<int64_t>(0, ws_bytes - base - 256) / per_slot;
    a.part_slots = std::min<int64_t>({a.part_slots, items * kMaxPieces, kMaxSlots});
    a.extra = reinterpret_cast<int2*>(p + base);
    a.part = reinterpret_cast<float*>(p + base + align256(a.part_slots * (int64_t)sizeof(int2)));
}

hipError_t launch_bwd_bf16(const BwdArgs& a, Mode mode, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, mode, stream);
    return launch_d<128>(a, mode, stream);
}

}  // namespace bsattn
