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
//   * NW waves x 32 query rows.  Each wave computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16, so a lane holds 16 scores of ONE query row per
//     32-key block: the row max and row sum stay inside the lane plus one
//     exchange with lane l^32 (v_permlane32_swap), no LDS reductions.
//   * The S^T accumulator converts in place to the B operand of O^T += V^T P^T.
//     The key order inside each 16-key MFMA step is permuted to the keys a lane
//     already holds.  The V^T operand is read from a row-major V tile with the
//     gfx950 transposing LDS load (ds_read_b64_tr_b16: two per operand, each
//     giving a lane 4 consecutive keys of its dimension), so V is used in
//     place and no transpose pass over V is needed.  A caller that reuses V
//     can also prepare V^T once in the permuted order and have the kernel read
//     plain 16-byte V^T rows instead.
//   * K and V tiles go from global memory straight into LDS
//     (global_load_lds_dwordx4: no VGPR staging, no LDS store instructions),
//     NSTAGE tiles in flight, 16-byte chunks XOR-swizzled per row so the
//     fragment reads are bank-conflict free.
//   * Logits are handled in base-2 units (scale * log2 e folded into one FMA
//     before v_exp_f32).  The reference value m of a row (the running max of
//     the pages' update) is not recomputed tile by tile: the exponentials of a
//     tile are taken against the current m and checked afterwards.  If every
//     lane's sum over the tile is finite and at most 2^64, no exponential can
//     have overflowed and the tile is folded in as is -- exact in real
//     arithmetic for any m, since A and l share it.  Otherwise, and while a row
//     has no m yet (its first tile), the tile's row max raises m, the state is
//     rescaled by exp2(m_old - m), and the tile's exponentials are recomputed.
//     The common path thus has no per-tile max reduction (a serial chain of
//     dependent vector operations) and almost never rescales the accumulator.
//   * The K fragments of the score product and the V fragments of the PV
//     product are read from LDS four MFMAs ahead of their use, so the matrix
//     core does not wait for each read.
//   * Causal: key tiles wholly in the future are never visited, a wave skips
//     the tiles that lie past all of its rows, and only tiles that cross the
//     diagonal get the element mask.  Block-sparse: the tile loop runs over the
//     canonical list of active key blocks of the query block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <cstring>

#include "fwd_common.h"
#include "gfx950_util.h"

namespace bsattn {
namespace {

constexpr int kBN = 64;                // keys per tile step (32 for 64-key sparse blocks at d = 128)
constexpr int kVtKeys = 64;            // keys per workgroup of the V^T pass
constexpr float kSumMax = 0x1p64f;     // largest per-lane tile sum folded in without a rescale
constexpr int kKAhead = 4;             // K fragment reads in flight ahead of their MFMAs
constexpr int kVAhead = 4;             // V fragment reads in flight ahead of their MFMAs
constexpr float kLn2 = 0.69314718055994530942f;

// Where the V operand of a tile comes from:
//   kVsTr: the V tile copied straight into LDS row-major, like K, and read
//          with the transposing LDS load ds_read_b64_tr_b16 (V in place);
//   kVsT:  a V^T tile (written beforehand by the transpose pass) copied
//          straight into LDS and read with plain 16-byte LDS loads.
enum VSrc : int { kVsTr = 0, kVsT = 1 };

template <int D, int NW, int NS, int VSRC, int BN_ = kBN>
struct Geo {
    static constexpr int BN = BN_;                   // keys per tile step
    static constexpr int NT = 64 * NW;               // threads per workgroup
    static constexpr int BM = 32 * NW;               // query rows per workgroup
    static constexpr int K_BYTES = BN * D * 2;       // K tile: BN rows of D bf16
    static constexpr int V_BYTES = D * BN * 2;       // V^T tile (D rows of BN) or V tile (BN rows of D)
    static constexpr int K_PER_W = K_BYTES / 1024 / NW;   // 1 KiB direct-to-LDS loads per wave
    static constexpr int V_PER_W = V_BYTES / 1024 / NW;
    static constexpr int PER_W = K_PER_W + V_PER_W;
    static_assert(K_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0, "tile must split over waves");
    static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
    static_assert((NS - 2) * PER_W < 64, "vmcnt range");
};

// One 64-key tile of the schedule.
struct TileDesc {
    int kb0;       // first key
    int nlim;      // keys j >= nlim are masked (N; 0 for an invalid metadata entry)
    int causal;    // element mask j <= i applies
    int masked;    // any element mask needed (uniform over the workgroup)
};

template <int D, int NW, int NS, int MODE, int VSRC, int BN = kBN>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(FwdArgs a) {
    using G = Geo<D, NW, NS, VSRC, BN>;
    constexpr bool VTR = VSRC == kVsTr;
    // One array per stage: distinct objects let the compiler see that a tile in
    // flight never aliases the tile being read.
    constexpr int KB2 = NS > 2 ? G::K_BYTES : 16, KB3 = NS > 3 ? G::K_BYTES : 16;
    constexpr int VB2 = NS > 2 ? G::V_BYTES : 16, VB3 = NS > 3 ? G::V_BYTES : 16;
    __shared__ __attribute__((aligned(1024))) unsigned char sK0[G::K_BYTES], sK1[G::K_BYTES], sK2[KB2], sK3[KB3];
    __shared__ __attribute__((aligned(1024))) unsigned char sV0[G::V_BYTES], sV1[G::V_BYTES], sV2[VB2], sV3[VB3];
    unsigned char* const kbuf[4] = {sK0, sK1, sK2, sK3};
    unsigned char* const vbuf[4] = {sV0, sV1, sV2, sV3};
    const unsigned kl[4] = {lds_addr(sK0), lds_addr(sK1), lds_addr(sK2), lds_addr(sK3)};
    const unsigned vl[4] = {lds_addr(sV0), lds_addr(sV1), lds_addr(sV2), lds_addr(sV3)};

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const TrLane<D> trl = tr_lane<D>(lane);   // transposing-read offsets of the V^T operand
    // Byte offsets of this lane's K fragments (row l32, chunk 2k + hi) in a K
    // tile; the swizzle depends on the low row bits only, so the second
    // 32-key block is at a constant distance.  With the stage buffers inside
    // the 64 KiB the LDS instructions' offset field reaches, every fragment
    // read is one register plus an immediate: no address arithmetic per tile.
    int koff[D / 16];
#pragma unroll
    for (int k = 0; k < D / 16; ++k) koff[k] = l32 * (2 * D) + k_swz<D>(l32, 2 * k + hi) * 16;
    constexpr bool RANGE = MODE == (int)Mode::kRange;
    const int N = a.N;                   // query rows
    const int NK = RANGE ? a.Nk : N;     // keys
    const int nqt = (N + G::BM - 1) / G::BM;
    const int nsplit = RANGE ? a.nsplit : 1;
    const int64_t total = (int64_t)nqt * a.BH * nsplit;
    // The query tiles of one (head, split) run on one XCD: they share its K/V.
    // Causal tiles differ in cost by up to N / BM times: the costliest tiles
    // of all the XCD's heads go first.  Block-sparse tiles cost about the same
    // (a few blocks each): head by head, which keeps one head's K/V hot in L2.
    int64_t rest;
    int qt;
    // folded causal schedule: jobs (head, query tile) of this workgroup
    int njobs = 1;
    int64_t jhead[2] = {0, 0};
    int jqt[2] = {0, 0};
    const bool FOLD = MODE == (int)Mode::kCausal && a.fold_slots > 0;
    if (FOLD) {
        // per XCD: Tx tiles ranked heavy first (rank-major, head-minor), Sx
        // slots; the Tx - Sx lightest ranks ride with the heaviest, the
        // singles alternate heavy and light halves so each CU's three
        // workgroups add up to the same work
        const int x = blockIdx.x % 8, l = blockIdx.x / 8;
        const int Tx = (int)(total / 8), Sx = a.fold_slots / 8, Px = Tx - Sx;
        const int hx = Tx / nqt;
        auto job_of = [&](int r, int k) {
            jhead[k] = (int64_t)x * hx + r % hx;
            jqt[k] = nqt - 1 - r / hx;
        };
        if (l < Px) {
            job_of(l, 0);
            job_of(Tx - 1 - l, 1);
            njobs = 2;
        } else {
            const int i = l - Px, nsing = Tx - 2 * Px, h = (nsing + 1) / 2;
            job_of(i < h ? Px + i : Tx - Px - 1 - (i - h), 0);
        }
        rest = jhead[0];
        qt = jqt[0];
    } else if (MODE == (int)Mode::kCausal || (RANGE && a.causal)) {
        rank_major_order(blockIdx.x, total, nqt, rest, qt);
        qt = nqt - 1 - qt;
    } else {
        const int64_t ord = xcd_tile_order(blockIdx.x, total);
        rest = ord / nqt;
        qt = (int)(ord % nqt);
        if (MODE == (int)Mode::kSparse) qt = nqt - 1 - qt;
    }
    // The workgroup's query tiles, one after the other (two only in a folded
    // causal launch); the loop body keeps the indentation of the kernel.
    for (int job = 0; job < njobs; ++job) {
    if (FOLD) {
        rest = jhead[job];
        qt = jqt[job];
        if (job > 0) barrier();   // every wave is done with the stage buffers
    }
    const int split = (int)(rest % nsplit);
    const int64_t bh = rest / nsplit;
    const int q0 = qt * G::BM;
    const int q0w = q0 + 32 * w;
    const int qi = q0w + l32;  // this lane's query row
    // Causal limits in key indices: key j is allowed for row i when j <= i +
    // shift (shift = q_off - k_off for key-range launches, else 0).
    const int64_t shift = RANGE ? a.q_off - a.k_off : 0;
    auto diag_of = [&](int64_t row) { return (int)min<int64_t>(max<int64_t>(row + shift, -1), (int64_t)NK); };
    const int qdiag = diag_of(qi);           // last key this lane's row may see
    const int wdiag = diag_of(q0w + 31);     // last key any row of this wave may see

    const int64_t kvh = kv_head_of(bh, a.H, a.Hkv);
    const __bf16* Qh = static_cast<const __bf16*>(a.q) + bh * (int64_t)N * D;
    const __bf16* Kh = static_cast<const __bf16*>(a.k) + kvh * (int64_t)NK * D;
    const __bf16* Vth = VTR ? nullptr : static_cast<const __bf16*>(a.vt) + kvh * (int64_t)a.npad * D;
    const __bf16* Vh = VTR ? static_cast<const __bf16*>(a.v) + kvh * (int64_t)NK * D : nullptr;

    // Query fragments (B operand of S^T = K Q^T): dims 16k+8hi..+7 of row qi,
    // loaded before the block-sparse schedule is read so the two latencies
    // overlap.
    bf16x8 qf[D / 16];
    {
        const int qrow = min(qi, N - 1);
#pragma unroll
        for (int k = 0; k < D / 16; ++k)
            qf[k] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qrow * D + 16 * k + 8 * hi);
    }

    // ---- tile schedule ----
    int ntiles = 0, e0 = 0, subs = 1, nqb_meta = 0, kv_lo = 0, kv_hi = 0;
    if (MODE == (int)Mode::kDense) {
        ntiles = (N + BN - 1) / BN;
    } else if (MODE == (int)Mode::kCausal) {
        ntiles = (min(N, q0 + G::BM) + BN - 1) / BN;
    } else if (RANGE) {
        kv_lo = split * a.kv_chunk;
        kv_hi = min(NK, kv_lo + a.kv_chunk);
        // causal: keys past the last row's diagonal are never visited
        const int vis = a.causal ? min(kv_hi, diag_of(q0 + G::BM - 1) + 1) : kv_hi;
        ntiles = vis > kv_lo ? (vis - kv_lo + BN - 1) / BN : 0;
    } else {
        subs = a.block / BN;
        nqb_meta = (N + a.block - 1) / a.block;
        const int64_t r = meta_of(bh, a.H, a.Hkv, a.meta_heads) * nqb_meta + qt;   // BM == block for sparse launches
        int lo = ld_meta(a.row_ptr, r), hi_ = ld_meta(a.row_ptr, r + 1);
        lo = (int)min<int64_t>(max(lo, 0), a.nnz);
        hi_ = (int)min<int64_t>(max(hi_, lo), a.nnz);
        e0 = lo;
        ntiles = (hi_ - lo) * subs;
    }
    auto describe = [&](int it) -> TileDesc {
        TileDesc t;
        if (MODE == (int)Mode::kSparse) {
            const int e = e0 + it / subs;
            const int kb = ld_meta(a.col, e);
            const bool valid = kb >= 0 && kb < nqb_meta;
            t.kb0 = valid ? kb * a.block + (it % subs) * BN : 0;
            t.nlim = valid ? N : 0;
            // the flag comes from canonical metadata; the geometric test keeps a
            // causal launch correct even for lists that were not pruned
            t.causal = ((ld_meta_byte(a.flags, e) & 1) != 0) || (a.causal && t.kb0 + BN - 1 > q0);
        } else if (RANGE) {
            t.kb0 = kv_lo + it * BN;
            t.nlim = kv_hi;
            t.causal = a.causal && (t.kb0 + BN - 1 > diag_of(q0));
        } else {
            t.kb0 = it * BN;
            t.nlim = N;
            t.causal = (MODE == (int)Mode::kCausal) && (t.kb0 + BN - 1 > q0);
        }
        t.masked = t.causal || (t.kb0 + BN > t.nlim);
        return t;
    };

    // Source offsets of this wave's direct-to-LDS loads: lane i of load g fills
    // bytes [1024 g + 16 i, +16) of the tile, i.e. row r, physical chunk p,
    // with logical chunk swz(r, p) of that row.
    int k_row[G::K_PER_W], k_col[G::K_PER_W], v_off[G::V_PER_W > 0 ? G::V_PER_W : 1];
    int64_t vt_off[VTR ? 1 : G::V_PER_W];   // V^T source offsets: dimension row d * npad can pass 2^31
    int v_row[VTR ? G::V_PER_W : 1];
#pragma unroll
    for (int i = 0; i < G::K_PER_W; ++i) {
        const int byte = (w * G::K_PER_W + i) * 1024 + lane * 16;
        const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
        k_row[i] = r;
        k_col[i] = k_swz<D>(r, p) * 8;
    }
#pragma unroll
    for (int i = 0; i < G::V_PER_W; ++i) {
        const int byte = (w * G::V_PER_W + i) * 1024 + lane * 16;
        if constexpr (VTR) {   // row-major V tile: offset of the key row's chunk; the row goes in v_row
            const int r = byte / (2 * D), p = (byte % (2 * D)) / 16;
            v_row[i] = r;
            v_off[i] = rt_swz<D>(r, p) * 8;
        } else {
            const int d = byte / (2 * BN), p = (byte % (2 * BN)) / 16;
            vt_off[i] = (int64_t)d * a.npad + v_swz<BN>(d, p) * 8;
        }
    }
    // Row-major K and V tiles: byte offsets inside the tile, fixed for the
    // whole loop, from a tile base that moves in scalar registers.  A tile
    // that reaches past the last key clamps its rows to that key instead.
    unsigned k_boff[G::K_PER_W], v_boff[VTR ? G::V_PER_W : 1];
#pragma unroll
    for (int i = 0; i < G::K_PER_W; ++i) k_boff[i] = (unsigned)(2 * (k_row[i] * D + k_col[i]));
#pragma unroll
    for (int i = 0; i < (VTR ? G::V_PER_W : 0); ++i) v_boff[i] = (unsigned)(2 * (v_row[i] * D + v_off[i]));
    const unsigned wk = __builtin_amdgcn_readfirstlane(w * G::K_PER_W * 1024);   // this wave's part of a tile
    const unsigned wv = __builtin_amdgcn_readfirstlane(w * G::V_PER_W * 1024);
    auto issue_tile = [&](int kb0, int u) {
        if (kb0 + BN <= NK) {
            const __bf16* kt = Kh + (int64_t)kb0 * D;
#pragma unroll
            for (int i = 0; i < G::K_PER_W; ++i) dma16_at(kt, k_boff[i], kl[u] + wk + i * 1024);
            if constexpr (VTR) {
                const __bf16* vt = Vh + (int64_t)kb0 * D;
#pragma unroll
                for (int i = 0; i < G::V_PER_W; ++i) dma16_at(vt, v_boff[i], vl[u] + wv + i * 1024);
            }
        } else {
            const int rb = min(kb0, NK - 1);   // rows clamped to NK - 1 stay at or after rb
            const __bf16* kt = Kh + (int64_t)rb * D;
#pragma unroll
            for (int i = 0; i < G::K_PER_W; ++i) {
                const int key = min(kb0 + k_row[i], NK - 1);
                dma16_at(kt, (unsigned)(2 * ((key - rb) * D + k_col[i])), kl[u] + wk + i * 1024);
            }
            if constexpr (VTR) {
                const __bf16* vt = Vh + (int64_t)rb * D;
#pragma unroll
                for (int i = 0; i < G::V_PER_W; ++i) {
                    const int key = min(kb0 + v_row[i], NK - 1);
                    dma16_at(vt, (unsigned)(2 * ((key - rb) * D + v_off[i])), vl[u] + wv + i * 1024);
                }
            }
        }
        if constexpr (!VTR) {
#pragma unroll
            for (int i = 0; i < G::V_PER_W; ++i)
                dma16(Vth + kb0 + vt_off[i], vbuf[u] + (w * G::V_PER_W + i) * 1024);
        }
    };
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -__builtin_inff();   // reference value m of the row, base-2 units (see the file comment)
    float ell = 0.f;                   // this lane's share of the denominator
    const float sl2 = a.scale_log2;

    if (ntiles == 0) wait_vmcnt<0>();   // nothing to compute: let the query loads land
    if (ntiles > 0) {
        // The first tiles' loads are issued behind the Q loads, so the two
        // latencies overlap.  Loads complete in issue order: the wait for tile
        // 0 below (at most the later tiles' loads outstanding) also covers Q.
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < ntiles) issue_tile(describe(s).kb0, s);

        // One tile's math for this wave, in three steps: scores (and masks),
        // online softmax, PV.
        f32x16 s[BN / 32];
        bf16x8 pf[BN / 16];
        auto scores = [&](const TileDesc& t, const unsigned char* bK) {
            // ---- S^T: lane (l32, hi) gets, in s[c][v], the score of query l32
            // and key kb0 + 32c + 8(v>>2) + 4hi + (v&3) ----
            // fragment f: 32-key block c = f % NC, chunk f / NC -- the blocks'
            // accumulation chains alternate, so consecutive MFMAs are independent
            // (each chain still adds its chunks in order)
            constexpr int NC = BN / 32, NF = NC * (D / 16);
            auto kfrag = [&](int f) {
                return *reinterpret_cast<const bf16x8*>(bK + koff[f / NC] + 32 * (f % NC) * (2 * D));
            };
            bf16x8 kfr[NF];
#pragma unroll
            for (int f = 0; f < kKAhead; ++f) kfr[f] = kfrag(f);
#pragma unroll
            for (int c = 0; c < NC; ++c) s[c] = f32x16{};
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                if (f + kKAhead < NF) kfr[f + kKAhead] = kfrag(f + kKAhead);
                s[f % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[f], qf[f / NC], s[f % NC], 0, 0, 0);
            }
            // keep the reads kKAhead MFMAs ahead (DS reads: 0x100, MFMA: 0x008)
            __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
            for (int f = 0; f < NF - kKAhead; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
            if (t.masked) {
                // key j is masked when j >= nlim or, causal, j > qdiag: one bound
                // lim; element (c, v) holds j = kb0 + 4hi + (32c + 8(v>>2) + (v&3)),
                // so each element is one compare of a constant with r
                const int lim = t.causal ? min(t.nlim - 1, qdiag) : t.nlim - 1;
                const int r = lim - t.kb0 - 4 * hi;
#pragma unroll
                for (int c = 0; c < BN / 32; ++c)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        s[c][v] = 32 * c + 8 * (v >> 2) + (v & 3) > r ? -__builtin_inff() : s[c][v];
            }
        };
        auto softmax = [&]() {
            // ---- online softmax ----
            // P rounds to bf16 for the PV product; the denominator sums the fp32
            // values so LSE keeps fp32 accuracy even for rows with few keys.
            float ts[8];
            auto exps = [&](float mu) {
#pragma unroll
                for (int g = 0; g < BN / 16; ++g) {
                    const int c = g >> 1, t8 = (g & 1) * 8;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][t8 + i], sl2, -mu));
                        ts[i] = g == 0 ? p : ts[i] + p;
                        pf[g][i] = (__bf16)p;
                    }
                }
                return ((ts[0] + ts[1]) + (ts[2] + ts[3])) + ((ts[4] + ts[5]) + (ts[6] + ts[7]));
            };
            // Common path: the exponentials against the row's current m,
            // checked afterwards (see the file comment).
            float tsum = 0.f;
            bool redo = __builtin_amdgcn_ballot_w64(m_run == -__builtin_inff()) != 0;
            if (!redo) {
                tsum = exps(m_run);
                redo = __builtin_amdgcn_ballot_w64(!(tsum <= kSumMax)) != 0;
            }
            if (redo) {   // raise m to the tile's row max, rescale, recompute
                float mx = -__builtin_inff();
#pragma unroll
                for (int c = 0; c < BN / 32; ++c)
#pragma unroll
                    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[c][v]);
                mx = xor32_max(mx);
                const float mt = mx * sl2;
                const bool upd = mt > m_run;
                if (__builtin_amdgcn_ballot_w64(upd) != 0) {
                    const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
                    m_run = upd ? mt : m_run;
                    ell *= alpha;
#pragma unroll
                    for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
                }
                tsum = exps((m_run == -__builtin_inff()) ? 0.f : m_run);
            }
            ell += tsum;
        };
        auto pv = [&](const unsigned char* bV) {
            // ---- O^T += V^T P^T ----
            // fragment f: 16-key group g = f / (D/32), dimension block db = f % (D/32);
            // read kVAhead MFMAs ahead of its use, like the K fragments
            constexpr int NV = (BN / 16) * (D / 32);
            constexpr int RD = VTR ? 2 : 1;            // LDS reads per fragment
            auto vfrag = [&](int f) {
                const int g = f / (D / 32), db = f % (D / 32);
                if constexpr (VTR) {
                    return tr_operand<D>(bV, trl, g, db);   // keys in the order pf[g] holds them
                } else {
                    const int d = 32 * db + l32;
                    return *reinterpret_cast<const bf16x8*>(bV + d * (2 * BN) + v_swz<BN>(d, 2 * g + hi) * 16);
                }
            };
            bf16x8 vfr[NV];
#pragma unroll
            for (int f = 0; f < kVAhead; ++f) vfr[f] = vfrag(f);
#pragma unroll
            for (int f = 0; f < NV; ++f) {
                if (f + kVAhead < NV) vfr[f + kVAhead] = vfrag(f + kVAhead);
                oacc[f % (D / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[f], pf[f / (D / 32)],
                                                                           oacc[f % (D / 32)], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, RD * kVAhead, 0);
#pragma unroll
            for (int f = 0; f < NV - kVAhead; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 0);
        };
        // Tile it, in stage buffer u = it % NS: wait for its loads, barrier
        // (every wave's loads have landed and every wave is done with tile
        // it-1), refill the buffer of tile it-1 with tile it+NS-1, compute.
        auto tile = [&](int it, int u) {
            const int ahead = min(NS - 2, ntiles - 1 - it);   // tiles issued after this one
            if (ahead >= 2) wait_vmcnt<2 * G::PER_W>();
            else if (ahead == 1) wait_vmcnt<G::PER_W>();
            else wait_vmcnt<0>();
            barrier();
            const int un = (u + NS - 1) % NS;
            if (it + NS - 1 < ntiles) issue_tile(describe(it + NS - 1).kb0, un);
            const TileDesc t = describe(it);
            // a wave whose rows all precede the tile skips its math
            if (!(t.causal && t.kb0 > wdiag)) {
                scores(t, kbuf[u]);
                softmax();
                pv(vbuf[u]);
            }
        };

        for (int base = 0; base < ntiles; base += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u)
                if (base + u < ntiles) tile(base + u, u);
        }
    }

    // ---- epilogue: O = A / l, LSE = (m + log2 l) * ln 2 ----
    const float l_tot = xor32_sum(ell);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (RANGE) {   // normalised fp32 partial state of this split
        if (qi < N) {
            const int64_t row = ((int64_t)split * a.BH + bh) * N + qi;
            float* Or = a.o_part + row * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float4 ov;
                    ov.x = oacc[db][4 * j + 0] * inv;
                    ov.y = oacc[db][4 * j + 1] * inv;
                    ov.z = oacc[db][4 * j + 2] * inv;
                    ov.w = oacc[db][4 * j + 3] * inv;
                    *reinterpret_cast<float4*>(Or + 32 * db + 8 * j + 4 * hi) = ov;
                }
            if (hi == 0) a.lse_part[row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        }
        continue;
    }
    if (qi < N) {
        __bf16* Oh = static_cast<__bf16*>(a.o) + bh * (int64_t)N * D + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[db][4 * j + i] * inv);
                *reinterpret_cast<bf16x4*>(Oh + 32 * db + 8 * j + 4 * hi) = ov;
            }
        if (hi == 0) {
            a.lse[bh * (int64_t)N + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        }
    }
    }   // query tiles of the workgroup
}

// V [BH][N][D] -> V^T [BH][D][npad].  Inside each 16-key group, slot 8h + w of
// a row holds key 4h + (w & 3) + 8 (w >> 2): the keys that lane half h owns in
// the S^T layout, so one 16-byte chunk is one MFMA operand.  Keys >= N are 0.
// One workgroup per (64-key block, b*h).
template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(const __bf16* __restrict__ v, __bf16* __restrict__ vt,
                                                           int N, int npad) {
    __shared__ __bf16 tile[kVtKeys][D + 2];
    const int kb0 = blockIdx.x * kVtKeys;
    const int64_t bh = blockIdx.y;
    const __bf16* src = v + bh * (int64_t)N * D;
    for (int c = threadIdx.x; c < kVtKeys * D / 8; c += 256) {
        const int r = c / (D / 8), ch = c % (D / 8);
        const int key = kb0 + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < N) x = *reinterpret_cast<const u32x4*>(src + (int64_t)key * D + 8 * ch);
        const __bf16* xs = reinterpret_cast<const __bf16*>(&x);
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[r][8 * ch + i] = xs[i];
    }
    __syncthreads();
    __bf16* dst = vt + bh * (int64_t)npad * D;
    for (int c = threadIdx.x; c < D * (kVtKeys / 8); c += 256) {
        const int d = c / (kVtKeys / 8), ch = c % (kVtKeys / 8);
        bf16x8 out;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int slot = 8 * ch + i;
            const int grp = slot >> 4, h = (slot >> 3) & 1, ww = slot & 7;
            out[i] = tile[16 * grp + 4 * h + (ww & 3) + 8 * (ww >> 2)][d];
        }
        *reinterpret_cast<bf16x8*>(dst + (int64_t)d * npad + kb0 + 8 * ch) = out;
    }
}

template <int D, int NW, int NS, int MODE, int VSRC, int BN = kBN>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    using G = Geo<D, NW, NS, VSRC, BN>;
    const int64_t nqt = (a.N + G::BM - 1) / G::BM;
    const int64_t grid = (MODE == (int)Mode::kCausal && a.fold_slots > 0) ? a.fold_slots
                         : nqt * a.BH * (MODE == (int)Mode::kRange ? a.nsplit : 1);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NS, MODE, VSRC, BN>), dim3((unsigned)grid), dim3(G::NT), 0, stream,
                       a);
    return hipGetLastError();
}

// V^T from the caller's workspace when a.vt is set, else V read in place.
template <int D, int NW, int NS, int MODE, int BN = kBN>
hipError_t launch_v(const FwdArgs& a, hipStream_t stream) {
    if (a.vt != nullptr) return launch<D, NW, NS, MODE, kVsT, BN>(a, stream);
    return launch<D, NW, NS, MODE, kVsTr, BN>(a, stream);
}

// Workgroups of the 4-wave causal instance (head dimension D, V source vt)
// that the current device holds at once: CUs x resident workgroups per CU,
// asked once per device (-1, and asked again on the next call, when the
// runtime cannot say).
template <int D>
int resident_slots(int vt) {
    static int cached[2][64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    int& c = cached[vt][dev];
    if (c == 0) {
        int cus = 0, per = 0;
        hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = vt ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                         &per, fwd_bf16_kernel<D, 4, 2, (int)Mode::kCausal, kVsT>, 256, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                         &per, fwd_bf16_kernel<D, 4, 2, (int)Mode::kCausal, kVsTr>, 256, 0);
        if (e != hipSuccess || cus <= 0 || per <= 0) return -1;   // not cached: asked again next time
        c = cus * per;
    }
    return c;
}

// Causal launches whose query tiles number more than one resident round of
// workgroups but at most two: the dispatcher would start the lightest tiles
// only when the first slots free up, and they would run into a tail.  Folded,
// the grid is exactly the resident slots S: on each XCD the Tx - Sx lightest
// tiles ride in the workgroups of the heaviest (two tiles in a row), and the
// remaining single tiles are ordered heavy, then light in reverse, so the
// three workgroups a CU receives add up to the same work.  Needs the tiles in
// whole heads per XCD (B*H a multiple of 8); returns S, or 0 for the plain
// one-tile-per-workgroup grid.
template <int D, int NW>
int fold_slots(const FwdArgs& a) {
    const int64_t nqt = (a.N + 32 * NW - 1) / (32 * NW);
    const int64_t T = nqt * a.BH;
    const int S = resident_slots<D>(a.vt != nullptr ? 1 : 0);
    if (S <= 0 || S % 8 != 0 || a.BH % 8 != 0) return 0;
    if (T <= S || T > 2 * (int64_t)S) return 0;
    return S;
}

// Tuning override of the dense and causal workgroup shape, read once per
// process from the environment variable ATTN_TILE: "128" (4 waves, 128 query
// rows per workgroup) or "256" (8 waves, 256 rows); unset or any other value
// keeps the automatic choice.  The outputs do not depend on it: a wave's 32
// rows, the key tiles it visits and their order are the same in both shapes.
int tile_rows_override() {
    static const int rows = [] {
        const char* e = std::getenv("ATTN_TILE");
        if (e == nullptr) return 0;
        if (std::strcmp(e, "128") == 0) return 128;
        if (std::strcmp(e, "256") == 0) return 256;
        return 0;
    }();
    return rows;
}

// The d = 128 forward with 64 query rows per wave (fwd_bf16_w64.hip, dense or
// causal, large grids) takes V in place and whole 64-key tiles (N a multiple
// of 64, at least two tiles); ATTN_W64=0 in the environment (read once per
// process) keeps the 32-row kernel instead.
bool w64_eligible(const FwdArgs& a) {
    static const bool off = [] {
        const char* e = std::getenv("ATTN_W64");
        return e != nullptr && std::strcmp(e, "0") == 0;
    }();
    return !off && a.vt == nullptr && a.N >= 128 && a.N % 64 == 0;
}

template <int D>
hipError_t launch_d(const FwdArgs& a, Mode mode, hipStream_t stream) {
    // dense, causal and key ranges: 8 waves (256 query rows) share each K/V
    // tile, one workgroup per CU, 2 tiles in flight (4 waves on small grids,
    // below).  Two stages keep the 64 KiB of K and V buffers within reach of
    // the LDS offset field, so every fragment read is a register plus an
    // immediate; three stages were slower on every shape measured (B1 H8
    // N131072 d128 causal: 1126 -> 1239 TFLOP/s with two; four key ranges
    // of B1 H32 N8192 d128: 848 -> 943).  Block-sparse: the workgroup is one
    // query block, two workgroups per CU, 2 tiles in flight.
    // Fewer than 4 rounds of 256-row workgroups over the 256 CUs: 128-row
    // workgroups (two per CU, 2 tiles in flight) fill the chip better (B=4
    // H=16 N=2048 causal: 343 -> 410 TFLOP/s); larger grids keep 256 rows,
    // which halves the K/V tile traffic per query.  Large dense and causal
    // d = 128 grids of whole 64-key tiles use the 64-row kernel (w64_eligible);
    // at d = 64 its one-wave softmax made the causal B=4 H=16 N=2048 launch
    // slower (52.3 against 50.7 us).
    const int forced = tile_rows_override();
    const bool small_grid = forced ? forced == 128 : (int64_t)((a.N + 255) / 256) * a.BH < 1024;
    switch (mode) {
        case Mode::kDense:
            if (small_grid) return launch_v<D, 4, 2, (int)Mode::kDense>(a, stream);
            if (D == 128 && w64_eligible(a)) return launch_fwd_w64(a, false, stream);
            return launch_v<D, 8, 2, (int)Mode::kDense>(a, stream);
        case Mode::kCausal:
            if (D == 128 && !small_grid && w64_eligible(a)) return launch_fwd_w64(a, true, stream);
            if (small_grid) {
                FwdArgs f = a;
                f.fold_slots = fold_slots<D, 4>(a);
                return launch_v<D, 4, 2, (int)Mode::kCausal>(f, stream);
            }
            return launch_v<D, 8, 2, (int)Mode::kCausal>(a, stream);
        case Mode::kRange: return launch_v<D, 8, 2, (int)Mode::kRange>(a, stream);
        case Mode::kSparse:
            if (a.block == 128) return launch_v<D, 4, 2, (int)Mode::kSparse>(a, stream);
            // 64-key blocks at d = 128: 32-key tile steps, so a workgroup's two
            // stages take 32 KiB of LDS and four workgroups (two waves per SIMD)
            // fit a CU; 64-key steps left one wave per SIMD (LDS-bound)
            return launch_v<D, 2, 2, (int)Mode::kSparse, D == 128 ? 32 : kBN>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int64_t vt_padded_keys(int64_t N) { return (N + 127) / 128 * 128; }

hipError_t launch_v_transpose(const FwdArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.npad / kVtKeys), (unsigned)a.BH);
    if (a.d == 64)
        hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(256), 0, stream, static_cast<const __bf16*>(a.v),
                           static_cast<__bf16*>(a.vt), a.N, a.npad);
    else
        hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, stream, static_cast<const __bf16*>(a.v),
                           static_cast<__bf16*>(a.vt), a.N, a.npad);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, Mode mode, hipStream_t stream) {
    if (a.d == 64) return launch_d<64>(a, mode, stream);
    return launch_d<128>(a, mode, stream);
}

}  // namespace bsattn
