// Fused attention forward, bf16, d = 128, dense or causal: one wave per SIMD
// holding 64 query rows, with the softmax of one 32-key sub-tile overlapped with
// the matrix products of its neighbours.
//
// The method is the one of fwd_bf16.hip ("Exact Blocks, Rings, and Sparsity",
// section 2, "What the forward kernel keeps on chip"; FlashAttention notes,
// section 5.2): a query tile stays on chip, key/value tiles stream through LDS,
// and each score tile is folded into the running (m, l, A) state of its rows.
// Only the schedule differs.
//
// Why this shape on gfx950.  Ordinary vector instructions issued between
// independent MFMAs of the same wave execute in the MFMA's shadow, up to about
// four FMAs per MFMA (a register-only measurement: 16 32x32x16 MFMAs take 512
// cycles alone, 520 with 64 FMAs interleaved, 688 with 128: each MFMA holds
// the wave's issue for ~11 of its 32 cycles, and an exponential there costs
// ~12 cycles of issue).  The softmax of a tile, though, depends on that tile's
// score products and feeds its PV products, so in the one-tile-at-a-time loop
// it runs between them and the matrix core idles.  Here a wave splits each
// 64-key tile into two 32-key sub-tiles k and runs a three-stage pipeline: in
// stage k it issues the score MFMAs of sub-tile k+1 and the PV MFMAs of
// sub-tile k-1, and between them the exponentials of sub-tile k.  The two
// products and the vector work of a stage are independent of each other; a
// stage (32 MFMAs, 32 exponentials, ~90 other vector instructions, 24 LDS
// reads) needs about as many issue cycles as its matrix work takes.
//
// Each wave holds 64 query rows (two 32-row blocks r) instead of 32, so every
// K or V fragment read from LDS feeds two MFMAs: half the LDS reads per flop.
// Its registers: O^T of 64 rows (128 accumulators, kept in AGPRs), Q (64), the
// scores of two sub-tiles (64), P of two sub-tiles (32) and the fragments in
// flight -- more than two waves per SIMD could hold, so a workgroup is 4 waves
// (256 query rows) and a CU runs one.
//
// The online softmax is the one of fwd_bf16.hip: the exponentials of sub-tile
// k are taken against each row's current reference value m and folded in as is
// when every lane's sum is finite and at most 2^64; otherwise m is raised to the
// sub-tile's row max, the state rescaled and the exponentials recomputed.  The
// PV products of sub-tile k-1, issued in the same stage, used P relative to the
// old m, so rescaling A after them is exact.  A row's first sub-tile takes m
// from its own row max before its exponentials (its scores are complete when
// its stage begins), so it needs no check.
//
// Tiles: K and V tiles of 64 keys go straight into LDS (global_load_lds_dwordx4),
// two buffers each.  Stage 2t+1 needs K of tile t+1 (its first half) and V of
// tile t, so one barrier per tile, before that stage, publishes K(t+1) and V(t)
// and frees K(t) and V(t-1), whose buffers then receive K(t+2) and V(t+1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fwd_common.h"
#include "gfx950_util.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kNW = 4;                       // waves per workgroup
constexpr int kRows = 64;                    // query rows per wave
constexpr int kBM = kNW * kRows;             // query rows per workgroup
constexpr int kBN = 64;                      // keys per tile
constexpr float kSumMax = 0x1p64f;
constexpr float kLn2 = 0.69314718055994530942f;

// acc += a * b with acc in AGPRs (v_mfma_f32_32x32x16_bf16, AGPR form).  The
// compiler does not see an MFMA here, so the wait states that a vector access
// of the accumulators needs after it (and it after a vector write of them) are
// inserted by hand with settle_acc().
static __device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 24 wait states between the AGPR-form products and vector accesses of their
// accumulators (in either order); the operands pin the accesses to this point.
static __device__ __forceinline__ void settle_acc(f32x16 (&o)[2][4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                   "+a"(o[1][2]), "+a"(o[1][3]));
}

template <bool CAUSAL>
__global__ __launch_bounds__(64 * kNW, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_w64_kernel(FwdArgs a) {
    constexpr int kD = 128;
    constexpr int kTileBytes = kBN * kD * 2;         // one K or V tile
    constexpr int kPerW = kTileBytes / 1024 / kNW;   // 1 KiB direct-to-LDS loads per wave per tile
    constexpr int NF = kD / 16;                      // K chunks (and V^T fragments) per 32-key half
    constexpr int NDB = kD / 32;                     // 32-dimension blocks of O
    // two K tiles, then two V tiles
    __shared__ __attribute__((aligned(1024))) unsigned char sK[2 * kTileBytes], sV[2 * kTileBytes];
    const unsigned kl = lds_addr(sK), vl = lds_addr(sV);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const TrLane<kD> trl = tr_lane<kD>(lane);
    // K fragment of chunk c (dims 16c..16c+15), row l32 of a 32-key half
    int koff[NF];
#pragma unroll
    for (int c = 0; c < NF; ++c) koff[c] = l32 * (2 * kD) + rt_swz<kD>(l32, 2 * c + hi) * 16;

    const int N = a.N;
    const int nqt = (N + kBM - 1) / kBM;
    int64_t bh;
    int qt;
    if constexpr (CAUSAL) {   // the costliest query tiles of the XCD's heads first
        rank_major_order(blockIdx.x, (int64_t)nqt * a.BH, nqt, bh, qt);
        qt = nqt - 1 - qt;
    } else {
        const int64_t ord = xcd_tile_order(blockIdx.x, (int64_t)nqt * a.BH);
        bh = ord / nqt;
        qt = (int)(ord % nqt);
    }
    const int q0 = qt * kBM + kRows * w;   // this wave's first row

    const int64_t kvh = kv_head_of(bh, a.H, a.Hkv);
    const __bf16* Qh = static_cast<const __bf16*>(a.q) + bh * (int64_t)N * kD;
    const __bf16* Kh = static_cast<const __bf16*>(a.k) + kvh * (int64_t)N * kD;
    const __bf16* Vh = static_cast<const __bf16*>(a.v) + kvh * (int64_t)N * kD;

    // Q fragments (B operand of S^T = K Q^T) of rows q0 + 32r + l32
    bf16x8 qf[2][NF];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int qrow = min(q0 + 32 * r + l32, N - 1);
#pragma unroll
        for (int c = 0; c < NF; ++c)
            qf[r][c] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qrow * kD + 16 * c + 8 * hi);
    }

    // direct-to-LDS loads: lane i of load g fills bytes [1024 g + 16 i, +16) of
    // the tile, i.e. row rr, physical chunk p, holding logical chunk rt_swz(rr, p)
    unsigned ld_boff[kPerW];
#pragma unroll
    for (int i = 0; i < kPerW; ++i) {
        const int byte = (w * kPerW + i) * 1024 + lane * 16;
        const int rr = byte / (2 * kD), p = (byte % (2 * kD)) / 16;
        ld_boff[i] = (unsigned)(2 * (rr * kD + rt_swz<kD>(rr, p) * 8));
    }
    const unsigned wl = __builtin_amdgcn_readfirstlane(w * kPerW * 1024);
    // load i (of kPerW) of this wave's part of the tile at key kb0 (N is a
    // multiple of the tile, so every tile is whole)
    auto issue_one = [&](const __bf16* base, int kb0, unsigned lds, int i) __attribute__((always_inline)) {
        dma16_at(base + (int64_t)kb0 * kD, ld_boff[i], lds + wl + i * 1024);
    };
    auto issue = [&](const __bf16* base, int kb0, unsigned lds) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kPerW; ++i) issue_one(base, kb0, lds, i);
    };

    f32x16 oacc[2][NDB];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[r][i] = f32x16{};
    settle_acc(oacc);
    float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
    float ell[2] = {0.f, 0.f};
    const float sl2 = a.scale_log2;
    // tiles; sub-tiles 0 .. 2T-1 (causal: keys up to the workgroup's last row)
    const int T = CAUSAL ? min(N, qt * kBM + kBM) / kBN : N / kBN;

    // exponentials of s against m_run into p; per-row-block lane sums
    auto exps = [&](const f32x16 (&s)[2], bf16x8 (&p)[2][2], float (&tsum)[2], int r, float mu) __attribute__((always_inline)) {
        float ts[4];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r][8 * g + i], sl2, -mu));
                ts[i & 3] = (g == 0 && i < 4) ? e : ts[i & 3] + e;
                p[r][g][i] = (__bf16)e;
            }
        tsum[r] = (ts[0] + ts[1]) + (ts[2] + ts[3]);
    };
    // causal: key j of the sub-tile starting at kb is masked for row i when
    // j > i; s[r][v] holds key kb + 8(v>>2) + 4hi + (v&3) of row q0 + 32r + l32
    auto mask = [&](f32x16 (&s)[2], int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int rlim = q0 + 32 * r + l32 - kb - 4 * hi;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[r][v] = 8 * (v >> 2) + (v & 3) > rlim ? -__builtin_inff() : s[r][v];
        }
    };
    // the check after the exponentials of a sub-tile (see the file comment)
    auto settle = [&](const f32x16 (&s)[2], bf16x8 (&p)[2][2], float (&tsum)[2], bool bad) __attribute__((always_inline)) {
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                float mx = -__builtin_inff();
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[r][v]);
                mx = xor32_max(mx);
                const float mt = mx * sl2;
                const bool upd = mt > m_run[r];
                if (__builtin_amdgcn_ballot_w64(upd) != 0) {
                    const float alpha = upd ? __builtin_amdgcn_exp2f(m_run[r] - mt) : 1.0f;
                    m_run[r] = upd ? mt : m_run[r];
                    ell[r] *= alpha;
                    settle_acc(oacc);
#pragma unroll
                    for (int i = 0; i < NDB; ++i) oacc[r][i] *= alpha;
                    settle_acc(oacc);
                }
                exps(s, p, tsum, r, m_run[r] == -__builtin_inff() ? 0.f : m_run[r]);
            }
        }
        ell[0] += tsum[0];
        ell[1] += tsum[1];
    };

    // ---- the pipeline ----
    // Stage k: SM(k), the softmax of sub-tile k (scores sin -> P pout); S(k+1),
    // the scores of the next sub-tile (K at bK -> sout); PV(k-1), the product of
    // the previous sub-tile (P pin, V^T fragments of half vhalf of the V tile
    // at bV).  Fragment j (j < 8): K chunk j (dims 16j..16j+15) and the V^T
    // fragment of 16-key group j / 4 and dimension block j % 4; each feeds the
    // MFMAs of both row blocks.  Group j issues those four MFMAs, a share of
    // the exponentials (groups 0-5) and of the sums and bf16 packing (lagging
    // one group), and the reads of fragment j + 2; groups 6 and 7 read the
    // first two fragments of the next stage (kN, vN) so that they are in
    // flight across the check.  In a stage before a tile boundary the tile
    // barrier sits before group 7, after this wave's fragment reads of the
    // retiring tiles have returned: the loads of the tiles after next are
    // issued there, and the next stage's fragments are read from the new ones.
    enum : int {
        fS = 1,         // S(k+1)
        fP = 2,         // PV(k-1)
        fSM = 4,        // SM(k) and its check
        fBar = 8,       // tile barrier before group 7
        fLoad = 16,     // K and V tile loads, one in every fourth slot
        fLoadV = 512,   // the V tile load only
        fNK = 32,       // read the next stage's first K fragments
        fNV = 64,       // read the next stage's first V fragments
        fCold = 256,    // no fragments were read ahead for this stage
        fFirst = 1024,  // sub-tile 0: m from its row max first, no check
    };
    f32x16 sE[2], sO[2];          // scores of even / odd sub-tiles
    bf16x8 pE[2][2], pO[2][2];    // P of even / odd sub-tiles
    bf16x8 kN[2], vN[2];          // first fragments of the next stage
    auto stage = [&](auto flags, f32x16 (&sin)[2], bf16x8 (&pout)[2][2], f32x16 (&sout)[2],
                     const unsigned char* bK, const bf16x8 (&pin)[2][2], const unsigned char* bV, int vhalf,
                     const unsigned char* bKn, const unsigned char* bVn, int vhalf_n, int k_load, unsigned k_lds,
                     int v_load, unsigned v_lds, int kb_in) __attribute__((always_inline)) {
        constexpr int F = decltype(flags)::value;
        constexpr bool DS = F & fS, DP = F & fP, SM = F & fSM;
        // causal: the element mask on a sub-tile that reaches past this wave's
        // first row (sub-tiles wholly past its rows are computed and masked)
        if constexpr (CAUSAL && SM) {
            if (kb_in + 31 > q0) mask(sin, kb_in);
        }
        bf16x8 kf[NF], vf[NF];
        auto read = [&](int j) __attribute__((always_inline)) {
            if constexpr (DS) kf[j] = *reinterpret_cast<const bf16x8*>(bK + koff[j]);
            if constexpr (DP) vf[j] = tr_operand<kD>(bV, trl, 2 * vhalf + j / NDB, j % NDB);
        };
        auto read_next = [&](int j) __attribute__((always_inline)) {
            if constexpr ((F & fNK) != 0) kN[j] = *reinterpret_cast<const bf16x8*>(bKn + koff[j]);
            if constexpr ((F & fNV) != 0) vN[j] = tr_operand<kD>(bVn, trl, 2 * vhalf_n + j / NDB, j % NDB);
        };
        // softmax element e: row block e / 16, register e % 16
        float ex[32], ts[2][4];
        auto expo = [&](int e) __attribute__((always_inline)) {
            const int r = e / 16, v = e % 16;
            ex[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sin[r][v], sl2, -m_run[r]));
        };
        // the empty asm statements keep each sum and pack in its slot (the
        // compiler would otherwise sink them all to the end of the stage)
        auto fold = [&](int e) __attribute__((always_inline)) {
            const int r = e / 16, v = e % 16;
            if (v >= 4) {
                ts[r][v & 3] = v < 8 ? ex[e - 4] + ex[e] : ts[r][v & 3] + ex[e];
                asm volatile("" : "+v"(ts[r][v & 3]));
            }
            if (v & 1) {
                bf16x2 pr = {(__bf16)ex[e - 1], (__bf16)ex[e]};
                asm volatile("" : "+v"(pr));
                pout[r][v / 8][(v & 7) - 1] = pr[0];
                pout[r][v / 8][v & 7] = pr[1];
            }
        };
        if constexpr (DS) {
            sout[0] = f32x16{};
            sout[1] = f32x16{};
        }
        if constexpr ((F & fFirst) != 0) {
            // every row's first sub-tile: its scores are complete, so m starts
            // at their row max and no exponential can exceed 1 (whole tiles
            // and no masks here, so the max is finite)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                float mx = sin[r][0];
#pragma unroll
                for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sin[r][v]);
                m_run[r] = xor32_max(mx) * sl2;
            }
        }
        if constexpr ((F & fCold) != 0) {
            read(0);
            read(1);
        } else {
            if constexpr (DS) {
                kf[0] = kN[0];
                kf[1] = kN[1];
            }
            if constexpr (DP) {
                vf[0] = vN[0];
                vf[1] = vN[1];
            }
        }
        // One slot per MFMA, fenced so that the compiler keeps the order: the
        // MFMA, one exponential (two in 16-slot stages), the sum and packing of
        // an element exponentiated LAG slots earlier, and at most one fragment
        // read.  Slot order per fragment j: S r0, S r1, PV r0, PV r1.
        constexpr int NSL = (DS ? 2 * NF : 0) + (DP ? 2 * NF : 0);
        // element e is exponentiated in slot (e * SPAN) / 32 and folded LAG
        // slots later; the slot after the last fold computes the check's
        // inputs, so that only the ballot and the branch follow the last MFMA
        constexpr int SPAN = NSL * 3 / 4, LAG = NSL / 8;
        float tsum[2];
        bool bad = false;
        int slot = 0;
        auto work = [&](int i) __attribute__((always_inline)) {
            if constexpr (SM) {
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    if ((e * SPAN) / 32 == i) expo(e);
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    if ((e * SPAN) / 32 + LAG == i) fold(e);
                if (i == SPAN + LAG) {
                    tsum[0] = (ts[0][0] + ts[0][1]) + (ts[0][2] + ts[0][3]);
                    tsum[1] = (ts[1][0] + ts[1][1]) + (ts[1][2] + ts[1][3]);
                    bad = !(tsum[0] <= kSumMax) || !(tsum[1] <= kSumMax);
                }
            }
        };
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            // fragment reads issued in the slots of group j: fragment j + 2,
            // then (the last two groups) the next stage's fragments 0 and 1
            if constexpr ((F & fBar) != 0) {
                if (j == NF - 1) {
                    __builtin_amdgcn_sched_barrier(0);
                    // this wave's reads of the retiring tiles have returned;
                    // every wave's loads of the next tiles have landed
                    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
                    barrier();
                }
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const bool isS = q4 < 2;
                const int r = q4 & 1;
                if (isS && !DS) continue;
                if (!isS && !DP) continue;
                __builtin_amdgcn_sched_barrier(0);
                if (isS) sout[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[r][j], sout[r], 0, 0, 0);
                else mfma_acc(oacc[r][j % NDB], vf[j], pin[r][j / NDB]);
                work(slot);
                // tile loads (into buffers freed by the last barrier), one per slot
                if constexpr ((F & fLoad) != 0) {   // every fourth slot
                    if (slot % 4 == 0 && slot < 4 * kPerW) issue_one(Kh, k_load, k_lds, slot / 4);
                    else if (slot % 4 == 0 && slot < 8 * kPerW) issue_one(Vh, v_load, v_lds, slot / 4 - kPerW);
                } else if constexpr ((F & fLoadV) != 0) {
                    if (slot % 4 == 0 && slot < 4 * kPerW) issue_one(Vh, v_load, v_lds, slot / 4);
                }
                // reads: first slot of the group reads fragment j+2 (or the
                // next stage's first fragments in groups 6 and 7)
                if (q4 == (DS ? 0 : 2)) {   // the group's first slot
                    if (j + 2 < NF) read(j + 2);
                    else if ((F & fBar) == 0 || j == NF - 1) {
                        if constexpr ((F & fBar) != 0) {
                            read_next(0);
                            read_next(1);
                        } else {
                            read_next(j - (NF - 2));
                        }
                    }
                }
                ++slot;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SM && (F & fFirst) != 0) {
            ell[0] = tsum[0];
            ell[1] = tsum[1];
        } else if constexpr (SM) {
            // P complete before the check (which may recompute it)
            asm volatile("" : "+v"(pout[0][0]), "+v"(pout[0][1]), "+v"(pout[1][0]), "+v"(pout[1][1]));
            settle(sin, pout, tsum, bad);
        }
    };
    constexpr unsigned kHalf = 32 * 2 * kD;   // bytes of a 32-key half of a tile
    const unsigned char* const sK1 = sK + kTileBytes;
    const unsigned char* const sV1 = sV + kTileBytes;

    // Prologue: K(0), V(0), K(1) in flight; S(0) once K(0) has landed, then
    // stage 0 (S(1), SM(0)), whose barrier B_0 publishes K(1) and V(0).
    issue(Kh, 0, kl);
    issue(Vh, 0, vl);
    issue(Kh, kBN, kl + kTileBytes);
    wait_vmcnt<2 * kPerW>();
    barrier();
    stage(std::integral_constant<int, fS | fCold | fNK>{}, sO, pO, sE, sK, pE, sV, 0, sK + kHalf, sV, 0, 0, 0, 0, 0,
          0);
    stage(std::integral_constant<int, fS | fSM | fFirst | fBar | fNK | fNV>{}, sE, pE, sO, sK + kHalf, pO, sV, 0, sK1,
          sV, 0, 0, 0, 0, 0, 0);

    // Tile t+1 for t <= T-3: stage 2t+1 (S(2t+2) <- K(t+1) half 0, PV(2t) <-
    // V(t) half 0, SM(2t+1); loads of K(t+2) and V(t+1) into the buffers of
    // K(t) and V(t-1), freed by B_t), stage 2t+2 (S(2t+3) <- K(t+1) half 1,
    // PV(2t+1) <- V(t) half 1, SM(2t+2), barrier B_{t+1}).  Two tiles per
    // trip, so that every LDS address is a register plus an immediate.
    auto iter = [&](int t, auto par) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;   // t & 1
        const unsigned char* const bK = P ? sK : sK1;    // K(t+1)
        const unsigned char* const bV = P ? sV1 : sV;    // V(t)
        const unsigned char* const bKn = P ? sK1 : sK;   // K(t+2)
        const unsigned char* const bVn = P ? sV : sV1;   // V(t+1)
        stage(std::integral_constant<int, fS | fP | fSM | fLoad | fNK | fNV>{}, sO, pO, sE, bK, pE, bV, 0, bK + kHalf,
              bV, 1, (t + 2) * kBN, kl + P * kTileBytes, (t + 1) * kBN, vl + (1 - P) * kTileBytes, t * kBN + 32);
        stage(std::integral_constant<int, fS | fP | fSM | fBar | fNK | fNV>{}, sE, pE, sO, bK + kHalf, pO, bV, 1, bKn,
              bVn, 0, 0, 0, 0, 0, (t + 1) * kBN);
    };
    int t = 0;
    for (; t + 3 < T; t += 2) {   // t, t+1 <= T-3
        iter(t, std::integral_constant<int, 0>{});
        iter(t + 1, std::integral_constant<int, 1>{});
    }
    if (t + 2 < T) iter(t, std::integral_constant<int, 0>{});   // t = T-3, even
    {   // t = T-2: load of V(T-1), published by the last barrier
        const int tl = T - 2;
        const unsigned char* bK = (tl & 1) ? sK : sK1;
        const unsigned char* bV = (tl & 1) ? sV1 : sV;
        const unsigned char* bVn = (tl & 1) ? sV : sV1;
        stage(std::integral_constant<int, fS | fP | fSM | fLoadV | fNK | fNV>{}, sO, pO, sE, bK, pE, bV, 0,
              bK + kHalf, bV, 1, 0, 0, (tl + 1) * kBN, vl + ((tl + 1) & 1) * kTileBytes, tl * kBN + 32);
        stage(std::integral_constant<int, fS | fP | fSM | fBar | fNV>{}, sE, pE, sO, bK + kHalf, pO, bV, 1, nullptr,
              bVn, 0, 0, 0, 0, 0, (tl + 1) * kBN);
        // stage 2T-1: PV(2T-2) <- V(T-1) half 0, SM(2T-1)
        stage(std::integral_constant<int, fP | fSM | fNV>{}, sO, pO, sE, nullptr, pE, bVn, 0, nullptr, bVn, 1, 0, 0,
              0, 0, (tl + 1) * kBN + 32);
        // PV(2T-1) <- V(T-1) half 1
        stage(std::integral_constant<int, fP>{}, sE, pE, sO, nullptr, pO, bVn, 1, nullptr, nullptr, 0, 0, 0, 0, 0,
              0);
    }

    // ---- epilogue: O = A / l, LSE = (m + log2 l) ln 2 ----
    // O goes through LDS (the tile buffers are idle now): each wave writes
    // its 64 x 128 bf16 rows there, 16-byte chunks XOR-swizzled by the row,
    // and reads them back four whole rows per instruction, so every global
    // store writes 1 KiB of consecutive bytes.
    settle_acc(oacc);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's last fragment reads have returned
    barrier();                            // ... and every other wave's
    unsigned char* const stg = (w < 2 ? sK : sV) + (w & 1) * (kRows * kD * 2);
    constexpr int CPR = kD / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;   // rows per 1 KiB read
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 32 * r + l32;   // of the wave's 64
        const float l_tot = xor32_sum(ell[r]);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 ov;
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(oacc[r][db][4 * j + i] * inv);
                const int chunk = (4 * db + j) ^ (row & (CPR - 1));   // dims 32 db + 8 j .. + 7
                *reinterpret_cast<bf16x4*>(stg + row * (2 * kD) + chunk * 16 + 8 * hi) = ov;
            }
        const int qi = q0 + row;
        if (hi == 0 && qi < N)
            a.lse[bh * (int64_t)N + qi] = l_tot > 0.f ? (m_run[r] + __log2f(l_tot)) * kLn2 : -__builtin_inff();
    }
    __bf16* const Oh = static_cast<__bf16*>(a.o) + bh * (int64_t)N * kD;
#pragma unroll
    for (int s4 = 0; s4 < kRows / RPI; ++s4) {
        const int row = RPI * s4 + lane / CPR, c = lane % CPR;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stg + row * (2 * kD) + (c ^ (row & (CPR - 1))) * 16);
        if (q0 + row < N) *reinterpret_cast<u32x4*>(Oh + (int64_t)(q0 + row) * kD + 8 * c) = val;
    }
}

}  // namespace

hipError_t launch_fwd_w64(const FwdArgs& a, bool causal, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)((a.N + kBM - 1) / kBM) * a.BH)), block(64 * kNW);
    if (causal) hipLaunchKernelGGL(fwd_w64_kernel<true>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(fwd_w64_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace bsattn
