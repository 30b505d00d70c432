// Device helpers shared by the gfx950 attention kernels: operand types, the
// direct-to-LDS tile load, explicit counter waits, the LDS swizzles of the
// tile layouts and the cross-half lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds + 16 i; lds must be the same for the whole wave (it goes to M0).  Issued
// as inline asm so the compiler does not make every later LDS read wait for
// every load in flight (it cannot tell the stage buffers apart); completion is
// tracked by hand with wait_vmcnt before the barrier that publishes a tile.
// Nothing else in these kernels uses M0.
static __device__ __forceinline__ void dma16(const void* gsrc, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const unsigned lds_addr =
        __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds_addr) : "memory");
#endif
}

// The same load from a uniform base address (an SGPR pair) plus this lane's
// 32-bit byte offset, into the uniform LDS byte address lds: a tile whose
// base moves in scalar registers needs no per-lane address arithmetic.
static __device__ __forceinline__ void dma16_at(const void* sbase, unsigned voff, unsigned lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
#endif
}

// LDS byte address of a pointer into __shared__ memory.
static __device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int n>
static __device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence: the direct-to-LDS data was waited
// for explicitly; the empty asm keeps the compiler from moving LDS accesses
// across it.
static __device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Row r, logical 16-byte chunk c -> physical chunk.  Sixteen consecutive rows
// read at one logical chunk land in 16 distinct slots of a 256-byte bank window.
template <int D>
static __device__ __forceinline__ int k_swz(int r, int c) {
    return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}
// Transposed V^T tiles hold KEYS tokens per row: 2 KEYS-byte rows of KEYS / 8
// chunks (8 for 64 keys, 4 for 32); the mask stays inside the row.
template <int KEYS = 64>
static __device__ __forceinline__ int v_swz(int d, int c) { return c ^ ((d >> 1) & (KEYS / 8 - 1)); }

// Row r, logical chunk c of a row-major tile that is read both with plain
// 16-byte loads (16 consecutive rows at one chunk) and with transposing loads
// (tr_operand below: 4 consecutive rows x 4 consecutive chunks per 32 lanes):
// the XOR mask is a bijection of the row's low bits (plain reads hit 16
// distinct slots of a 256-byte bank window) that also moves each of 4
// consecutive rows to a different 4-chunk quad (transposing reads do too).
template <int D>
static __device__ __forceinline__ int rt_swz(int r, int c) {
    if (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    const int x = (r >> 1) & 7;
    return c ^ (((x & 1) << 2) | (x >> 1));
}

// Byte offsets of lane (l32, hi)'s plain 16-byte fragments (row l32, chunk
// 2k + hi, k < D / 16) in a row-major rt_swz tile.  rt_swz depends on the low
// 4 row bits only, so row 32c + l32 is at off[k] + 64 D c: with the tile inside
// the 64 KiB the LDS offset field reaches, each read is a register plus an
// immediate.
template <int D>
struct RtLane {
    int off[D / 16];
};

template <int D>
static __device__ __forceinline__ RtLane<D> rt_lane(int lane) {
    RtLane<D> t;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) t.off[k] = l32 * (2 * D) + rt_swz<D>(l32, 2 * k + hi) * 16;
    return t;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane L supplies the
// address of 4 consecutive 16-bit values; lane j receives element j % 4 of the
// values read by lanes 4e + j / 4, for e = 0..3.  Read with lane L pointing at
// row e = L / 4, columns 4 (L % 4) .. +3 of a 4 x 16 block, lane j gets column
// j, rows 0..3.
typedef short v4s_t __attribute__((ext_vector_type(4)));
static __device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
    typedef __attribute__((address_space(3))) v4s_t lds_v4s;
    const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// A operand of one v_mfma_f32_32x32x16_bf16 step taken from a row-major
// [tokens][D] LDS tile (rt_swz layout): lane l holds dim 32 db + l % 32 of the
// 16 tokens 16g..16g+15, element i of lane half h being token
// 16g + 8 (i >> 2) + 4h + (i & 3), the order in which the S^T (or S)
// accumulator registers hold tokens.  Two transposing reads of 4 tokens each;
// lane L of a 16-lane group points at token 4h + L / 4 (+8 for the second
// read), dims 32 db + 16 ((l >> 4) & 1) + 4 (L % 4) .. +3.  rt_swz depends on
// the low 4 bits of the row only, so the byte offsets for g = 0 (TrLane, per
// lane, computed once) plus 32 D g address every step.
template <int D>
struct TrLane {
    int off[2][D / 32];
};

template <int D>
static __device__ __forceinline__ TrLane<D> tr_lane(int lane) {
    TrLane<D> t;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int row = 8 * a + 4 * (lane >> 5) + ((lane >> 2) & 3);
            const int ch = 4 * db + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
            t.off[a][db] = row * (2 * D) + rt_swz<D>(row, ch) * 16 + 8 * (lane & 1);
        }
    return t;
}

template <int D>
static __device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, const TrLane<D>& t, int g, int db) {
    const bf16x4 lo = lds_read_tr(tile + t.off[0][db] + 32 * D * g);
    const bf16x4 hi = lds_read_tr(tile + t.off[1][db] + 32 * D * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Read of block-sparse metadata, which an earlier launch (or the host) wrote
// and nothing changes during this one, through the constant address space: a
// uniform index compiles to a scalar load, counted by lgkmcnt, so reading the
// next tile's key block never waits for the direct-to-LDS tile loads in flight
// (a vector load would need vmcnt(0), which waits for them too).
template <typename T>
static __device__ __forceinline__ T ld_meta(const T* p, int64_t i) {
    return ((const __attribute__((address_space(4))) T*)p)[i];
}

// One byte of metadata the same way: the scalar unit reads aligned 32-bit
// words, so the word holding the byte is read (an aligned word never crosses
// a page, so it is mapped whenever the byte is) and the byte extracted.
static __device__ __forceinline__ unsigned ld_meta_byte(const uint8_t* p, int64_t i) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(i);
    const uint32_t word = *((const __attribute__((address_space(4))) uint32_t*)(addr & ~uintptr_t(3)));
    return (word >> (8 * (addr & 3))) & 0xffu;
}

static __device__ __forceinline__ float xor32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

static __device__ __forceinline__ float xor32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace bsattn
