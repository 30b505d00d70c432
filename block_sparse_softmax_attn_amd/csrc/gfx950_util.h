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
// Transposed tiles (V^T, Q^T, ...) hold 64 tokens per row: 128-byte rows, 8 chunks.
static __device__ __forceinline__ int v_swz(int d, int c) { return c ^ ((d >> 1) & 7); }

// Slot of the first key of quad kq (keys 4kq..4kq+3 of a tile) in a V^T row:
// inside each 16-key group, keys {4h..4h+3, 8+4h..8+4h+3} (the ones lane half
// h holds in its S^T registers) take slots 8h..8h+7.  Same order as the
// transpose pass writes.
static __device__ __forceinline__ int vt_pos_of_quad(int kq) {
    return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
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
