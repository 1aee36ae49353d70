// Device helpers shared by the matrix-unit MMQ kernels that stream their operands
// global -> LDS directly (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kRawBufferWord3 = 0x00020000;   // raw buffer resource: 32-bit data format, no swizzle

// Row (within a 32-row MFMA tile) of accumulator element v of a 32x32 f32 tile for lane
// group g (lanes 32 g .. 32 g + 31; the lane's column is lane % 32).
__device__ __forceinline__ int mfma32_acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// A raw buffer resource over `bytes` bytes at `base`: accesses at or past `bytes` read
// zeros and drop stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRawBufferWord3);
}

// x as bf16 hi = bf16(x) and lo = bf16(x - hi) (both round to nearest even), packed
// hi | lo << 16: hi + lo carries 16 significant bits of x.
__device__ __forceinline__ uint32_t bf16_hilo_bits(float x) {
    const __bf16 hi = static_cast<__bf16>(x);
    const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
    return uint32_t(__builtin_bit_cast(uint16_t, hi)) | (uint32_t(__builtin_bit_cast(uint16_t, lo)) << 16);
}

// Workgroup barrier after this wave's LDS accesses are done.  (__syncthreads would also
// wait for every global load in flight -- its workgroup fence covers global memory -- and
// so drain loads issued steps ahead.)  The "memory" clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_publish_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N vector memory operations of this wave are outstanding.  gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from buffer offset voff + soff to LDS
// bytes lds + 16 lane.  Written as asm so that the compiler does not track these loads
// (it would otherwise wait for some of them before reads of unrelated LDS); the kernels'
// own protocol -- every wave waits for its own loads of a step, then a workgroup barrier
// -- orders them.  M0, which nothing else in these kernels uses, carries the LDS address
// and needs one wait state before the load.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}

}  // namespace mq
