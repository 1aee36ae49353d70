// K-split output tiles of the MMQ kernels, summed inside the product launch.
//
// A tile whose K range is cut into P pieces is computed by P workgroups.  Each piece
// stores its partial accumulator tile to its own slot of the caller's scratch and
// counts itself in on the tile's counter; the piece that counts in last adds the P
// partials in piece order (0, 1, ..., P - 1: the same sums in the same order whichever
// piece finishes last, so the result is deterministic) and writes Y.  Nothing waits
// on another workgroup.
//
// The counter is a wrapping increment (atomic inc with limit P - 1): it reads 0 before
// a tile's first piece and is back at 0 after its last, so a scratch buffer that starts
// zeroed stays ready for the next call without any clearing launch.
//
// Scratch layout for T split tiles (T <= kSplitkMaxTiles) of P pieces and F floats per
// partial tile: uint32 counters [kSplitkMaxTiles] at 0, partial slots f32 [T][P][F] from
// kSplitkCounterBytes.  The counters sit at the same place for every shape, so calls of
// different shapes may share one buffer: no call's partial tiles cover another's counters.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mq {

constexpr int kSplitkMaxTiles = 256;                       // both plans cut at most half a round
constexpr size_t kSplitkCounterBytes = kSplitkMaxTiles * 4;
inline size_t splitk_scratch_bytes(int64_t tiles, int64_t pieces, int64_t tile_floats) {
    if (tiles == 0) return 0;
    return kSplitkCounterBytes + size_t(tiles) * size_t(pieces) * size_t(tile_floats) * 4;
}

// The partials move through buffer loads and stores with the sc1 cache policy: on gfx950
// these are coherent across the XCDs' L2 caches (written through past this XCD's L2, read
// past any line another call left in it), the same policy as relaxed agent-scope atomic
// loads and stores.  That is all the exchange needs: no fence, so no cache-wide write-back
// or invalidate that would evict the data of every other workgroup on the XCD.
//
// A thread's partial is E = TI TJ 16 floats (element e = (i TJ + j) 16 + v of its
// accumulator tiles), moved 4 at a time: group q = e / 4 of thread t sits at byte
// 16 (q THREADS + t) of its piece's slot, so that the THREADS threads of a workgroup move
// one contiguous block per 16-byte access.

typedef unsigned splitk_u4 __attribute__((ext_vector_type(4)));
typedef float splitk_f4 __attribute__((ext_vector_type(4)));
constexpr int kSplitkSc1 = 16;   // cache-policy bit sc1 of a buffer access

// Store group q (4 floats) of this thread's partial into a slot that starts `slot_off`
// bytes into the buffer `r`.
template <int THREADS>
__device__ __forceinline__ void splitk_put(__amdgpu_buffer_rsrc_t r, uint32_t slot_off, int q, splitk_f4 value) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(splitk_u4, value), r,
                                           uint32_t((q * THREADS + int(threadIdx.x)) * 16), slot_off, kSplitkSc1);
}

// After every thread has put its whole partial into its piece's slot: count the piece in.
// Returns true in the piece that counts in last; `ticket` is a word of LDS that no thread
// reads or writes at this point.
__device__ __forceinline__ bool splitk_arrive(unsigned* __restrict__ counter, int pieces, unsigned* ticket) {
    // this thread's partial has reached the device-coherent level before the count below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        *ticket = __builtin_amdgcn_atomic_inc32(counter, unsigned(pieces - 1), __ATOMIC_RELAXED, "agent");
    __syncthreads();
    return *ticket == unsigned(pieces - 1);
}

// In the last piece: the sums, in piece order, of E elements of this thread's partial
// (groups q0 .. q0 + E / 4 - 1) over the `pieces` slots of a tile (slot p at byte
// p * slot_bytes of `r`; its own partial is read back as well: the same bits it stored).
// Two pieces' loads are in flight at a time.
template <int E, int THREADS>
__device__ __forceinline__ void splitk_sum(__amdgpu_buffer_rsrc_t r, uint32_t slot_bytes, int pieces, int q0,
                                           float (&s)[E]) {
    constexpr int G = E / 4;
    auto load = [&](int p, int q) {
        return __builtin_bit_cast(splitk_f4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, uint32_t(((q0 + q) * THREADS + int(threadIdx.x)) * 16),
                                                 uint32_t(p) * slot_bytes, kSplitkSc1));
    };
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const splitk_f4 u = load(0, q);
#pragma unroll
        for (int c = 0; c < 4; ++c) s[4 * q + c] = u[c];
    }
    for (int p = 1; p < pieces; p += 2) {
        const bool two = p + 1 < pieces;
        splitk_f4 u[G], w[G];
#pragma unroll
        for (int q = 0; q < G; ++q) u[q] = load(p, q);
        if (two) {
#pragma unroll
            for (int q = 0; q < G; ++q) w[q] = load(p + 1, q);
        }
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[4 * q + c] += u[q][c];
        if (two) {
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) s[4 * q + c] += w[q][c];
        }
    }
}

}  // namespace mq
