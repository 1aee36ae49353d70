// K-split output tiles of the fp8 MMQ kernel, summed inside the product launch.
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
// Scratch layout for T split tiles of P pieces and F floats per partial tile:
//   partial slots f32 [T][P][F] at 0, then uint32 counters [T] at the next 256-byte
//   boundary.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mq {

inline size_t splitk_counter_offset(int64_t tiles, int64_t pieces, int64_t tile_floats) {
    return (size_t(tiles) * size_t(pieces) * size_t(tile_floats) * 4 + 255) & ~size_t(255);
}
inline size_t splitk_scratch_bytes(int64_t tiles, int64_t pieces, int64_t tile_floats) {
    if (tiles == 0) return 0;
    return splitk_counter_offset(tiles, pieces, tile_floats) + size_t(tiles) * 4;
}

// The partials move with relaxed agent-scope atomic loads and stores: on gfx950 these are
// plain loads and stores with the sc1 cache policy, coherent across the XCDs' L2 caches
// (written through past this XCD's L2, read past any line another call left in it).  That
// is all the exchange needs: no fence, so no cache-wide write-back or invalidate that
// would evict the data of every other workgroup on the XCD.

// Element v of accumulator tile (i, j) of thread t in a partial slot: [element][thread],
// so that for a fixed element the THREADS threads of a workgroup store contiguously.
template <int TI, int TJ, int THREADS>
__device__ __forceinline__ int splitk_index(int i, int j, int v, int t) {
    return ((i * TJ + j) * 16 + v) * THREADS + t;
}

// Store element v of tile (i, j) of this thread's partial (relaxed agent-scope atomic
// store: a plain store with the sc1 policy).
__device__ __forceinline__ void splitk_put(float* slot, int index, float value) {
    __hip_atomic_store(slot + index, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// In the last piece: the sums, in piece order, of the 16 elements of this thread's
// accumulator tile (i, j) over every piece (its own partial is read back as well: the same
// bits it stored).  A piece's 16 loads are issued together, so one tile costs `pieces`
// memory latencies, not 16 x pieces.
template <int TI, int TJ, int THREADS>
__device__ __forceinline__ void splitk_sum_tile(const float* tile_slots, int pieces, int i, int j, float (&s)[16]) {
    constexpr int kSlot = TI * TJ * 16 * THREADS;
    const float* base = tile_slots + splitk_index<TI, TJ, THREADS>(i, j, 0, threadIdx.x);
#pragma unroll
    for (int v = 0; v < 16; ++v)
        s[v] = __hip_atomic_load(base + v * THREADS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int p = 1; p < pieces; ++p) {
        float u[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            u[v] = __hip_atomic_load(base + size_t(p) * kSlot + v * THREADS, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] += u[v];
    }
}

}  // namespace mq
