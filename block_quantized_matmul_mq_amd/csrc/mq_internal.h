// Host-side declarations shared by the libmq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mq_device.h"

namespace mq {

// Values per block, and per "unit" of the GEMV kernels (64 for the 256-value K-quants,
// one block for the 32-value types).
inline bool is_kquant(int type) { return type == kQ4_K || type == kQ5_K || type == kQ6_K; }
inline int block_values_of(int type) { return is_kquant(type) ? 256 : 32; }
inline int unit_values(int type) { return is_kquant(type) ? 64 : 32; }
inline bool is_legacy(int type) { return type == kQ4_0 || type == kQ4_1 || type == kQ5_0 || type == kQ5_1; }

// Activation plane layout (see include/mq.h): codes [M][K] | scales [M][K/32] | sums [M][K/32]
// | the fp6 section below, each array starting on a 256-byte boundary.
inline size_t round_up256(size_t v) { return (v + 255) & ~size_t(255); }
inline int64_t act_steps(int64_t K) { return (K + 63) / 64; }
inline size_t act_scale_offset(int64_t M, int64_t K) { return round_up256(size_t(M) * size_t(K)); }
inline size_t act_sum_offset(int64_t M, int64_t K) {
    return act_scale_offset(M, K) + round_up256(size_t(M) * size_t(K / 32) * 4);
}
// The fp6 section (the activation half of the MMQ plane of the fp6 kernel): per 64-value
// step t a slab of 128 Mp bytes, Mp = M rounded up to kF6TileRows (the padding rows are
// zero), holding the step's two blocks u = 0, 1:
//   digits16 [2u + g][Mp][16 B] at 0    bytes 0..15 of the 24-byte fp6 record of the block's
//                                       h / 2 (g = 0) or l / 2 (g = 1) digits
//   digits8  [2u + g][Mp][8 B]  at 64 Mp  bytes 16..23 of it
//   outer    [u][Mp][8 B]       at 96 Mp  (dx_hi | dx_lo << 16) twice, bf16 bits
//   min      [u][Mp][8 B]       at 112 Mp (tx_hi | tx_hi << 16, tx_lo | tx_lo << 16), tx = dx * S
// (hi = bf16(v) and lo = bf16(v - hi), both rounded to nearest even.)  The weight plane
// (mq_repack of Q4_K) is the same per step for Np = N rounded up to kF6TileCols: codes16
// [u][Np][16 B] at 0, codes8 [u][Np][8 B] at 32 Np, outer [u][Np][8 B]
// (dw_hi | dw_hi << 16, dw_lo | dw_lo << 16) at 48 Np, min [u][Np][8 B]
// (mw_hi | mw_lo << 16) twice at 64 Np, dw = d sc and mw = -dmin m; 80 Np bytes a step.
// As bf16 matrix operands (4 values per lane) each pair multiplies out to the full product
// (x_hi + x_lo)(y_hi + y_lo) of its two factors.
constexpr int kF6TileRows = 128;
constexpr int kF6TileCols = 256;
inline int64_t f6_act_rows(int64_t M) { return (M + kF6TileRows - 1) / kF6TileRows * kF6TileRows; }
inline int64_t f6_weight_rows(int64_t N) { return (N + kF6TileCols - 1) / kF6TileCols * kF6TileCols; }
inline size_t f6_weight_plane_bytes(int64_t N, int64_t K) {
    return size_t(act_steps(K)) * 80 * size_t(f6_weight_rows(N));
}
inline size_t act_f6_offset(int64_t M, int64_t K) {
    return act_sum_offset(M, K) + round_up256(size_t(M) * size_t(K / 32) * 4);
}
inline size_t act_bytes(int64_t M, int64_t K) {
    return act_f6_offset(M, K) + size_t(act_steps(K)) * 128 * size_t(f6_act_rows(M));
}

struct DeviceInfo {
    int cu_count = 0;
    size_t lds_per_block = 0;
    uint8_t* noalloc_scratch = nullptr;   // this device's copy of mq_gemm_noalloc's scratch array
    bool ready = false;
};
const DeviceInfo* device_info();  // null if mq_init has not succeeded on the current device

// How weight blocks are stored: bytes per block slot and the offset of the GGUF block in
// its slot.  The GGUF payload itself is {34, 0} (Q8_0), {144, 0} (Q4_K), {210, 0} (Q6_K);
// mq_repack writes Q8_0 as {36, 2} and Q6_K as {224, 0}.
struct BlockLayout {
    int stride = 0;
    int off = 0;
    bool row_tiled = false;   // Q4_K's row-tiled layout (below)
};

// Q4_K's row-tiled layout (MQ_ROW_TILED), for the GEMV of rows of more than 16
// super-blocks: rows in groups of row_tile_rows(N) (at most 16; at most 256 groups up to
// 4096 rows); a group stores its rows' super-block 0 blocks one after another (row order),
// then their super-block 1 blocks, and so on; the last group is filled with zero rows.
// One group's super-block is then one contiguous run of R x 144 bytes.
inline int row_tile_rows(int64_t N) { return int(N >= 16 * 256 ? 16 : (N + 255) / 256); }
inline bool row_tiled_k(int64_t K) { return K % 256 == 0 && K / 256 > 16; }
inline size_t row_tiled_bytes(int64_t N, int64_t K) {
    const int64_t R = row_tile_rows(N);
    return size_t((N + R - 1) / R * R) * size_t(K / 256) * 144;
}
hipError_t launch_repack_q4k_row_tiled(const uint8_t* W, uint8_t* Wr, int64_t N, int64_t K, hipStream_t s);
// The long-row Q4_K GEMV on the row-tiled layout (gemv_mfma.hip): one group per workgroup.
hipError_t launch_gemv_row_tiled(const uint8_t* W, const float* x, float* y, int64_t N, int64_t K, hipStream_t s,
                                 const char** kernel_name);

// Kernel launchers: they enqueue on `s` and return the launch status (hipGetLastError read
// right after the launch).  Arguments are validated by the callers in mq_api.hip.
hipError_t launch_quantize_act(const float* X, int8_t* codes, float* scales, int32_t* sums, uint8_t* f6, int64_t M,
                               int64_t K, hipStream_t s);
int gemv_tile_units(int type, int64_t K, size_t lds_limit);
// LDS of the vector GEMV besides its row tile: the staged x (digit planes, block
// exponents and sums), and of the int8 MMQ kernel (per type and tile rows).
size_t fixed_lds_bytes(int type, int64_t K);
size_t mmq_smem_bytes(int type, int bm);
hipError_t gemv_set_attributes(size_t lds_limit);
hipError_t launch_gemv(int type, BlockLayout layout, const uint8_t* W, const float* x, float* y, int64_t N,
                       int64_t K, hipStream_t s, const char** kernel_name);
// Q4_K GEMV with the dot products on int8 matrix cores and the weights streamed through
// LDS, for wide matrices (gemv_mfma.hip).
bool gemv_mfma_applies(int type, int64_t N, int64_t K, int cu_count);
hipError_t launch_gemv_mfma(const uint8_t* W, const float* x, float* y, int64_t N, int64_t K, int cu_count,
                            hipStream_t s, const char** kernel_name);
// GEMV on int8 matrix cores with whole 16-row tiles streamed through LDS, for wide
// matrices of the other block types in the GGUF layout (gemv_mfma.hip).
bool gemv_tiled_applies(int type, BlockLayout layout, const uint8_t* W, int64_t N, int64_t K, int cu_count);
hipError_t launch_gemv_tiled(int type, const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                             int cu_count, hipStream_t s, const char** kernel_name);
// GEMV on int8 matrix cores with per-wave items, for wide Q8_0 and Q4_0 matrices in the
// GGUF layout (gemv_mfma.hip).
bool gemv_wide_applies(int type, BlockLayout layout, const uint8_t* W, int64_t N, int64_t K, int cu_count);
hipError_t launch_gemv_wide(int type, const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                            int cu_count, hipStream_t s, const char** kernel_name);
// mq_gemm for M <= 8 q8 rows on the same whole-tile stream (Q6_K, wide, GGUF layout).
bool gemv_q8_tiled_applies(int type, BlockLayout layout, const uint8_t* W, const int8_t* codes, int64_t M,
                           int64_t N, int64_t K, int cu_count);
hipError_t launch_gemv_q8_tiled(int type, const uint8_t* W, const int8_t* codes, const float* xs, float* Y,
                                int32_t* dots, int64_t M, int64_t N, int64_t K, int cu_count, hipStream_t s,
                                const char** kernel_name);
// MMQ work split over bm x 128 (int8) or 128 x 128 (fp6) output tiles: the first `full`
// tiles are computed whole; each of the remaining `split_tiles` is cut into `splits` ranges
// of whole K-steps, whose f32 partial tiles go to scratch and are summed in the same launch
// by the range that finishes last (mmq_splitk.h).  mmq_scratch_bytes is the scratch the
// int8 kernel needs (the counters, then the partial tiles), mmq_partial_bytes its partial
// tiles.
struct MmqPlan {
    int bm;            // output tile rows
    int full;
    int split_tiles;
    int splits;
    int steps;
};
MmqPlan mmq_plan(int type, int64_t M, int64_t N, int64_t K);
size_t mmq_scratch_bytes(int type, int64_t M, int64_t N, int64_t K);
size_t mmq_partial_bytes(int type, int64_t M, int64_t N, int64_t K);
// Y: the product (null for the block-dot export); dots: the export (null for the product);
// scratch: at least mmq_scratch_bytes of device memory when the plan has splits > 1;
// counters: the cut tiles' counters (zero between calls) with scratch holding only the
// partial tiles, or null when scratch holds both (mmq_splitk.h's layout).
hipError_t launch_mmq(int type, BlockLayout layout, const uint8_t* W, const int8_t* codes, const float* scales,
                      const int32_t* sums, float* Y, int32_t* dots, void* scratch, unsigned* counters, int64_t M,
                      int64_t N, int64_t K, hipStream_t s, const char** kernel_name);
// Q4_K (GGUF layout) with few output tiles: one 32 x 32 tile per workgroup, its K range
// split over the workgroup's waves (mmq_kw.hip); taken by launch_mmq whenever
// mmq_kw_applies.  It needs no scratch.
bool mmq_kw_applies(int type, BlockLayout layout, int64_t M, int64_t N, int64_t K);
size_t mmq_kw_lds_bytes();
hipError_t launch_mmq_kw(const uint8_t* W, const int8_t* codes, const float* scales, const int32_t* sums, float* Y,
                         int32_t* dots, int64_t M, int64_t N, int64_t K, hipStream_t s, const char** kernel_name);
// Q4_K in the MMQ plane (mq_repack's layout): block dots on the fp6 matrix units from the
// activation plane's fp6 section (mmq_f6.hip).  Any M.
MmqPlan mmq_f6_plan(int64_t M, int64_t N, int64_t K);
size_t mmq_f6_scratch_bytes(int64_t M, int64_t N, int64_t K);
size_t mmq_f6_partial_bytes(int64_t M, int64_t N, int64_t K);
size_t mmq_f6_lds_bytes();
hipError_t launch_mmq_f6(const uint8_t* Wp, const uint8_t* Ap, float* Y, int32_t* dots, void* scratch,
                         unsigned* counters, int64_t M, int64_t N, int64_t K, hipStream_t s, const char** name);
// mq_repack of Q4_K: the GGUF payload -> the MMQ plane (repack.hip).
hipError_t launch_repack_q4k_plane(const uint8_t* W, uint8_t* Wp, int64_t N, int64_t K, hipStream_t s);
// mq_gemm for M <= kGemvQ8MaxRows: a multi-row GEMV over the quantized activation plane
// (gemv_q8.hip), taken by launch_mmq whenever gemv_q8_applies; it needs no scratch.
constexpr int kGemvQ8MaxRows = 8;
constexpr size_t kGfx950LdsBytes = 160 * 1024;
bool gemv_q8_applies(int type, int64_t M, int64_t K);
hipError_t gemv_q8_set_attributes(size_t lds_limit);
hipError_t launch_gemv_q8(int type, BlockLayout lay, const uint8_t* W, const int8_t* codes, const float* scales,
                          const int32_t* sums, float* Y, int32_t* dots, int64_t M, int64_t N, int64_t K,
                          hipStream_t s, const char** kernel_name);
// mq_repack: every `in_bytes`-byte block of W into a `slot_bytes`-byte slot of Wr at offset
// `off`, the rest of the slot zero (repack.hip).
hipError_t launch_repack(const uint8_t* W, uint8_t* Wr, int64_t blocks, int in_bytes, int slot_bytes, int off,
                         hipStream_t s);

}  // namespace mq
