/*
 * mq.h -- C ABI of libmq: matrix products of GGUF block-quantized weights
 * (Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q4_K, Q5_K, Q6_K) with f32 activations on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (page title, section):
 *   [BD2.3] "minfer CUDA Backend Design", 2.3 Weight residency and registry:
 *           Q4_K payload is exactly od * (id / 256) * 144 bytes; q8_0 is 34 bytes
 *           per 32 values; Q6_K is repacked into 16-byte-aligned 224-byte slots;
 *           a derived plane is admitted by a type gate plus an exact-length
 *           payload gate ("equality, not a lower bound").
 *   [BD4.3] same page, 4.3 Eligibility: a quantized matmul needs id % 32 == 0;
 *           the matmul weight types are Q4_0/Q4_1/Q5_0/Q5_1/Q8_0/Q4_K/Q5_K/Q6_K;
 *           an invariant violation is an error, never a silent fallback.
 *   [GS3]   "GPU Safety (Metal + CUDA Backends)", 3. Audit findings: the Q5_K
 *           block is 176 bytes.
 *   [BD4.4] same page, 4.4 Execution dispatch: decode (one token) runs a
 *           matrix-vector product; prefill runs the int8 "MMQ" GEMM over an
 *           activation plane quantized to q8 blocks, which is computed once and
 *           can be reused by consecutive matmuls that share the input.
 *   [BD4.9] same page, 4.9 GPU safety: errors are errors; a return value that
 *           gates a later launch is read at the call site; device limits are
 *           queried at run time.
 *   [EP-C4] "minfer Architecture Execution Plan", C4 S2b design decision 4:
 *           the Q8_0 quantizer is amax over the 32-block, scale amax / 127,
 *           codes rounded half to even.
 *
 * Layouts (all little-endian):
 *   W  : N rows (outputs) x K columns (inputs), row-major; each row is K / bv
 *        consecutive blocks (bv = 32 for Q4_0/Q4_1/Q5_0/Q5_1/Q8_0, 256 for
 *        Q4_K/Q5_K/Q6_K).  Block bytes: Q8_0 34 (f16 d, int8 q[32]); Q4_0 18
 *        (f16 d, 16 bytes of 4-bit codes, value i in the low and value 16 + i in
 *        the high nibble of byte i; value d (code - 8)); Q4_1 20 (f16 d, f16 m,
 *        the codes; value d code + m); Q5_0 22 (f16 d, 32 high bits, the low
 *        nibbles; value d (code - 16)); Q5_1 24 (f16 d, f16 m, high bits, low
 *        nibbles; value d code + m); Q4_K 144 (f16 d, f16 dmin, 12 bytes of
 *        6-bit scale/min pairs, 128 bytes of 4-bit codes); Q5_K 176 (Q4_K's
 *        header, 32 bytes of high bits, Q4_K's codes); Q6_K 210 (128 bytes low
 *        4 bits, 64 bytes high 2 bits, 16 int8 sub-scales, f16 d).  These are
 *        the public GGUF layouts; the pages fix only some sizes and the types.
 *   x  : K f32.   y : N f32.   X : M x K f32 row-major.   Y : M x N f32 row-major.
 *   Xq : the quantized activation plane written by mq_quantize_act, four
 *        arrays in one buffer of mq_act_bytes(M, K) bytes (T = ceil(K / 64)):
 *          codes  int8  [M][K]          at offset 0
 *          scales f32   [M][K / 32]     at offset mq_act_scale_offset(M, K)
 *          sums   int32 [M][K / 32]     at offset mq_act_sum_offset(M, K)
 *          fp6 section [T][128 Mp bytes] at mq_act_f6_offset(M, K), Mp = M rounded
 *                up to a multiple of 128 (rows M..Mp-1 zero)
 *        For block b of row m: scale = f32(amax) / f32(127) with IEEE division,
 *        code_i = clamp(round_half_even(x_i / scale), -127, 127) (a true f32
 *        division), scale 0 and codes 0 when amax == 0, and sum = sum of the 32
 *        codes.
 *        The fp6 section re-encodes the codes for the fp6 matrix units, each code
 *        q = 16 h + l (h = q >> 4 in -8..7, l = q & 15) as the 6-bit OCP FP6
 *        E2M3 codes of h / 2 and of l / 2 (exact); a block's 32 codes of one
 *        digit form a 24-byte record, value i at bits 6 i .. 6 i + 5 (little
 *        endian).  In step t's slab, for block b = 2 t + u of row m:
 *          bytes 16 ((2 u + g) Mp + m) ..        record bytes 0..15, g = 0: h, g = 1: l
 *          bytes 64 Mp + 8 ((2 u + g) Mp + m) .. record bytes 16..23
 *          bytes 96 Mp + 8 (u Mp + m) ..         words (dx_hi | dx_lo << 16) twice
 *          bytes 112 Mp + 8 (u Mp + m) ..        words (tx_hi | tx_hi << 16,
 *                                                       tx_lo | tx_lo << 16)
 *        with dx the block scale and tx = dx * sum (the f32 product), each split
 *        as hi = bf16(v), lo = bf16(v - hi) (round to nearest even, bf16 bits).
 *        When K % 64 == 32 the last step's second block is all zeros.
 *
 * Ownership and streams: the caller allocates and frees every buffer (device
 * memory, e.g. from torch).  Weights and inputs are read only.  No call
 * allocates, frees or synchronizes; every kernel runs on the caller's stream
 * (a hipStream_t passed as void*, NULL = the null stream), so calls may be
 * captured into a HIP graph.  Pointers must be 16-byte aligned unless stated.
 *
 * Errors: every call returns MQ_OK (0) or a negative MQ_ERR_* code and never
 * falls back to another kernel or to the host.  Argument checks run before
 * any HIP call.  mq_last_error() returns a thread-local message naming the
 * call, the offending values and, for HIP failures, hipGetErrorName.
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight type ids: the GGUF tensor-type ids. */
#define MQ_Q4_0 2
#define MQ_Q4_1 3
#define MQ_Q5_0 6
#define MQ_Q5_1 7
#define MQ_Q8_0 8
#define MQ_Q4_K 12
#define MQ_Q5_K 13
#define MQ_Q6_K 14
/* OR-ed into MQ_Q8_0, MQ_Q6_K or MQ_Q4_K: the weights are in the layout mq_repack
 * writes (every call that takes a weight type accepts it, except that mq_gemv refuses
 * Q4_K's, which is a plane for mq_gemm only). */
#define MQ_REPACKED 0x100
/* OR-ed into MQ_Q4_K only: the weights are in Q4_K's row-tiled layout, which
 * mq_repack(.., MQ_Q4_K | MQ_ROW_TILED, ..) writes and mq_gemv reads (for rows of
 * more than 16 super-blocks; see mq_repack). */
#define MQ_ROW_TILED 0x200

/* Status codes. */
#define MQ_OK 0
#define MQ_ERR_ARG (-1)    /* null pointer, negative or zero size            */
#define MQ_ERR_SHAPE (-2)  /* K not a multiple of the block size, M/N/K limit */
#define MQ_ERR_TYPE (-3)   /* unsupported weight type id                      */
#define MQ_ERR_SIZE (-4)   /* a byte count that is not exactly the required one */
#define MQ_ERR_ALIGN (-5)  /* pointer not 16-byte aligned                     */
#define MQ_ERR_DEVICE (-6) /* no usable gfx950 device, or a HIP runtime error */
#define MQ_ERR_LAUNCH (-7) /* a kernel launch was refused                     */
#define MQ_ERR_NOINIT (-8) /* mq_init has not succeeded on the current device */

/* Upper bounds accepted by the calls (sizes beyond them are MQ_ERR_SHAPE). */
#define MQ_MAX_K 32768          /* inputs per row                 */
#define MQ_MAX_N (1 << 24)      /* output rows                    */
#define MQ_MAX_M (1 << 20)      /* activation rows for mq_gemm    */

/*
 * mq_init -- select `device`, check that it is gfx950, record its compute-unit
 * count and LDS limit, and set every kernel attribute the library needs.  Call
 * once per device before any other call on it, outside any stream capture
 * [BD4.9: limits queried at run time].  Returns MQ_ERR_DEVICE when there is no
 * such device or it is not gfx950.  Idempotent.
 */
int mq_init(int device);

/* Exact byte size of a GGUF payload of N x K weights of `type` [BD2.3] (of
 * the repacked layout for type | MQ_REPACKED, of the row-tiled layout for
 * MQ_Q4_K | MQ_ROW_TILED); 0 for an unsupported type, a K that is not a whole
 * number of blocks, or (row-tiled) K <= 4096. */
size_t mq_weight_bytes(int type, int64_t N, int64_t K);

/*
 * mq_repack_bytes / mq_repack -- the one-time device-layout transform of a
 * weight matrix [BD2.3: Q6_K is repacked into 16-byte-aligned 224-byte slots;
 * a derived plane is admitted only with an exact-length payload].  Each block
 * of the GGUF payload W (device, nbytes bytes, which must equal
 * mq_weight_bytes(type, N, K) exactly, else MQ_ERR_SIZE) is copied into its own
 * slot of Wr (device, at least mq_repack_bytes(type, N, K) bytes), rows and
 * blocks in the same order, the other slot bytes zero:
 *   MQ_Q6_K: 224-byte slots, the 210-byte block at offset 0 (16-byte aligned);
 *   MQ_Q8_0: 36-byte slots, the 34-byte block at offset 2 (its 32 codes start
 *            4-byte aligned).
 * Pass type | MQ_REPACKED with Wr to mq_gemv / mq_gemm: the results are the
 * same as with W.
 *   MQ_Q4_K: the MMQ plane of the fp6 prefill product (the pre-decoded weight plane
 *            of [BD2.3]'s reference, here for the prefill only), T = K / 64 steps of
 *            80 Np bytes, Np = N rounded up to a multiple of 256 (rows N..Np-1
 *            zero).  In step t's slab, for sub-block b = 2 t + u of row n: bytes
 *            16 (u Np + n) .. and 32 Np + 8 (u Np + n) .. hold bytes 0..15 and
 *            16..23 of the 24-byte record of its codes c, each the OCP FP6 E2M3
 *            code of c / 2, value i at bits 6 i .. 6 i + 5; bytes
 *            48 Np + 8 (u Np + n) .. the words (dw_hi | dw_hi << 16,
 *            dw_lo | dw_lo << 16), bytes 64 Np + 8 (u Np + n) .. the word
 *            (mw_hi | mw_lo << 16) twice, dw = d sc and mw = -dmin m split into bf16
 *            hi + lo as in the Xq fp6 section.  mq_gemm (any M) reads it with
 *            the fp6 kernel; the product agrees with the GGUF payload's within the
 *            2e-4 tolerance, not bit for bit (the scales are held to 16 bits), and
 *            its block dots are the same exact integers.  mq_gemv refuses it
 *            (MQ_ERR_TYPE): decode reads the GGUF payload.
 * Other types have no repacked layout: MQ_ERR_TYPE, and mq_repack_bytes returns
 * 0.
 * MQ_Q4_K | MQ_ROW_TILED (instead of MQ_REPACKED) asks for Q4_K's row-tiled
 * layout, for the GEMV of rows of more than 16 super-blocks (K > 4096; else
 * MQ_ERR_SHAPE): rows in groups of R = min(16, ceil(N / 256)); a group stores
 * its R rows' 144-byte super-block 0 blocks one after another (row order),
 * then their super-block 1 blocks, and so on, groups in order, the last group
 * filled with zero rows (mq_repack_bytes = ceil(N / R) R (K / 256) 144).  One
 * group's super-block is then one contiguous run of R x 144 bytes.  mq_gemv
 * reads it with type MQ_Q4_K | MQ_ROW_TILED and gives the GGUF payload's
 * result bit for bit; mq_gemm refuses it (MQ_ERR_TYPE).
 * W and Wr must be 16-byte aligned and must not overlap (MQ_ERR_ARG).  Runs on
 * `stream`; W may be freed once the stream has passed the call.
 */
size_t mq_repack_bytes(int type, int64_t N, int64_t K);
int mq_repack(const void* W, int type, int64_t N, int64_t K, size_t nbytes, void* Wr, size_t wr_bytes,
              void* stream);

/* Bytes of the quantized activation plane for M x K, and the offsets of its
 * scale, sum and fp6 arrays (each 256-byte aligned).  0 if K % 32 != 0. */
size_t mq_act_bytes(int64_t M, int64_t K);
size_t mq_act_scale_offset(int64_t M, int64_t K);
size_t mq_act_sum_offset(int64_t M, int64_t K);
size_t mq_act_f6_offset(int64_t M, int64_t K);

/*
 * mq_quantize_act -- X f32 [M][K] (device) -> Xq (device, mq_act_bytes(M, K)
 * bytes) per the Xq layout above [EP-C4; BD4.4].  K % 32 == 0.  The output is
 * bit-exact: the same codes, scales and sums as the definition for any finite
 * X.  X must be finite (NaN/Inf are outside the contract).
 */
int mq_quantize_act(const float* X, void* Xq, int64_t M, int64_t K, void* stream);

/*
 * mq_gemv -- y[n] = sum_k deq(W)[n][k] * x[k] for a single f32 activation row
 * (the decode product, [BD4.4]).  W: mq_weight_bytes(type, N, K) bytes of GGUF
 * payload (device, 16-byte aligned); x: K f32 (device); y: N f32 (device,
 * overwritten).  K must be a multiple of the block size (32 or 256) [BD4.3].
 * f32 accumulation; the result is within 2e-4 of the exact product relative to
 * ||deq(W)[n]|| * ||x||.
 */
int mq_gemv(const void* W, int type, const float* x, float* y, int64_t N, int64_t K, void* stream);

/*
 * mq_gemm_scratch_bytes -- device scratch that mq_gemm needs for (type, M, N,
 * K); 0 when the chosen work split needs none, and 0 for a shape mq_gemm
 * refuses.  The int8 kernel (every type on the GGUF payload) computes Y in
 * BM x 128 tiles, sized for 512 resident workgroups: BM = 128, or 32 when
 * M <= 32 or when the 128-row tiles would be at most 256.  Tiles are computed
 * whole while they fill rounds of 512; the tiles of a last round that is at
 * most half full (or all tiles, when there are at most 256) are cut into S
 * ranges of whole 128-value K-steps (at least 2 per range, ranges for at most
 * 256 workgroups).  The fp6 kernel
 * (MQ_Q4_K | MQ_REPACKED) computes 128 x 128 tiles with two workgroups per CU
 * (rounds of 512, 64-value K-steps, at least 4 per range, ranges for at most 256
 * workgroups).  Both sum a cut
 * tile's S f32 partial tiles in the same launch, in range order
 * (deterministic): the scratch is 1 KiB of uint32 counters (one per cut tile;
 * no plan cuts more than 256), which must be zero before the first call and
 * which every call leaves at zero, followed by S x (cut tiles) x (tile rows x
 * tile columns) f32.  The counters sit at the start for every shape, so calls
 * of different shapes may share one buffer.  The split depends on the shape
 * only, never on the device.  Q4_K on the GGUF payload, when the int8 kernel
 * would take at most 256 tiles of 32 x 128 and its ranges would not be more
 * than 5 K-steps shorter than a quarter of K's steps (e.g. the 7B attn_k and
 * attn_v products at M = 512), runs instead one 32 x 32 tile per workgroup
 * with the K range split over its four waves and summed in LDS (in wave
 * order, deterministic): no scratch (0 here).
 */
size_t mq_gemm_scratch_bytes(int type, int64_t M, int64_t N, int64_t K);

/*
 * mq_gemm -- the prefill product on the int8 path [BD4.4]:
 *   Y[m][n] = sum_b scale_x[m][b] * sum_{i<32} deq(W)[n][32b+i] * code_x[m][32b+i]
 * Xq is a plane written by mq_quantize_act(.., M, K, ..) (it may be reused for
 * several weights that share the input).  Per 32-value block the kernel forms
 * exact int32 dot products of weight codes and activation codes on int8 MFMA
 * (per 16-value group for Q6_K) and applies the block scales in f32 (and, for
 * Q4_K, Q5_K, Q4_1 and Q5_1, the min term through the block's code sum).  Y: M x N f32 (device,
 * overwritten).  scratch / scratch_bytes: device memory of at least
 * mq_gemm_scratch_bytes(type, M, N, K) bytes, 16-byte aligned (may be NULL/0
 * when that is 0), zeroed before its first use (the counters); its partial
 * tiles are overwritten, and calls that share one scratch buffer must be
 * ordered on one stream.  MQ_ERR_SIZE when it is too small, MQ_ERR_ALIGN when
 * misaligned.
 */
int mq_gemm(const void* W, int type, const void* Xq, float* Y, int64_t M, int64_t N, int64_t K,
            void* scratch, size_t scratch_bytes, void* stream);

/* Partial-tile bytes of mq_gemm_noalloc's per-device scratch array. */
#define MQ_NOALLOC_PARTIAL_BYTES (32u << 20)

/*
 * mq_gemm_noalloc -- mq_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same product, kernels and result bits as mq_gemm, with the
 * work split's scratch taken from an array the library holds on each device
 * (MQ_NOALLOC_PARTIAL_BYTES of partial tiles plus 4 KiB of counters; each
 * device that the library runs on holds it until the process ends).  The call
 * allocates and frees nothing; the caller still passes W, Xq and Y as for
 * mq_gemm.  Every call on a device shares that device's array: calls that may
 * overlap on one device (two streams, or two host threads) race and give wrong
 * results; order them on one stream.  A shape whose partial tiles exceed the
 * array is refused with MQ_ERR_SIZE (no valid shape does: a plan cuts at most
 * 32 MiB of tiles).  The array's address is taken, and its counters cleared,
 * the first time mq_init succeeds on the device.
 */
int mq_gemm_noalloc(const void* W, int type, const void* Xq, float* Y, int64_t M, int64_t N, int64_t K,
                    void* stream);

/*
 * mq_debug_lds_bytes -- test helper: the LDS sizes the kernels are built and
 * launched with, computed on the host from the same formulas and structs the
 * kernels use ("minfer CUDA Backend Design", 2.4: one shared-memory formula per
 * kernel, checked by tests).  No device is needed.  Returns 0 for an unknown
 * `what`, type or K.
 *   MQ_LDS_GEMV_FIXED       vector GEMV, bytes besides the row tile (staged x
 *                           digit planes, block exponents and sums) for (type, K)
 *   MQ_LDS_GEMV_TILE_UNITS  vector GEMV, row-tile units (4 bytes each) that fit
 *                           next to them in MQ_GFX950_LDS_BYTES
 *   MQ_LDS_MMQ_I8_BM128 / _BM32  int8 MMQ workgroup LDS for the type at 128- /
 *                           32-row tiles (two workgroups share a CU)
 *   MQ_LDS_MMQ_F6           fp6 MMQ (Q4_K plane) workgroup LDS (two workgroups per CU)
 *   MQ_LDS_MMQ_KW           Q4_K MMQ with the K range over a workgroup's waves: the
 *                           LDS where the waves' partial tiles meet
 */
#define MQ_GFX950_LDS_BYTES (160 * 1024)
#define MQ_LDS_GEMV_FIXED 0
#define MQ_LDS_GEMV_TILE_UNITS 1
#define MQ_LDS_MMQ_I8_BM128 2
#define MQ_LDS_MMQ_I8_BM32 3
#define MQ_LDS_MMQ_F6 5
#define MQ_LDS_MMQ_KW 6
size_t mq_debug_lds_bytes(int what, int type, int64_t K);

/*
 * mq_debug_gemm_blockdots -- test export: the exact int32 block dot products
 * the mq_gemm kernel forms, written to D (device) as int32 [M][N][G] with
 * G = K / 16 for Q6_K (dot of (code - 32) per 16-value group) and G = K / 32
 * for every other type (dot per 32-value block of: the signed q of Q8_0;
 * code - 8 of Q4_0; code - 16 of Q5_0; the unsigned code of Q4_1, Q5_1, Q4_K
 * (0..15) and Q5_K (0..31)).  Runs the
 * same kernel template as mq_gemm with its store of block dots switched on.
 * D must hold M * N * G int32.
 */
int mq_debug_gemm_blockdots(const void* W, int type, const void* Xq, int32_t* D,
                            int64_t M, int64_t N, int64_t K, void* stream);

/*
 * mq_debug_refuse_launches -- test helper for the MQ_ERR_LAUNCH path: the
 * next `count` launching calls on this thread take the path of a launch the
 * runtime refused (their kernels are not launched; the call returns
 * MQ_ERR_LAUNCH with a message naming the call and the kernel, and its
 * outputs are unspecified).  count = 0 turns it off.  Returns MQ_OK, or
 * MQ_ERR_ARG for a negative count.
 */
int mq_debug_refuse_launches(int count);

/*
 * mq_last_error -- the message of the last failing call on this thread (empty
 * string if none).  Valid until the next failing call on the same thread.
 */
const char* mq_last_error(void);

/* LDS bytes one workgroup may use on the current device (0 before mq_init). */
int mq_device_lds_bytes(void);

/* Name of the kernel the last successful launching call on this thread ran
 * (for tests that must prove which path executed).  The path is a function of
 * the type, the shape, the layout and the 16-byte alignment of W:
 *   "quantize_act", "repack";
 *   mq_gemv: "gemv_mfma<q4_K>" (wide: at least two 16-row tiles per CU, 12..16
 *     super-blocks per row), "gemv_mfma_long<q4_K>" (more than 16 super-blocks,
 *     8..16 rows per CU), "gemv_mfma_long<q4_K row-tiled>" (MQ_Q4_K |
 *     MQ_ROW_TILED), "gemv_mfma<q6_K>" (wide, GGUF layout, matrix ending
 *     on a 16-byte boundary), "gemv_mfma<q8_0>" / "gemv_mfma<q4_0>" /
 *     "gemv_mfma<q5_0>" (wide, GGUF layout), else "gemv<type>" (with " repacked" for MQ_REPACKED);
 *   mq_gemm: "mmq_f6<q4_K plane>" (MQ_Q4_K | MQ_REPACKED, any M),
 *     "gemv_q8_mfma<q6_K>" (M <= 8, Q6_K, as gemv_mfma<q6_K>),
 *     "gemv_q8<type>" (other M <= 8 shapes that fit LDS), "mmq_kw<q4_K>" (Q4_K,
 *     GGUF payload, few output tiles: see mq_gemm_scratch_bytes), else "mmq<type>". */
const char* mq_last_kernel(void);

/* Library version string. */
const char* mq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
