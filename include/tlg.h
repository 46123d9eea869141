/*
 * tlg: C = ReLU(A . B) on AMD Instinct MI355X (gfx950).
 *
 * The operation is TileLang's quick-start kernel `matmul_relu` (TileLang
 * article, aiwiki.ai/wiki/tilelang, section "Programming model", the listing):
 * A is an (M, K) float16 matrix and B a (K, N) float16 matrix; the products
 * are accumulated in float32 over the whole K range; ReLU is applied to the
 * float32 accumulator; the result is written to the float16 (M, N) matrix C.
 * Tile sizes, pipeline depth and thread counts are schedule choices of the
 * library and never change what is computed.
 *
 * Conventions for every entry point below:
 *   - Matrices are row-major with leading dimensions in ELEMENTS:
 *       A[i][k] is at A + i*lda + k,  B[k][j] at B + k*ldb + j,
 *       C[i][j] at C + i*ldc + j.
 *   - A, B and C are DEVICE pointers on the handle's GPU, IEEE binary16,
 *     at least 2-byte aligned. The caller owns them. Any alignment and any
 *     leading dimension is accepted; 16-byte-aligned pointers with leading
 *     dimensions, K and N all multiples of 8 select the fastest kernels.
 *   - C is overwritten inside its M x N window only; elements of a padded
 *     row beyond column N are never written. C must not overlap A or B.
 *   - Calls are asynchronous: work is enqueued on `stream` (0 = the null
 *     stream) and the call returns at once; results are visible once the
 *     caller synchronises that stream. No entry point allocates device
 *     memory except tlg_create, and none synchronises the device.
 *   - Rounding: float32 sums in an order chosen by the kernel; ReLU maps
 *     every value that is not > 0 to +0; the float32 -> float16 conversion
 *     rounds to nearest, ties to even, keeps subnormals and overflows to
 *     +infinity.
 *   - No C++ exception crosses this interface.
 */
#ifndef TLG_H
#define TLG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tlg_context *tlg_handle; /* opaque */

typedef enum {
    TLG_SUCCESS = 0,
    TLG_ERROR_INVALID_VALUE = 1, /* a bad argument; nothing was enqueued */
    TLG_ERROR_NOT_SUPPORTED = 2, /* the device is not gfx950, or a request the library cannot serve */
    TLG_ERROR_OUT_OF_MEMORY = 3, /* tlg_create could not allocate its workspace */
    TLG_ERROR_HIP = 4            /* the HIP runtime reported an error (e.g. a launch failure) */
} tlg_status;

/* Kernel families the dispatcher can choose. */
typedef enum {
    TLG_VARIANT_AUTO = 0,          /* let tlg_gemm_relu choose (the default) */
    TLG_VARIANT_NOOP = 1,          /* M == 0 or N == 0: nothing to do */
    TLG_VARIANT_FILL_ZERO = 2,     /* K == 0: C = +0 (the empty sum after ReLU) */
    TLG_VARIANT_TILED_DMA = 3,     /* MFMA tiles fed by direct global->LDS loads; needs the aligned fast-path conditions */
    TLG_VARIANT_TILED_GENERAL = 4, /* MFMA tiles fed through registers; any alignment and leading dimension */
    TLG_VARIANT_SPLITK = 5,        /* skinny M: K split across work-groups, fp32 partials, then an ordered reduce + ReLU + cast */
    TLG_VARIANT_NAIVE = 6,         /* one thread per output, sequential k; for cross-checks only, never chosen automatically */
    TLG_VARIANT_TILED_PIPE = 7,    /* MFMA tiles fed by direct global->LDS loads, loads and LDS reads slotted between MFMAs; aligned, large problems */
    TLG_VARIANT_PINGPONG = 8       /* wave-role schedule: two groups of waves alternate loads + LDS reads and MFMAs (forced only) */
} tlg_variant;

/* What tlg_gemm_relu will launch for a given problem (pure host logic). */
typedef struct {
    int32_t variant;          /* a tlg_variant */
    int32_t config;           /* tile configuration index inside the variant (see tlg_plan_config_name) */
    int32_t block_m, block_n, block_k; /* output tile and K step of one work-group (0 if none) */
    int32_t threads;          /* threads per work-group */
    int32_t splits;           /* K splits (1 unless variant == TLG_VARIANT_SPLITK) */
    int32_t kernels;          /* kernel launches per call */
    int64_t grid;             /* work-groups of the main kernel */
    int64_t workspace_bytes;  /* bytes of the handle's fp32 workspace the call uses */
} tlg_plan_info;

/* Creates a handle bound to the CURRENT HIP device. Checks that the device
 * is gfx950 (TLG_ERROR_NOT_SUPPORTED otherwise), allocates the handle's
 * split-K workspace (TLG_ERROR_OUT_OF_MEMORY on failure) and zeroes its
 * small counter area, waiting for the device to finish that
 * (TLG_ERROR_HIP on failure). *out is set only on success. One handle may be
 * used by one stream at a time, because calls on it share its workspace. */
tlg_status tlg_create(tlg_handle *out);

/* Releases the handle and its workspace. NULL is a no-op. The caller must
 * make sure no call enqueued with the handle is still running. */
tlg_status tlg_destroy(tlg_handle h);

/* C = ReLU(A . B) (the quick-start `matmul_relu` of the TileLang article,
 * "Programming model"). M, N, K >= 0. lda >= max(1, K), ldb >= max(1, N),
 * ldc >= max(1, N). M == 0 or N == 0: success, nothing enqueued. K == 0:
 * every C element in the window becomes +0. A, B and C may be NULL only when
 * nothing would be read or written through them. Returns
 * TLG_ERROR_INVALID_VALUE (nothing enqueued) for a NULL handle, negative
 * sizes, a leading dimension below the row width, a needed NULL pointer or a
 * pointer that is not 2-byte aligned; TLG_ERROR_NOT_SUPPORTED (nothing
 * enqueued) when M, N or K exceeds 2^31 - 1024 or the launch would need more
 * than 2^31 - 1 work-groups (an output of more than 2^45 elements);
 * TLG_ERROR_HIP if a launch fails. Device faults surface when the caller
 * synchronises. */
tlg_status tlg_gemm_relu(tlg_handle h, int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda,
                         const void *B, int64_t ldb,
                         void *C, int64_t ldc,
                         hipStream_t stream);

/* Same operation as tlg_gemm_relu with a forced kernel family, tile
 * configuration and split count, for tests and measurements: variant is a
 * tlg_variant (AUTO picks as tlg_gemm_relu does, and then config must be -1);
 * config is the index of one of the variant's tile configurations (names from
 * tlg_plan_config_name) or -1 to let the library choose; splits <= 0 lets the
 * library choose. Returns TLG_ERROR_INVALID_VALUE for an unknown variant or
 * configuration, TLG_ERROR_NOT_SUPPORTED if the forced variant cannot serve
 * the problem (e.g. direct-to-LDS tiles on unaligned data); in both cases
 * nothing is enqueued. */
tlg_status tlg_gemm_relu_variant(tlg_handle h, int32_t variant, int32_t config, int32_t splits,
                                 int64_t M, int64_t N, int64_t K,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 void *C, int64_t ldc,
                                 hipStream_t stream);

/* Argument check used by tlg_gemm_relu, without a handle or a GPU (pure host
 * logic): TLG_SUCCESS or TLG_ERROR_INVALID_VALUE. */
tlg_status tlg_check_args(int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda,
                          const void *B, int64_t ldb,
                          const void *C, int64_t ldc);

/* The launch plan for a problem (pure host logic, no GPU needed). variant,
 * config and splits have the meaning of tlg_gemm_relu_variant; workspace_cap_bytes is
 * the workspace available (tlg_workspace_bytes() for a handle). Returns
 * TLG_ERROR_INVALID_VALUE for bad arguments, TLG_ERROR_NOT_SUPPORTED when the
 * forced variant cannot serve the problem. */
tlg_status tlg_plan(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    const void *C, int64_t ldc,
                    int32_t variant, int32_t config, int32_t splits, int64_t workspace_cap_bytes,
                    tlg_plan_info *out);

/* Name of a tile configuration reported by tlg_plan ("" if unknown). */
const char *tlg_plan_config_name(int32_t variant, int32_t config);

/* Bytes of workspace a handle allocates at creation (the split-K partials
 * and the stream-K tile counters). tlg_plan assumes a 256-CU device when it
 * sizes a stream-K grid; tlg_gemm_relu uses the handle's device. */
int64_t tlg_workspace_bytes(void);

/* 1 if a device architecture name (as in hipDeviceProp_t::gcnArchName, e.g.
 * "gfx950:sramecc+:xnack-") is one this library runs on, else 0. */
int32_t tlg_arch_supported(const char *gcn_arch_name);

/* A static description of a status code; never NULL. */
const char *tlg_status_string(tlg_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t tlg_version(void);

/* ---- allocation-free call ----
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. */

/* Bytes of the library's static per-device scratch array used by
 * tlg_gemm_relu_noalloc (64 KiB of split-kernel counters, 8 MiB of fp32
 * partials). */
#define TLG_NOALLOC_SCRATCH_BYTES ((int64_t)(64 << 10) + ((int64_t)8 << 20))

/* tlg_gemm_relu without a handle, allocating nothing: same operation,
 * arguments, checks and errors as tlg_gemm_relu on the CURRENT device (the
 * library's own choice of kernel). The split kernels' counters and partials
 * live in a static device array of TLG_NOALLOC_SCRATCH_BYTES that every GPU
 * the library runs on holds until the process ends; its address is looked
 * up on the first call on each device (which also checks that the device is
 * gfx950: TLG_ERROR_NOT_SUPPORTED otherwise). No hipMalloc, hipFree or other
 * allocating call is made, on the first call or later. Kernels are planned
 * to fit the scratch (fewer K splits than tlg_gemm_relu where a handle's
 * larger workspace would allow more); a plan that could not fit it is
 * refused with TLG_ERROR_NOT_SUPPORTED, nothing enqueued. The counter area
 * is cleared by a kernel on `stream` before each split kernel that uses it.
 * All calls on one GPU share its scratch array: calls that may overlap in
 * time on one GPU (other streams, other threads) race and must be ordered
 * by the caller. */
tlg_status tlg_gemm_relu_noalloc(int64_t M, int64_t N, int64_t K,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 void *C, int64_t ldc,
                                 hipStream_t stream);

/* TLG_NOALLOC_SCRATCH_BYTES, as built into the library. */
int64_t tlg_noalloc_scratch_bytes(void);

/* ---- layout and batching variants ----
 * The same operation with B given transposed, and several problems in one
 * launch. The forum post "TileLang: Writing Near-Hardware-Limit GPU Kernels
 * in 70 Lines of Python" (zhichai.net, "Key Technical Milestones") lists a
 * grouped GEMM with a transposed B matrix among the kernels built with the
 * DSL; the operation of each problem is still the quick-start matmul_relu. */

/* C = ReLU(A . Bt^T): Bt is the N x K fp16 row-major matrix (B transposed),
 * ldbt >= max(1, K); everything else as tlg_gemm_relu. B's tiles are loaded
 * and read like A's: by the pipelined kernel on 256 x 256 tiles when the
 * problem has at least 128 of them (16 x 16 x 32 MFMA when K is whole 64-deep
 * stages or there are at least 256 tiles, but not 257 to 319; else 32 x 32 x
 * 16; with K whole stages 192 x 256 or 128 x 256 tiles where they take fewer
 * rounds of work-groups, as tlg_gemm_relu does), else on 128 x 256 tiles
 * (16 x 16 x 32 MFMA) when it has at least 192 of those; with M at most 32
 * (K >= 512) or 64 (K >= 2048) and aligned data, by the column-strip split-K
 * kernel as tlg_gemm_relu; else by the direct-to-LDS tiled
 * kernel (tile by tile count). Any K and N. TLG_ERROR_NOT_SUPPORTED when a
 * tile's byte offsets exceed 2 GB (e.g. ldbt * 256 * 2 >= 2^31); nothing is
 * enqueued then. */
tlg_status tlg_gemm_relu_bt(tlg_handle h, int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda,
                            const void *Bt, int64_t ldbt,
                            void *C, int64_t ldc,
                            hipStream_t stream);

/* tlg_gemm_relu_bt with a forced kernel family and tile configuration, for
 * tests and measurements: variant TLG_VARIANT_AUTO (then config must be -1),
 * TLG_VARIANT_TILED_DMA (configs 0..2), TLG_VARIANT_TILED_PIPE (configs 2,
 * 4 and 7, the 256 x 256 ones with a third A buffer, and the 16 x 16 x 32
 * MFMA tiles 17 (256 x 256), 21 (128 x 256) and 26 (192 x 256)) or
 * TLG_VARIANT_SPLITK (the column-strip configurations 3..9 with the library's
 * parts per strip; M within the strip, 16-byte aligned pointers, leading
 * dimensions, K and N multiples of 8, else TLG_ERROR_NOT_SUPPORTED; split
 * strips use the handle's workspace); config -1 lets the library choose
 * inside the family. */
tlg_status tlg_gemm_relu_bt_variant(tlg_handle h, int32_t variant, int32_t config, int64_t M, int64_t N, int64_t K,
                                    const void *A, int64_t lda,
                                    const void *Bt, int64_t ldbt,
                                    void *C, int64_t ldc,
                                    hipStream_t stream);

/* What tlg_gemm_relu_bt(_variant) would launch (host only, no GPU), planned
 * for a handle's workspace of tlg_workspace_bytes() (only split strips use it;
 * out->workspace_bytes says how much). */
tlg_status tlg_plan_bt(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                       const void *Bt, int64_t ldbt, const void *C, int64_t ldc,
                       int32_t variant, int32_t config, tlg_plan_info *out);

/* One problem of a grouped call: C (M x N) = ReLU(A (M x K) . B), B being
 * K x N (ldb >= N) or, for a transposed call, N x K (ldb >= K). */
typedef struct {
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    void *C;
    int64_t ldc;
} tlg_gemm_desc;

#define TLG_GROUP_MAX 16

/* count independent problems (0 <= count <= TLG_GROUP_MAX; descs is a host
 * array the call reads before it returns) in one launch of the direct-to-LDS
 * tiled kernel: the work-groups of all problems share the device, so many
 * small problems (e.g. the experts of a mixture-of-experts layer) fill it
 * together. trans_b: 0 for K x N B matrices, 1 for N x K (transposed) ones,
 * the same for every problem. Each problem is checked as by tlg_check_args
 * (or its transposed form); any failure returns TLG_ERROR_INVALID_VALUE (or
 * TLG_ERROR_NOT_SUPPORTED for offsets beyond 2 GB) and enqueues nothing.
 * Problems with M or N = 0 are skipped, K = 0 writes +0. The C windows must
 * not overlap each other or any A or B. count = 0 is a no-op. */
tlg_status tlg_gemm_relu_grouped(tlg_handle h, int32_t count, const tlg_gemm_desc *descs, int32_t trans_b,
                                 hipStream_t stream);

/* tlg_gemm_relu_grouped with a forced tile configuration: -1 the library's
 * choice (from 128 tiles of 256 x 256 in total the pipelined kernel, in its
 * 16 x 16 x 32 form when every K is a multiple of 64 and, B not transposed,
 * every N a multiple of 8, else in its 32 x 32 x 16 form; below, the
 * direct-to-LDS tiles by tile count); 0, 1, 2 the direct-to-LDS
 * 256 x 256 x 32, 128 x 128 x 32 and 64 x 64 x 64 tiles; 3 the eight-wave
 * 32 x 32 x 16 pipelined 256 x 256 x 64 kernel; 4 the four-wave
 * 16 x 16 x 32 pipelined 256 x 256 x 64 kernel (any K; B not transposed:
 * every N a multiple of 8, TLG_ERROR_NOT_SUPPORTED otherwise). */
tlg_status tlg_gemm_relu_grouped_variant(tlg_handle h, int32_t config, int32_t count, const tlg_gemm_desc *descs,
                                         int32_t trans_b, hipStream_t stream);

/* ---- Block-scaled (MX) element formats ----
 *
 * The project page "TileLang: a tile-level DSL for writing GPU kernels in
 * Python" (hysenlabs.com, "Three backends under one language dialect") names
 * FP4 E2M1 matrix cores on CDNA4 (gfx950) and a block-scaled MMA path; the
 * forum post "TileLang: Writing Near-Hardware-Limit GPU Kernels in 70 Lines
 * of Python" (zhichai.net, "Key Technical Milestones") names MXFP8 grouped
 * GEMM with block scaling and a transposed B. Neither page defines the
 * formats; they are read as the OCP Microscaling (MX) formats:
 *
 *   C[i][j] = fp16_rne( ReLU( sum over blocks b = 0 .. K/32-1 of
 *               2^(SA[i][b]-127) * 2^(SB[j][b]-127)
 *               * sum over k = 32b .. 32b+31 of a[i][k] * b[j][k] ) )
 *
 * with a and b decoded from their element codes, the sum accumulated in fp32
 * on the matrix cores, ReLU on the fp32 value and the fp16 copy-out rounding
 * to nearest even (the quick-start kernel's epilogue). Scale bytes are E8M0
 * (255 is NaN; ReLU then gives +0). Element codes that are NaN or infinite
 * give results the hardware defines (not specified here).
 *
 * Layout (all row-major):
 *   A  M x K element codes, lda elements per row (lda >= K);
 *   B  N x K element codes: B is given TRANSPOSED, so both operands are
 *      K-contiguous like their scale blocks (ldb >= K);
 *   SA M x K/32 scale bytes, ldsa bytes per row (ldsa >= K/32);
 *   SB N x K/32 scale bytes, ldsb bytes per row;
 *   C  M x N fp16, ldc elements per row (ldc >= N); only the M x N window
 *      is written.
 * 8-bit codes take one byte each; E2M1 codes are packed two per byte,
 * element 2t in the low nibble of byte t of the row (lda, ldb even).
 *
 * Requirements: K a multiple of 32 (else TLG_ERROR_INVALID_VALUE); K a
 * multiple of 128, A and B 16-byte aligned with rows a multiple of 16 bytes,
 * SA and SB 4-byte aligned with ldsa, ldsb multiples of 4, and C 2-byte
 * aligned (else TLG_ERROR_NOT_SUPPORTED). The caller owns every buffer;
 * nothing is allocated; the call is asynchronous on `stream`. M == 0 or
 * N == 0 is a no-op, K == 0 writes +0. */
typedef enum {
    TLG_MX_E4M3 = 1, /* 8-bit: 1 sign, 4 exponent (bias 7), 3 fraction bits; S.1111.111 is NaN */
    TLG_MX_E5M2 = 2, /* 8-bit: 1 sign, 5 exponent (bias 15), 2 fraction bits; IEEE-style inf/NaN */
    TLG_MX_E2M1 = 3  /* 4-bit: 1 sign, 2 exponent (bias 1), 1 fraction bit; packed two per byte */
} tlg_mx_format;

#define TLG_MX_BLOCK 32

/* C = ReLU(block-scaled A . B^T) as above, with the library's tile choice. */
tlg_status tlg_gemm_relu_mx(tlg_handle h, int32_t format, int64_t M, int64_t N, int64_t K, const void *A,
                            int64_t lda, const void *SA, int64_t ldsa, const void *B, int64_t ldb, const void *SB,
                            int64_t ldsb, void *C, int64_t ldc, hipStream_t stream);

/* tlg_gemm_relu_mx with a forced tile configuration (-1: library's choice;
 * 0: 256 x 256 tiles, eight waves; 1: 128 x 128 tiles, four waves;
 * 2: 256 x 256, eight waves, software-pipelined; 3: 256 x 256, four waves,
 * software-pipelined, 8-bit codes only, else TLG_ERROR_NOT_SUPPORTED). */
tlg_status tlg_gemm_relu_mx_variant(tlg_handle h, int32_t config, int32_t format, int64_t M, int64_t N, int64_t K,
                                    const void *A, int64_t lda, const void *SA, int64_t ldsa, const void *B,
                                    int64_t ldb, const void *SB, int64_t ldsb, void *C, int64_t ldc,
                                    hipStream_t stream);

/* What tlg_gemm_relu_mx(_variant) would launch (host only, no device call):
 * the same checks and status codes; out->variant is TLG_VARIANT_TILED_DMA
 * (the block-scaled kernel), TLG_VARIANT_NOOP or TLG_VARIANT_FILL_ZERO, and
 * tlg_plan_mx_config_name names the configuration. */
tlg_status tlg_plan_mx(int32_t format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SA,
                       int64_t ldsa, const void *B, int64_t ldb, const void *SB, int64_t ldsb, const void *C,
                       int64_t ldc, int32_t config, tlg_plan_info *out);

/* Name of a block-scaled tile configuration ("" if out of range). */
const char *tlg_plan_mx_config_name(int32_t config);

/* One problem of a grouped block-scaled call: the arguments of
 * tlg_gemm_relu_mx (all problems of a call share the element format). */
typedef struct {
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const void *SA;
    int64_t ldsa;
    const void *B;
    int64_t ldb;
    const void *SB;
    int64_t ldsb;
    void *C;
    int64_t ldc;
} tlg_mx_desc;

/* Grouped block-scaled GEMM+ReLU with B transposed (the forum post's "Key
 * Technical Milestones" list names an MXFP8 grouped GEMM with block scaling
 * and a transposed B): count (0 .. TLG_GROUP_MAX) independent
 * problems, each as tlg_gemm_relu_mx, in ONE launch of the block-scaled
 * kernel. The descriptor array is read on the host during the call (it may
 * be freed afterwards); nothing is allocated. Every descriptor is checked as
 * tlg_gemm_relu_mx checks its arguments (TLG_ERROR_INVALID_VALUE /
 * TLG_ERROR_NOT_SUPPORTED); any failure enqueues nothing. Problems with
 * M == 0 or N == 0 are skipped; K == 0 problems are not accepted here
 * (TLG_ERROR_NOT_SUPPORTED). The C windows must not overlap each other or
 * any input. */
tlg_status tlg_gemm_relu_mx_grouped(tlg_handle h, int32_t format, int32_t count, const tlg_mx_desc *descs,
                                    hipStream_t stream);

/* tlg_gemm_relu_mx_grouped with a forced tile configuration (-1: library's
 * choice by total tile count; 0: 256 x 256; 1: 128 x 128). */
tlg_status tlg_gemm_relu_mx_grouped_variant(tlg_handle h, int32_t config, int32_t format, int32_t count,
                                            const tlg_mx_desc *descs, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TLG_H */
