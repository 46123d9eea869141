// Internal interface between the C-ABI host code and the gfx950 kernels.
#ifndef TLG_KERNELS_H
#define TLG_KERNELS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tlg.h"

namespace tlg {

// One GEMM+ReLU problem: C (M x N) = ReLU(A (M x K) . B (K x N)), fp16,
// row-major, leading dimensions in elements. trans_b: B is given as its
// transpose, N x K row-major (ldb >= K).
struct Problem {
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    void *C;
    int64_t ldc;
    bool trans_b = false;
};

// Most problems one grouped launch takes.
constexpr int kGroupMax = 16;

// Tile configurations. The index is what tlg_plan reports as `config`.
struct TileConfig {
    int bm, bn, bk, threads, stages;
    const char *name;
};
// direct-to-LDS (aligned) configurations
enum DmaConfig {
    DMA_256x256x32 = 0,
    DMA_128x128x32 = 1,
    DMA_64x64x64 = 2,
    DMA_256x256x64_W8 = 3,  // eight waves, two per SIMD
    DMA_256x256x32_W8 = 4,
    DMA_CONFIGS = 5
};
// register-staged (any alignment) configurations
enum GenConfig { GEN_128x128x32 = 0, GEN_64x64x32 = 1, GEN_CONFIGS = 2 };
// split-K partial kernels (direct-to-LDS, aligned)
// (indices 0 and 1: two kernels, partials then an ordered reduce; index 2:
// one stream-K kernel that finishes split tiles itself; indices 3 and up:
// column strips, K split among work-groups and their waves, M <= 32)
enum SplitConfig { SPLIT_32x128x64 = 0, SPLIT_32x256x64 = 1, SPLIT_TWO_KERNEL_CONFIGS = 2,
                   SPLIT_STREAMK_32x128x64 = 2, SPLIT_WAVES_32x64x64 = 3, SPLIT_WAVES_32x64x64_W4 = 4,
                   SPLIT_WAVES_32x64x64_S4 = 5, SPLIT_WAVES_32x128x64 = 6, SPLIT_WAVES_32x128x64_W4 = 7,
                   SPLIT_WAVES_32x256x32 = 8, SPLIT_WAVES_64x64x64 = 9, SPLIT_STRIP_SK_32x64x64 = 10,
                   SPLIT_STRIP_SK_32x64x64_S2 = 11, SPLIT_CONFIGS = 12 };
// strip configuration j is split configuration SPLIT_WAVES_32x64x64 + j
constexpr int STRIP_CONFIGS = SPLIT_STRIP_SK_32x64x64 - SPLIT_WAVES_32x64x64;
inline bool is_strip_config(int config) { return config >= SPLIT_WAVES_32x64x64 && config < SPLIT_STRIP_SK_32x64x64; }
// stream-K strip configuration j is split configuration SPLIT_STRIP_SK_32x64x64 + j
inline bool is_strip_sk_config(int config) { return config >= SPLIT_STRIP_SK_32x64x64 && config < SPLIT_CONFIGS; }
// software-pipelined direct-to-LDS kernels (aligned, large problems)
enum PipeConfig {
    PIPE_256x256x32 = 0,
    PIPE_256x256x64 = 1,
    PIPE_256x256x64_A3 = 2,
    PIPE_256x256x64_W8 = 3,  // eight waves, two per SIMD
    PIPE_256x256x64_W8_A3 = 4,
    PIPE_256x128x64 = 5,  // four waves of 128 x 64, three stages
    PIPE_128x256x64 = 6,
    PIPE_256x256x64_W8_A3_EARLY = 7,  // stage barrier before the last half k-step (the default)
    PIPE_256x256x64_W8_B3_EARLY = 8,  // two A buffers, three B buffers
    PIPE_256x256x64_B3 = 9,           // four waves, two A buffers, three B buffers
    // v_mfma_f32_16x16x32_f16 tiles (any K and N; with B transposed
    // configurations 17, 21 and 26): four waves of 128 x 128 (128 x 256
    // tiles: four waves of 128 x 64)
    PIPE16_FIRST = 10,
    PIPE16_256x256x64_A3 = 10,
    PIPE16_256x256x64_A3_EARLY = 11,
    PIPE16_256x256x64_B3 = 12,
    PIPE16_256x256x64_A3_SP2 = 13,
    PIPE16_256x256x64_A3_SP6 = 14,
    PIPE16_256x256x64_A3_EARLY_SP2 = 15,
    PIPE16_256x256x64_A3_SP7 = 16,
    PIPE16_256x256x64_A3_SP8 = 17,
    PIPE16_256x256x64_A3_SP6_D5 = 18,
    PIPE16_256x256x64_B3_SP6 = 19,
    PIPE16_256x256x64_A3_EARLY_SP6 = 20,
    PIPE16_128x256x64_A3 = 21,  // four waves of 128 x 64
    PIPE16_128x256x64_A4 = 22,
    // eight waves of 128 x 64, two per SIMD
    PIPE16_256x256x64_W8_A3_SP8 = 23,
    PIPE16_256x256x64_W8_A3_SP4 = 24,
    PIPE16_256x256x64_W8_A3_EARLY_SP6 = 25,
    // 192 x 256 tiles, four waves of 96 x 128: a third more tiles than
    // 256 x 256 where those leave CUs idle
    PIPE16_192x256x64_A3_SP6 = 26,
    PIPE16_192x256x64_A3_SP7 = 27,
    PIPE_CONFIGS = 28
};

// wave-role (ping-pong) schedule: two groups of waves alternate between
// loads + fragment reads and MFMAs, slot by slot
enum PingPongConfig { PINGPONG_256x256x32 = 0, PINGPONG_CONFIGS = 1 };

extern const TileConfig kDmaConfigs[DMA_CONFIGS];
extern const TileConfig kPingPongConfigs[PINGPONG_CONFIGS];
extern const TileConfig kGenConfigs[GEN_CONFIGS];
extern const TileConfig kSplitConfigs[SPLIT_TWO_KERNEL_CONFIGS];
extern const TileConfig kPipeConfigs[PIPE_CONFIGS];

// Launchers: enqueue on `stream`, return the launch status.
hipError_t launch_tiled_dma(int config, const Problem &p, hipStream_t stream);
// count (1 .. kGroupMax) problems, all with the same trans_b, in one launch
// of the direct-to-LDS kernel (each must pass the direct-to-LDS checks)
hipError_t launch_tiled_dma_grouped(int config, const Problem *ps, int count, hipStream_t stream);
hipError_t launch_tiled_general(int config, const Problem &p, hipStream_t stream);
hipError_t launch_tiled_pipe(int config, const Problem &p, hipStream_t stream);
// the 16 x 16 x 32 MFMA configurations (PIPE16_FIRST and up); with B
// transposed only 17, 21 and 26 (hipErrorInvalidValue otherwise)
hipError_t launch_tiled_pipe16(int config, const Problem &p, hipStream_t stream);
// count (1 .. kGroupMax) problems, all with the same trans_b, in one launch
// of the eight-wave early-barrier pipelined kernel (each must pass its checks)
hipError_t launch_tiled_pipe_grouped(const Problem *ps, int count, hipStream_t stream);
// count (1 .. kGroupMax) problems, all with the same trans_b, in one launch of
// the default 16 x 16 x 32 pipelined configuration
hipError_t launch_tiled_pipe16_grouped(const Problem *ps, int count, hipStream_t stream);
hipError_t launch_pingpong(int config, const Problem &p, hipStream_t stream);
// Stage 1 writes fp32 partials W[s][m][n] (M x N packed per split) for
// splits s covering k in [s*k_split, (s+1)*k_split); stage 2 sums them in
// ascending s, applies ReLU and the fp16 cast, and writes C.
hipError_t launch_splitk(int config, int splits, int64_t k_split, const Problem &p, float *workspace,
                         hipStream_t stream);
// Stream-K split of K for skinny problems: `grid` work-groups take equal
// ranges of the (tile, k) iteration sequence; split tiles are finished in the
// same kernel through `partials` (grid x 2 x BM x BN fp32) and `counters`
// (one int per tile, zero on entry and on exit).
extern const TileConfig kStreamKConfig;
constexpr int kStreamKBlocksPerCU = 2;  // 80 KiB of LDS per work-group, 160 KiB per CU
hipError_t launch_streamk(const Problem &p, int grid, float *partials, int *counters, hipStream_t stream);
// Skinny strips (M <= 32): `parts` work-groups per strip of bn columns, each
// taking a contiguous part of K split among its waves and reduced in LDS in
// wave order; with parts > 1 the parts meet through `partials` (strips x
// parts x bm x bn fp32) and `counters` (one int per strip, zero on entry and
// exit). `config` indexes kStripConfigs; kStripConfig is the default.
extern const TileConfig kStripConfigs[STRIP_CONFIGS];
extern const TileConfig &kStripConfig;
hipError_t launch_skinny_strip(int config, const Problem &p, int parts, float *partials, int *counters,
                               hipStream_t stream);
// Stream-K over strips (M <= 32, at most `grid` strips): the strips' K blocks
// in one strip-major sequence, split into `grid` equal ranges; a strip split
// between ranges is finished in the kernel through `partials` (grid x 2 x
// bm x bn fp32) and `counters` (one int per strip, zero on entry and exit).
constexpr int STRIP_SK_CONFIGS = 2;
extern const TileConfig kStripSkConfigs[STRIP_SK_CONFIGS];
hipError_t launch_skinny_strip_sk(int config, const Problem &p, int grid, float *partials, int *counters,
                                  hipStream_t stream);
// Block-scaled (MX) problem: A (M x K codes) and B (N x K codes, i.e. B
// transposed), their scale bytes (M x K/32, N x K/32), fp16 C. Leading
// dimensions of A and B in elements (codes), of the scales in bytes, of C
// in elements. format: 1 E4M3, 2 E5M2, 3 E2M1 (two codes per byte).
struct MxProblem {
    int format;
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
};
enum MxConfig { MX_256x256_W8 = 0, MX_128x128_W4 = 1, MX_PIPE_256x256_W8 = 2, MX_PIPE_256x256_W4 = 3, MX_CONFIGS = 4 };
extern const TileConfig kMxConfigs[MX_CONFIGS];  // bk: bytes of K per stage and row
hipError_t launch_mx(int config, const MxProblem &p, hipStream_t stream);
// count (1 .. kGroupMax) block-scaled problems of one format in one launch
// (configurations MX_256x256_W8 and MX_128x128_W4)
hipError_t launch_mx_grouped(int config, const MxProblem *ps, int count, hipStream_t stream);

hipError_t launch_naive(const Problem &p, hipStream_t stream);
hipError_t launch_fill_zero(const Problem &p, hipStream_t stream);
// Sets `words` 32-bit words at `p` to zero (a kernel, so that it can be
// captured in a graph like the calls it precedes).
hipError_t launch_clear_words(int *p, int64_t words, hipStream_t stream);

// The first kCounterBytes of a workspace hold the split kernels' per-tile and
// per-strip counters; fp32 partials follow.
constexpr int64_t kCounterBytes = 64ll << 10;

// Plans one call (C = ReLU(A . B), any variant) for a device with `cus`
// compute units and `workspace_bytes` of workspace at `workspace` (device
// memory, counters first), and enqueues it on `stream`. With clear_counters
// the counter area is cleared on the stream before a split kernel that uses
// it. The caller has checked that the device is current and supported.
tlg_status run_with_workspace(float *workspace, int64_t workspace_bytes, int cus, bool clear_counters,
                              int32_t variant, int32_t config, int32_t splits, const Problem &p,
                              hipStream_t stream);
tlg::Problem make_problem_c(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                            void *C, int64_t ldc);

}  // namespace tlg

#endif
