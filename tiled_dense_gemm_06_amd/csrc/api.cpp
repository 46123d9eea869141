// C ABI of the tlg library: handle, argument checks, kernel choice, launch.
// The operation is the quick-start `matmul_relu` of the TileLang article
// (aiwiki.ai/wiki/tilelang, "Programming model"); see include/tlg.h for the
// contract of every entry point.
#include "tlg.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include "kernels.h"

struct tlg_context {
    int device;
    int cus;            // compute units of the device
    float *workspace;   // kCounterBytes of stream-K tile counters, then fp32 partials
    int64_t workspace_bytes;
};

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0
// fp32 split-K partials: 32 MiB covers S x M x N x 4 bytes for the skinny
// shapes the split path serves (S is lowered when a shape needs more).
constexpr int64_t kWorkspaceBytes = 32ll << 20;
// The first kCounterBytes (64 KiB) of the workspace hold the stream-K
// per-tile counters (zeroed once at creation; every call leaves them zero);
// partials follow.
using tlg::kCounterBytes;
constexpr int kPlanCUs = 256;  // tlg_plan plans for a 256-CU MI355X
// Largest in-tile byte offset a buffer load may use (see the kernels).
constexpr int64_t kMaxOffset = 0x7ffffff0ll - 16;
constexpr int64_t kMaxDim = (1ll << 31) - 1024;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// In-tile byte offsets of the direct-to-LDS kernels fit a buffer descriptor.
bool offsets_ok(const tlg::Problem &p, int bm, int bn, int bk) {
    if ((int64_t)bm * p.lda * 2 > kMaxOffset) return false;  // A tile loads
    if ((int64_t)bk * p.ldb * 2 > kMaxOffset) return false;  // B tile loads
    if ((int64_t)bm * p.ldc * 2 + (int64_t)bn * 2 > kMaxOffset) return false;  // C tile stores
    if ((int64_t)bm * p.N * 4 + (int64_t)bn * 4 > kMaxOffset) return false;    // split-K partial stores
    return true;
}

// The tiled and pipelined direct-to-LDS kernels take any 2-byte aligned data
// (gfx950 buffer loads and stores accept any 2-byte aligned offset). When K
// or N is not a multiple of 8 the loads stop at the largest multiple of 8
// below K and the last rows come from a staged block; a 16-byte chunk that
// crosses the N edge of B must then stay inside the next row (ldb >= 8).
bool dma_ok(const tlg::Problem &p, int bm, int bn, int bk) {
    if (p.N % 8 != 0 && p.ldb < 8) return false;
    return offsets_ok(p, bm, bn, bk);
}

// The split-K, stream-K and strip kernels also need every 16-byte chunk
// wholly inside or outside the matrix: 16-byte aligned pointers, leading
// dimensions, K and N multiples of 8.
bool dma_ok_aligned(const tlg::Problem &p, int bm, int bn, int bk) {
    if (!aligned(p.A, 16) || !aligned(p.B, 16) || !aligned(p.C, 16)) return false;
    if (p.lda % 8 || p.ldb % 8 || p.ldc % 8 || p.K % 8 || p.N % 8) return false;
    return offsets_ok(p, bm, bn, bk);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tuned choices by shape class (see tiled_dense_gemm_06_amd/autotune.py).
struct TuneEntry {
    int lm, ln, lk, ragged;  // ceil(log2) of M, N, K; K or N not a multiple of 8
    int variant, config, splits;
};
#include "tune_table.inc"

int clog2(int64_t x) {
    int l = 0;
    while (l < 62 && (int64_t(1) << l) < x) ++l;
    return l;
}

const TuneEntry *tune_lookup(const tlg::Problem &p) {
    const int lm = clog2(p.M), ln = clog2(p.N), lk = clog2(p.K), rg = (p.K % 8 || p.N % 8) ? 1 : 0;
    for (const TuneEntry &e : kTuneTable)
        if (e.lm == lm && e.ln == ln && e.lk == lk && e.ragged == rg && e.variant != TLG_VARIANT_AUTO) return &e;
    return nullptr;
}

void fill_info(tlg_plan_info *o, int variant, int config, const tlg::TileConfig *tc, int splits, int kernels,
               int64_t grid, int64_t ws);

// K == 0: C = +0 by the fill kernel (256 threads per work-group, at most
// 65536 work-groups striding over the window). M and N must already be
// known to be at most kMaxDim, so M * N cannot overflow.
void fill_zero_info(tlg_plan_info *o, int64_t M, int64_t N) {
    int64_t blocks = (M * N + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    fill_info(o, TLG_VARIANT_FILL_ZERO, 0, nullptr, 1, 1, blocks, 0);
    o->threads = 256;
}

void fill_info(tlg_plan_info *o, int variant, int config, const tlg::TileConfig *tc, int splits, int kernels,
               int64_t grid, int64_t ws) {
    memset(o, 0, sizeof *o);
    o->variant = variant;
    o->config = config;
    if (tc) {
        o->block_m = tc->bm;
        o->block_n = tc->bn;
        o->block_k = tc->bk;
        o->threads = tc->threads;
    }
    o->splits = splits;
    o->kernels = kernels;
    o->grid = grid;
    o->workspace_bytes = ws;
}

// Split count for the skinny path: enough work-groups to give every CU about
// two, each split at least two K steps long, partials within the workspace.
bool choose_splits(const tlg::Problem &p, const tlg::TileConfig &tc, int32_t forced, int64_t cap, int *splits_out,
                   int64_t *k_split_out) {
    const int64_t tiles = ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn);
    const int64_t ksteps = ceil_div(p.K, tc.bk);
    int64_t s;
    if (forced > 0) {
        s = forced;
    } else {
        s = ceil_div(512, tiles);
        if (s > 16) s = 16;
        if (s > ksteps / 2) s = ksteps / 2;
        if (s < 1) s = 1;
    }
    if (s > ksteps) s = ksteps > 0 ? ksteps : 1;
    const int64_t per_split = p.M * p.N * 4;
    if (per_split > 0 && s * per_split > cap) s = cap / per_split;
    if (s < 1) return false;
    // splits cover K in whole K steps; recompute the count so none is empty
    int64_t k_split = ceil_div(ksteps, s) * tc.bk;
    if (k_split <= 0) k_split = tc.bk;
    s = p.K > 0 ? ceil_div(p.K, k_split) : 1;
    *splits_out = (int)s;
    *k_split_out = k_split;
    return true;
}

// A forced tile configuration index must exist for its variant.
bool config_ok(int32_t config, int count) { return config < 0 || config < count; }

// Every kernel takes one work-group per grid entry and computes its tile
// indices in 32-bit integers, so a plan whose grid exceeds INT32_MAX (only
// an output of more than 2^45 elements can ask for one) is refused.
tlg_status grid_fits(tlg_status st, const tlg_plan_info *o) {
    return st == TLG_SUCCESS && o->grid > 0x7fffffff ? TLG_ERROR_NOT_SUPPORTED : st;
}

// Strip configuration cfg (checked by the caller): parts per strip, forced,
// else as many as fit the CUs whole (1x4096x4096: 4 parts 12 us vs 1 part
// 23 us; 16x14336x4096: 1 part 25 us vs 2 parts 29 us), at most 4
// (16x2048x4096: 4 parts 10.3 us vs 8 parts 10.9 us), within the workspace.
void plan_strip_parts(const tlg::Problem &p, int cfg, int32_t splits, int64_t cap, int cus, tlg_plan_info *o) {
    const tlg::TileConfig &ts = tlg::kStripConfigs[cfg - tlg::SPLIT_WAVES_32x64x64];
    const int64_t strips = ceil_div(p.N, ts.bn);
    int64_t parts = splits > 0 ? splits : (strips >= cus ? 1 : cus / strips);
    if (splits <= 0 && parts > 4) parts = 4;
    const int64_t nkb = ceil_div(p.K, ts.bk);
    if (parts > nkb) parts = nkb > 0 ? nkb : 1;
    const int64_t slot_bytes = (int64_t)ts.bm * ts.bn * 4;
    if (parts > 1 && strips * parts * slot_bytes > cap) parts = cap / (strips * slot_bytes);
    if (parts < 1) parts = 1;
    if (parts > 1 && strips * 4 > kCounterBytes) parts = 1;
    const int64_t ws = parts > 1 ? kCounterBytes + strips * parts * slot_bytes : 0;
    fill_info(o, TLG_VARIANT_SPLITK, cfg, &ts, (int)parts, 1, strips * parts, ws);
}

tlg_status plan_select(const tlg::Problem &p, int32_t variant, int32_t config, int32_t splits, int64_t cap, int cus,
                       tlg_plan_info *o, int64_t *k_split_out);
tlg_status plan_impl(const tlg::Problem &p, int32_t variant, int32_t config, int32_t splits, int64_t cap, int cus,
                     tlg_plan_info *o, int64_t *k_split_out) {
    return grid_fits(plan_select(p, variant, config, splits, cap, cus, o, k_split_out), o);
}

tlg_status plan_select(const tlg::Problem &p, int32_t variant, int32_t config, int32_t splits, int64_t cap, int cus,
                       tlg_plan_info *o, int64_t *k_split_out) {
    cap -= kCounterBytes;
    *k_split_out = 0;
    if (variant < TLG_VARIANT_AUTO || variant > TLG_VARIANT_PINGPONG) return TLG_ERROR_INVALID_VALUE;
    if (variant == TLG_VARIANT_AUTO && config >= 0) return TLG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0) {
        fill_info(o, TLG_VARIANT_NOOP, 0, nullptr, 1, 0, 0, 0);
        return TLG_SUCCESS;
    }
    if (variant == TLG_VARIANT_NOOP) return TLG_ERROR_NOT_SUPPORTED;
    if (p.M > kMaxDim || p.N > kMaxDim || p.K > kMaxDim) return TLG_ERROR_NOT_SUPPORTED;
    if (variant == TLG_VARIANT_AUTO && p.K == 0) variant = TLG_VARIANT_FILL_ZERO;
    if (variant == TLG_VARIANT_FILL_ZERO) {
        if (p.K != 0) return TLG_ERROR_NOT_SUPPORTED;
        fill_zero_info(o, p.M, p.N);
        return TLG_SUCCESS;
    }
    if (variant == TLG_VARIANT_NAIVE) {
        if (ceil_div(p.M, 16) > 65535) return TLG_ERROR_NOT_SUPPORTED;
        fill_info(o, TLG_VARIANT_NAIVE, 0, nullptr, 1, 1, ceil_div(p.M, 16) * ceil_div(p.N, 16), 0);
        o->threads = 256;
        return TLG_SUCCESS;
    }

    // the wave-role (ping-pong) schedule: forced only (see its measurements)
    if (variant == TLG_VARIANT_PINGPONG) {
        if (!config_ok(config, tlg::PINGPONG_CONFIGS)) return TLG_ERROR_INVALID_VALUE;
        const int cfg = config >= 0 ? config : tlg::PINGPONG_256x256x32;
        const tlg::TileConfig &tc = tlg::kPingPongConfigs[cfg];
        if (!dma_ok(p, tc.bm, tc.bn, tc.bk)) return TLG_ERROR_NOT_SUPPORTED;
        fill_info(o, TLG_VARIANT_PINGPONG, cfg, &tc, 1, 1, ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn), 0);
        return TLG_SUCCESS;
    }

    // a tuned choice for the shape's class, if it can serve this problem
    if (variant == TLG_VARIANT_AUTO) {
        if (const TuneEntry *e = tune_lookup(p)) {
            if (plan_impl(p, e->variant, e->config, e->splits, cap + kCounterBytes, cus, o, k_split_out) ==
                TLG_SUCCESS)
                return TLG_SUCCESS;
            *k_split_out = 0;
        }
    }

    // split-K for skinny M: by default when M fits one 32-row strip
    // (aligned); for 32 < M <= 64 on aligned data, 64-row strips from
    // K = 2048 up (one pass over B: 48x4096x4096 14.9 us vs 22.5 on 64 x 64
    // tiles and 27.9 stream-K, 48x14336x4096 29.6 vs 31.1, 64x1024x8192
    // 19.2 vs 42.0; at K = 1024 the tiles win, 7.8 vs 10.4); unaligned
    // M <= 64 with 64 x 64 tiles for fewer than half the CUs: stream-K
    const bool strip_fits = p.M <= tlg::kStripConfig.bm &&
                            dma_ok_aligned(p, tlg::kStripConfig.bm, tlg::kStripConfig.bn, tlg::kStripConfig.bk);
    const tlg::TileConfig &t64 = tlg::kStripConfigs[tlg::SPLIT_WAVES_64x64x64 - tlg::SPLIT_WAVES_32x64x64];
    const bool strip64_fits = !strip_fits && p.M <= t64.bm && dma_ok_aligned(p, t64.bm, t64.bn, t64.bk) &&
                              ceil_div(p.N, t64.bn) <= 0x7fffffff;
    const bool few_tiles = p.M <= 64 && ceil_div(p.N, 64) * 2 < cus;
    // M > 64 with long K and fewer 64 x 64 tiles than CUs: K split over
    // 32 x 128 tiles, partials summed by a second kernel in ascending split
    // order (interleaved, us: 512x512x4096 15.6 vs 23.2 on 64 x 64 tiles,
    // 1024x512x4096 16.0 vs 22.8, 896x896x8192 36.1 vs 42.7, 1024x1024x8192
    // 40.5 vs 44.2, 256x256x16384 15.8 vs 81.6; the vendor BLAS 19.4, 20.2,
    // 40.4, 46.3, 31.2); not at K = 2048 (512x512x2048 15.5 vs 12.9) nor
    // with a full round of tiles at K = 4096 (1024x1024x4096 24.7 vs 23.9)
    const int64_t tiles64 = ceil_div(p.M, 64) * ceil_div(p.N, 64);
    const tlg::TileConfig &ts0 = tlg::kSplitConfigs[tlg::SPLIT_32x128x64];
    const bool long_k_split = p.M > 64 && p.K >= 4096 && (tiles64 < cus || (p.K >= 8192 && tiles64 <= cus)) &&
                              dma_ok_aligned(p, ts0.bm, ts0.bn, ts0.bk);
    const bool auto_split = strip_fits || (strip64_fits ? p.K >= 2048 : few_tiles) || long_k_split;
    if (variant == TLG_VARIANT_SPLITK || (variant == TLG_VARIANT_AUTO && auto_split && p.K >= 512)) {
        if (!config_ok(config, tlg::SPLIT_CONFIGS)) return TLG_ERROR_INVALID_VALUE;
        // K split among the waves of a work-group per column strip, when M
        // fits one strip and there are strips for at least half the CUs
        int cfg = config;
        if (cfg < 0) {
            const tlg::TileConfig &t0 = tlg::kStripConfig;
            const bool ok0 = p.M <= t0.bm && dma_ok_aligned(p, t0.bm, t0.bn, t0.bk) &&
                             ceil_div(p.N, t0.bn) <= 0x7fffffff;
            cfg = ok0            ? tlg::SPLIT_WAVES_32x64x64
                  : strip64_fits ? tlg::SPLIT_WAVES_64x64x64
                  : long_k_split ? tlg::SPLIT_32x128x64
                                 : tlg::SPLIT_STREAMK_32x128x64;
        }
        if (tlg::is_strip_config(cfg)) {
            const tlg::TileConfig &ts = tlg::kStripConfigs[cfg - tlg::SPLIT_WAVES_32x64x64];
            const bool strip_ok = p.M <= ts.bm && dma_ok_aligned(p, ts.bm, ts.bn, ts.bk) &&
                                  ceil_div(p.N, ts.bn) <= 0x7fffffff;
            if (!strip_ok) return TLG_ERROR_NOT_SUPPORTED;
            plan_strip_parts(p, cfg, splits, cap, cus, o);
            return TLG_SUCCESS;
        }
        if (tlg::is_strip_sk_config(cfg)) {
            // stream-K over strips: one (three-stage) or two (two-stage)
            // work-groups per CU, each taking an equal range of the strips'
            // K blocks; needs at least one range per strip
            const int j = cfg - tlg::SPLIT_STRIP_SK_32x64x64;
            const tlg::TileConfig &ts = tlg::kStripSkConfigs[j];
            const int64_t strips = ceil_div(p.N, ts.bn);
            const int64_t total = strips * ceil_div(p.K, ts.bk);
            int64_t grid = (int64_t)cus * (j == 0 ? 1 : 2);
            if (grid > total) grid = total;
            const int64_t slot_bytes = 2ll * ts.bm * ts.bn * 4;
            const bool ok = p.M <= ts.bm && dma_ok_aligned(p, ts.bm, ts.bn, ts.bk) && strips <= grid &&
                            strips * 4 <= kCounterBytes && grid * slot_bytes <= cap && total < (1ll << 40);
            if (!ok) return TLG_ERROR_NOT_SUPPORTED;
            fill_info(o, TLG_VARIANT_SPLITK, cfg, &ts, (int)ceil_div(grid, strips), 1, grid,
                      kCounterBytes + grid * slot_bytes);
            return TLG_SUCCESS;
        }
        if (cfg == tlg::SPLIT_STREAMK_32x128x64) {
            // stream-K: as many work-groups as the CUs hold, each taking an
            // equal range of the (tile, k) iterations
            const tlg::TileConfig &tc = tlg::kStreamKConfig;
            const int64_t tiles = ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn);
            // one counter per tile (at most 16384 tiles, so the iteration
            // count below stays far from overflow)
            const bool counters_fit = tiles * 4 <= kCounterBytes;
            const int64_t total = counters_fit ? tiles * ceil_div(p.K, tc.bk) : 0;
            const int64_t slot_bytes = 2ll * tc.bm * tc.bn * 4;
            int64_t grid = (int64_t)cus * tlg::kStreamKBlocksPerCU;
            if (grid > total) grid = total;
            if (grid * slot_bytes > cap) grid = cap / slot_bytes;
            const bool ok = dma_ok_aligned(p, tc.bm, tc.bn, tc.bk) && counters_fit && grid >= 1 &&
                            total * grid < (1ll << 62) && total < (1ll << 31);
            if (ok) {
                fill_info(o, TLG_VARIANT_SPLITK, cfg, &tc, (int)ceil_div(grid, tiles), 1, grid,
                          kCounterBytes + grid * slot_bytes);
                return TLG_SUCCESS;
            }
            if (variant == TLG_VARIANT_SPLITK) return TLG_ERROR_NOT_SUPPORTED;
        } else {
            const tlg::TileConfig &tc = tlg::kSplitConfigs[cfg];
            int s = 1;
            int64_t k_split = 0;
            bool ok = dma_ok_aligned(p, tc.bm, tc.bn, tc.bk) && choose_splits(p, tc, splits, cap, &s, &k_split);
            if (ok && (s > 1 || variant == TLG_VARIANT_SPLITK)) {
                const int64_t grid = ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn) * s;
                fill_info(o, TLG_VARIANT_SPLITK, cfg, &tc, s, 2, grid, kCounterBytes + (int64_t)s * p.M * p.N * 4);
                *k_split_out = k_split;
                return TLG_SUCCESS;
            }
            if (variant == TLG_VARIANT_SPLITK) return TLG_ERROR_NOT_SUPPORTED;
        }
    }

    // large aligned problems: the software-pipelined 256 x 256 tiles, when
    // there are enough tiles to give most CUs one
    if (variant == TLG_VARIANT_TILED_PIPE || variant == TLG_VARIANT_AUTO) {
        if (!config_ok(config, tlg::PIPE_CONFIGS)) return TLG_ERROR_INVALID_VALUE;
        // The 16 x 16 x 32 MFMA tiles (loads every eight MFMA slots) against
        // the eight-wave 32 x 32 x 16 tiles, interleaved on one MI355X: the
        // smaller MFMA spends less energy per FLOP, which the power-limited
        // clock turns into speed (8192^3 804 vs 834 us, 4096^3 109.2 vs
        // 112.4, 8192x4096x8192 401.6 vs 429.5, 6144^3 406.7 vs 415.5,
        // 3072^3 74.8 vs 76.9). They are the default for N a multiple of 8
        // (whole 16-byte chunks of B's rows) and K in whole 64-deep stages,
        // or any K from 256 tiles up (a masked last stage: 8192x8192x8200
        // 806.9 vs 888.8, 4096x4096x4104 114.7 vs 119.6, 6144x6144x6152
        // 420.4 vs 442.9); below 256 tiles a K tail favours the 32 x 32 x 16
        // tiles (3072x3072x3080 77.0 vs 79.7, 5000x3000x2000 65.0 vs 70.2),
        // and so does one round of 256 x 256 tiles with a nearly empty second
        // one (272 tiles: 4096x4104x4096 174.9 vs 183.9, 4096x4352x4096
        // 173.2 vs 178.0; with K in whole stages such shapes take 192 x 256
        // tiles, below: 155.3).
        //
        // Tile height by waves of work-groups: a launch takes ceil(tiles /
        // CUs) rounds of one work-group per CU, each as long as one tile, so
        // the choice among 256 x 256, 192 x 256 and 128 x 256 tiles minimises
        // rounds x the tile's relative time. Relative times measured per
        // tile against 256 x 256 (area over efficiency): 192 x 256 0.9375
        // (3072^3 66.9 vs 73.4 us in one round each; 6144^3, three rounds
        // each, 380.9 vs 402.2), 128 x 256 0.75 (2048x4096x4096 67.9 vs
        // 90.9). So 128 x 256 where it fills one round that 256 x 256 leaves
        // part idle (2560^3 41.3 vs 48.0 on the 128 x 128 direct-to-LDS
        // tiles, 2816^3 47.7 vs 60.8, 1024x8192x4096 66.9 vs 94.7), 192 x
        // 256 where its rounds stay as few (2560x4096x4096 85.7 vs 93.3),
        // 256 x 256 otherwise (4096x3072x4096: 96.6, against 143.9 on two
        // rounds of 192 x 256). The 128 x 256 tiles are the 16 x 16 x 32
        // ones where those serve (within 5 % of the 32 x 32 x 16 ones, up to
        // 13 % ahead); the 192 x 256 tiles exist in that form only. A form
        // with fewer than 128 tiles of its own is not taken (the
        // direct-to-LDS tiles then serve), nor a smaller form at 128 tiles
        // (2048^3: 32.1 us against 29.9 on the 128 x 128 direct-to-LDS tiles).
        const int64_t tiles256 = ceil_div(p.M, 256) * ceil_div(p.N, 256);
        const bool k64 = p.K % 64 == 0 && p.N % 8 == 0 && !p.trans_b;
        const bool use16 = p.N % 8 == 0 && !p.trans_b && (p.K % 64 == 0 || tiles256 >= 256) &&
                           !(tiles256 > 256 && tiles256 < 320);
        int cfg = config;
        if (cfg < 0) {
            struct Cand {
                int cfg;
                int bm;
                double rel;
            };
            const Cand cands[3] = {
                {use16 ? tlg::PIPE16_256x256x64_A3_SP8 : tlg::PIPE_256x256x64_W8_A3_EARLY, 256, 1.0},
                {k64 ? tlg::PIPE16_192x256x64_A3_SP6 : -1, 192, 0.9375},
                {k64 ? tlg::PIPE16_128x256x64_A3 : tlg::PIPE_128x256x64, 128, 0.75}};
            double best = 0.0;
            cfg = cands[0].cfg;
            for (const Cand &c : cands) {
                if (c.cfg < 0) continue;
                const int64_t t = ceil_div(p.M, c.bm) * ceil_div(p.N, 256);
                if (t <= 128 && c.bm != 256) continue;
                const double score = (double)ceil_div(t, cus > 0 ? cus : 256) * c.rel;
                if (best == 0.0 || score < best) {
                    best = score;
                    cfg = c.cfg;
                }
            }
        }
        const tlg::TileConfig &tc = tlg::kPipeConfigs[cfg];
        const int64_t tiles = ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn);
        const bool shape_ok = cfg < tlg::PIPE16_FIRST || !p.trans_b;
        // 128 tiles of 256 x 256 (half the CUs) measured faster than the
        // 128 x 128 tiles already (3072^3: 72 vs 101 us)
        if (shape_ok && dma_ok(p, tc.bm, tc.bn, tc.bk) && (variant == TLG_VARIANT_TILED_PIPE || tiles >= 128)) {
            fill_info(o, TLG_VARIANT_TILED_PIPE, cfg, &tc, 1, 1, tiles, 0);
            return TLG_SUCCESS;
        }
        // Fewer: the 32 x 32 x 16 MFMA 128 x 256 tiles from 96 of them up
        // (interleaved, us: 2048^3 24.7 vs 28.4 on 128 x 128 direct-to-LDS
        // tiles and 27.4 on the 16 x 16 x 32 form, 2048x2048x8192 78.0 vs
        // 97.2 and 87.1, 1536x2048x4096 41.4 vs 46.4 on 64 x 64 tiles,
        // 1792x2048x2048 24.2 vs 27.9; the vendor BLAS 25.5, 77.7, 40.2,
        // 24.5); at 60 tiles the 64 x 64 ones stay ahead (1280x1536x4096
        // 32.0 vs 40.1)
        const tlg::TileConfig &th = tlg::kPipeConfigs[tlg::PIPE_128x256x64];
        const int64_t t_half = ceil_div(p.M, th.bm) * ceil_div(p.N, th.bn);
        if (variant == TLG_VARIANT_AUTO && tiles < 128 && t_half >= 96 && dma_ok(p, th.bm, th.bn, th.bk)) {
            fill_info(o, TLG_VARIANT_TILED_PIPE, tlg::PIPE_128x256x64, &th, 1, 1, t_half, 0);
            return TLG_SUCCESS;
        }
        if (variant == TLG_VARIANT_TILED_PIPE) return TLG_ERROR_NOT_SUPPORTED;
    }

    if (variant == TLG_VARIANT_TILED_DMA || variant == TLG_VARIANT_AUTO) {
        if (!config_ok(config, tlg::DMA_CONFIGS)) return TLG_ERROR_INVALID_VALUE;
        int cfg;
        const int64_t t256 = ceil_div(p.M, 256) * ceil_div(p.N, 256);
        const int64_t t128 = ceil_div(p.M, 128) * ceil_div(p.N, 128);
        if (config >= 0)
            cfg = config;
        else if (t256 >= 224)
            cfg = tlg::DMA_256x256x32;
        else if (t128 >= 192)
            cfg = tlg::DMA_128x128x32;
        else
            cfg = tlg::DMA_64x64x64;
        const tlg::TileConfig &tc = tlg::kDmaConfigs[cfg];
        if (dma_ok(p, tc.bm, tc.bn, tc.bk)) {
            fill_info(o, TLG_VARIANT_TILED_DMA, cfg, &tc, 1, 1, ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn), 0);
            return TLG_SUCCESS;
        }
        if (variant == TLG_VARIANT_TILED_DMA) return TLG_ERROR_NOT_SUPPORTED;
    }

    // TLG_VARIANT_TILED_GENERAL, or AUTO on data the DMA kernels cannot take
    if (!config_ok(config, tlg::GEN_CONFIGS)) return TLG_ERROR_INVALID_VALUE;
    const int cfg = config >= 0 ? config
                                : (ceil_div(p.M, 128) * ceil_div(p.N, 128) >= 192 ? tlg::GEN_128x128x32
                                                                                   : tlg::GEN_64x64x32);
    const tlg::TileConfig &tc = tlg::kGenConfigs[cfg];
    fill_info(o, TLG_VARIANT_TILED_GENERAL, cfg, &tc, 1, 1, ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn), 0);
    return TLG_SUCCESS;
}

tlg::Problem make_problem(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                          const void *C, int64_t ldc) {
    tlg::Problem p;
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = A;
    p.lda = lda;
    p.B = B;
    p.ldb = ldb;
    p.C = const_cast<void *>(C);
    p.ldc = ldc;
    return p;
}

}  // namespace

namespace tlg {

// Plans one call for a device with `cus` compute units and a workspace of
// `workspace_bytes` at `workspace` (its first kCounterBytes the split
// kernels' counters), then enqueues it. With clear_counters the counter area
// is cleared on the stream before a split kernel that uses it.
tlg_status run_with_workspace(float *workspace, int64_t workspace_bytes, int cus, bool clear_counters,
                              int32_t variant, int32_t config, int32_t splits, const Problem &p,
                              hipStream_t stream) {
    tlg_status st = tlg_check_args(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc);
    if (st != TLG_SUCCESS) return st;
    tlg_plan_info info;
    int64_t k_split = 0;
    st = plan_impl(p, variant, config, splits, workspace_bytes, cus, &info, &k_split);
    if (st != TLG_SUCCESS) return st;
    if (info.workspace_bytes > workspace_bytes) return TLG_ERROR_NOT_SUPPORTED;
    float *const ws = workspace;
    hipError_t e = hipSuccess;
    if (clear_counters && info.variant == TLG_VARIANT_SPLITK && info.workspace_bytes > 0) {
        e = launch_clear_words((int *)ws, kCounterBytes / 4, stream);
        if (e != hipSuccess) return TLG_ERROR_HIP;
    }
    switch (info.variant) {
        case TLG_VARIANT_NOOP: return TLG_SUCCESS;
        case TLG_VARIANT_FILL_ZERO: e = tlg::launch_fill_zero(p, stream); break;
        case TLG_VARIANT_NAIVE: e = tlg::launch_naive(p, stream); break;
        case TLG_VARIANT_TILED_DMA: e = tlg::launch_tiled_dma(info.config, p, stream); break;
        case TLG_VARIANT_TILED_GENERAL: e = tlg::launch_tiled_general(info.config, p, stream); break;
        case TLG_VARIANT_TILED_PIPE: e = tlg::launch_tiled_pipe(info.config, p, stream); break;
        case TLG_VARIANT_PINGPONG: e = tlg::launch_pingpong(info.config, p, stream); break;
        case TLG_VARIANT_SPLITK: {
            float *partials = ws + kCounterBytes / sizeof(float);
            if (tlg::is_strip_sk_config(info.config))
                e = tlg::launch_skinny_strip_sk(info.config - tlg::SPLIT_STRIP_SK_32x64x64, p, (int)info.grid,
                                                partials, (int *)ws, stream);
            else if (tlg::is_strip_config(info.config))
                e = tlg::launch_skinny_strip(info.config - tlg::SPLIT_WAVES_32x64x64, p, info.splits, partials,
                                             (int *)ws, stream);
            else if (info.config == tlg::SPLIT_STREAMK_32x128x64)
                e = tlg::launch_streamk(p, (int)info.grid, partials, (int *)ws, stream);
            else
                e = tlg::launch_splitk(info.config, info.splits, k_split, p, partials, stream);
            break;
        }
        default: return TLG_ERROR_NOT_SUPPORTED;
    }
    return e == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
}

tlg::Problem make_problem_c(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                            void *C, int64_t ldc) {
    return make_problem(M, N, K, A, lda, B, ldb, C, ldc);
}

}  // namespace tlg

namespace {

tlg_status run(tlg_handle h, int32_t variant, int32_t config, int32_t splits, const tlg::Problem &p,
               hipStream_t stream) {
    if (!h) return TLG_ERROR_INVALID_VALUE;
    tlg_status st = tlg_check_args(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc);
    if (st != TLG_SUCCESS) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TLG_ERROR_HIP;
    if (dev != h->device) return TLG_ERROR_INVALID_VALUE;  // the handle's device must be current
    return tlg::run_with_workspace(h->workspace, h->workspace_bytes, h->cus, false, variant, config, splits, p,
                                   stream);
}

// ---- transposed B and grouped calls ----

tlg_status check_args_bt(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *Bt, int64_t ldbt,
                         const void *C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return TLG_ERROR_INVALID_VALUE;
    if (lda < (K > 1 ? K : 1) || ldbt < (K > 1 ? K : 1) || ldc < (N > 1 ? N : 1)) return TLG_ERROR_INVALID_VALUE;
    if (M == 0 || N == 0) return TLG_SUCCESS;
    if (!C || !aligned(C, 2)) return TLG_ERROR_INVALID_VALUE;
    if (K > 0) {
        if (!A || !Bt || !aligned(A, 2) || !aligned(Bt, 2)) return TLG_ERROR_INVALID_VALUE;
    }
    return TLG_SUCCESS;
}

// In-tile byte offsets with a transposed B (its tile is bn rows of ldb).
bool offsets_ok_bt(const tlg::Problem &p, int bm, int bn) {
    if ((int64_t)bm * p.lda * 2 > kMaxOffset) return false;
    if ((int64_t)bn * p.ldb * 2 > kMaxOffset) return false;
    if ((int64_t)bm * p.ldc * 2 + (int64_t)bn * 2 > kMaxOffset) return false;
    return true;
}

// Direct-to-LDS configuration by tile count (the transposed-B and grouped
// calls use the square configurations 0..2 only).
int dma_config_by_tiles(int64_t t256, int64_t t128) {
    if (t256 >= 224) return tlg::DMA_256x256x32;
    if (t128 >= 192) return tlg::DMA_128x128x32;
    return tlg::DMA_64x64x64;
}
constexpr int kSquareDmaConfigs = 3;
// grouped calls: configurations 0..2 are those direct-to-LDS ones, 3 the
// eight-wave pipelined 256 x 256 kernel
constexpr int kGroupedPipe = kSquareDmaConfigs;
// 4: the 16 x 16 x 32 pipelined 256 x 256 kernel (B not transposed)
constexpr int kGroupedPipe16 = kGroupedPipe + 1;

tlg_status plan_bt_select(const tlg::Problem &p, int32_t variant, int32_t config, tlg_plan_info *o);
tlg_status plan_bt(const tlg::Problem &p, int32_t variant, int32_t config, tlg_plan_info *o) {
    return grid_fits(plan_bt_select(p, variant, config, o), o);
}
tlg_status plan_bt_select(const tlg::Problem &p, int32_t variant, int32_t config, tlg_plan_info *o) {
    if (variant != TLG_VARIANT_AUTO && variant != TLG_VARIANT_TILED_DMA && variant != TLG_VARIANT_TILED_PIPE &&
        variant != TLG_VARIANT_PINGPONG && variant != TLG_VARIANT_SPLITK)
        return TLG_ERROR_INVALID_VALUE;
    if (variant == TLG_VARIANT_SPLITK && config != -1 && !tlg::is_strip_config(config)) return TLG_ERROR_INVALID_VALUE;
    if (variant == TLG_VARIANT_AUTO && config != -1) return TLG_ERROR_INVALID_VALUE;
    if (variant == TLG_VARIANT_TILED_DMA && (config < -1 || config >= kSquareDmaConfigs))
        return TLG_ERROR_INVALID_VALUE;
    if (variant == TLG_VARIANT_TILED_PIPE && config != -1 && config != tlg::PIPE_256x256x64_A3 &&
        config != tlg::PIPE_256x256x64_W8_A3 && config != tlg::PIPE_256x256x64_W8_A3_EARLY &&
        config != tlg::PIPE16_256x256x64_A3_SP8 && config != tlg::PIPE16_128x256x64_A3 &&
        config != tlg::PIPE16_192x256x64_A3_SP6)
        return TLG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0) {
        fill_info(o, TLG_VARIANT_NOOP, 0, nullptr, 1, 0, 0, 0);
        return TLG_SUCCESS;
    }
    if (p.M > kMaxDim || p.N > kMaxDim || p.K > kMaxDim) return TLG_ERROR_NOT_SUPPORTED;
    if (p.K == 0) {
        fill_zero_info(o, p.M, p.N);
        return TLG_SUCCESS;
    }
    const int64_t t256 = ceil_div(p.M, 256) * ceil_div(p.N, 256);
    // Skinny M: the strip kernel, B's blocks loaded and read like A's rows,
    // under the plain call's rule (one 32-row strip from K = 512, the 64-row
    // strip for 32 < M <= 64 from K = 2048; aligned data), parts as there
    // (16x14336x4096: 21.6 vs 30.7 us on the 64 x 64 direct-to-LDS tiles;
    // 48x4096x14336: 27.8)
    {
        auto strip_ok = [&](int cfg) {
            const tlg::TileConfig &ts = tlg::kStripConfigs[cfg - tlg::SPLIT_WAVES_32x64x64];
            return p.M <= ts.bm && aligned(p.A, 16) && aligned(p.B, 16) && aligned(p.C, 16) && p.lda % 8 == 0 &&
                   p.ldb % 8 == 0 && p.ldc % 8 == 0 && p.K % 8 == 0 && p.N % 8 == 0 && offsets_ok_bt(p, ts.bm, ts.bn) &&
                   ceil_div(p.N, ts.bn) <= 0x7fffffff;
        };
        int cfg = -1;
        if (variant == TLG_VARIANT_SPLITK)
            cfg = config >= 0 ? config : tlg::SPLIT_WAVES_32x64x64;
        else if (variant == TLG_VARIANT_AUTO && p.K >= 512 && strip_ok(tlg::SPLIT_WAVES_32x64x64))
            cfg = tlg::SPLIT_WAVES_32x64x64;
        else if (variant == TLG_VARIANT_AUTO && p.K >= 2048 && strip_ok(tlg::SPLIT_WAVES_64x64x64))
            cfg = tlg::SPLIT_WAVES_64x64x64;
        if (cfg >= 0) {
            if (!strip_ok(cfg)) return TLG_ERROR_NOT_SUPPORTED;
            plan_strip_parts(p, cfg, 0, kWorkspaceBytes - kCounterBytes, kPlanCUs, o);
            return TLG_SUCCESS;
        }
    }
    if (variant == TLG_VARIANT_PINGPONG) {
        if (config < -1 || config >= tlg::PINGPONG_CONFIGS) return TLG_ERROR_INVALID_VALUE;
        const int cfg = config >= 0 ? config : tlg::PINGPONG_256x256x32;
        const tlg::TileConfig &tc = tlg::kPingPongConfigs[cfg];
        if (!offsets_ok_bt(p, tc.bm, tc.bn)) return TLG_ERROR_NOT_SUPPORTED;
        fill_info(o, TLG_VARIANT_PINGPONG, cfg, &tc, 1, 1, t256, 0);
        return TLG_SUCCESS;
    }
    // the same boundary as the plain call: 256 x 256 pipelined tiles from 128
    // tiles up (half the CUs; 3072^3 measured 72 vs 101 us on 128 x 128
    // tiles), on the 16 x 16 x 32 form under the plain call's conditions
    // (K whole 64-deep stages, or at least 256 tiles, not 257..319 of them;
    // B's rows need no condition on N here: 8192^3 823.0 vs 871.5 us, 4096^3
    // 139.6-145.6 vs 143.1-147.9 on the 32 x 32 x 16 early form)
    if (variant == TLG_VARIANT_TILED_PIPE || (variant == TLG_VARIANT_AUTO && t256 >= 128)) {
        const bool use16 = (p.K % 64 == 0 || t256 >= 256) && !(t256 > 256 && t256 < 320);
        int cfg = config >= 0 ? config : use16 ? tlg::PIPE16_256x256x64_A3_SP8 : tlg::PIPE_256x256x64_W8_A3_EARLY;
        if (config < 0 && p.K % 64 == 0) {
            // tile height by rounds x relative tile time, as for the plain
            // call (the 192 x 256 and 128 x 256 tiles in their 16 x 16 x 32
            // form, K whole stages; against the 256 x 256 ones, us: 3072^3
            // 64.7 vs 70.1, 6144^3 411.4 vs 419.5, 2560x4096x4096 82.2 vs
            // 89.5, 2048x4096x4096 62.8 vs 88.5)
            const int cus = kPlanCUs;
            const int cand_cfg[3] = {cfg, tlg::PIPE16_192x256x64_A3_SP6, tlg::PIPE16_128x256x64_A3};
            const int cand_bm[3] = {256, 192, 128};
            const double cand_rel[3] = {1.0, 0.9375, 0.75};
            double best = 0.0;
            for (int c = 0; c < 3; ++c) {
                const int64_t t = ceil_div(p.M, cand_bm[c]) * ceil_div(p.N, 256);
                if (t <= 128 && cand_bm[c] != 256) continue;
                const double score = (double)ceil_div(t, cus > 0 ? cus : 256) * cand_rel[c];
                if (best == 0.0 || score < best) {
                    best = score;
                    cfg = cand_cfg[c];
                }
            }
        }
        const tlg::TileConfig &tc = tlg::kPipeConfigs[cfg];
        if (offsets_ok_bt(p, tc.bm, tc.bn)) {
            fill_info(o, TLG_VARIANT_TILED_PIPE, cfg, &tc, 1, 1, ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn), 0);
            return TLG_SUCCESS;
        }
        if (variant == TLG_VARIANT_TILED_PIPE) return TLG_ERROR_NOT_SUPPORTED;
    }
    // below that, 128 x 256 pipelined tiles (16 x 16 x 32 MFMA) once there
    // are at least 192 of them: 3001 x 2049 x 1537 measured 34.4 vs 46.4 us
    // and 2560^3 41.0 vs 51.3 us on 128 x 128 direct-to-LDS tiles, while at
    // 128 of them (2048^3) 31.3 vs 28.6 us the smaller tiles still win
    if (variant == TLG_VARIANT_AUTO) {
        const tlg::TileConfig &th = tlg::kPipeConfigs[tlg::PIPE16_128x256x64_A3];
        const int64_t t_half = ceil_div(p.M, th.bm) * ceil_div(p.N, th.bn);
        if (t_half >= 192 && offsets_ok_bt(p, th.bm, th.bn)) {
            fill_info(o, TLG_VARIANT_TILED_PIPE, tlg::PIPE16_128x256x64_A3, &th, 1, 1, t_half, 0);
            return TLG_SUCCESS;
        }
    }
    const int cfg = config >= 0 && variant == TLG_VARIANT_TILED_DMA
                        ? config
                        : dma_config_by_tiles(t256, ceil_div(p.M, 128) * ceil_div(p.N, 128));
    const tlg::TileConfig &tc = tlg::kDmaConfigs[cfg];
    if (!offsets_ok_bt(p, tc.bm, tc.bn)) return TLG_ERROR_NOT_SUPPORTED;
    fill_info(o, TLG_VARIANT_TILED_DMA, cfg, &tc, 1, 1, ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn), 0);
    return TLG_SUCCESS;
}

tlg_status device_ok(tlg_handle h) {
    if (!h) return TLG_ERROR_INVALID_VALUE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TLG_ERROR_HIP;
    return dev == h->device ? TLG_SUCCESS : TLG_ERROR_INVALID_VALUE;
}

tlg_status run_bt(tlg_handle h, int32_t variant, int32_t config, tlg::Problem p, hipStream_t stream) {
    tlg_status st = device_ok(h);
    if (st != TLG_SUCCESS) return st;
    st = check_args_bt(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc);
    if (st != TLG_SUCCESS) return st;
    p.trans_b = true;
    tlg_plan_info info;
    st = plan_bt(p, variant, config, &info);
    if (st != TLG_SUCCESS) return st;
    hipError_t e = hipSuccess;
    switch (info.variant) {
        case TLG_VARIANT_NOOP: return TLG_SUCCESS;
        case TLG_VARIANT_FILL_ZERO: e = tlg::launch_fill_zero(p, stream); break;
        case TLG_VARIANT_TILED_DMA: e = tlg::launch_tiled_dma(info.config, p, stream); break;
        case TLG_VARIANT_TILED_PIPE: e = tlg::launch_tiled_pipe(info.config, p, stream); break;
        case TLG_VARIANT_PINGPONG: e = tlg::launch_pingpong(info.config, p, stream); break;
        case TLG_VARIANT_SPLITK: {
            if (!tlg::is_strip_config(info.config) || info.workspace_bytes > h->workspace_bytes)
                return TLG_ERROR_NOT_SUPPORTED;
            float *const ws = h->workspace;
            e = tlg::launch_skinny_strip(info.config - tlg::SPLIT_WAVES_32x64x64, p, info.splits,
                                         ws + kCounterBytes / sizeof(float), (int *)ws, stream);
            break;
        }
        default: return TLG_ERROR_NOT_SUPPORTED;
    }
    return e == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
}

tlg_status run_grouped(tlg_handle h, int32_t config, int32_t count, const tlg_gemm_desc *descs, int32_t trans_b,
                       hipStream_t stream) {
    tlg_status st = device_ok(h);
    if (st != TLG_SUCCESS) return st;
    if (count < 0 || count > TLG_GROUP_MAX || (trans_b != 0 && trans_b != 1)) return TLG_ERROR_INVALID_VALUE;
    if (config < -1 || config > kGroupedPipe16) return TLG_ERROR_INVALID_VALUE;
    if (count == 0) return TLG_SUCCESS;
    if (!descs) return TLG_ERROR_INVALID_VALUE;
    tlg::Problem ps[TLG_GROUP_MAX];
    int n = 0;
    int64_t t256 = 0, t128 = 0;
    for (int i = 0; i < count; ++i) {
        const tlg_gemm_desc &d = descs[i];
        st = trans_b ? check_args_bt(d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc)
                     : tlg_check_args(d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc);
        if (st != TLG_SUCCESS) return st;
        if (d.M == 0 || d.N == 0) continue;
        tlg::Problem p = make_problem(d.M, d.N, d.K, d.A, d.lda, d.B, d.ldb, d.C, d.ldc);
        p.trans_b = trans_b != 0;
        ps[n++] = p;
        t256 += ceil_div(d.M, 256) * ceil_div(d.N, 256);
        t128 += ceil_div(d.M, 128) * ceil_div(d.N, 128);
    }
    if (n == 0) return TLG_SUCCESS;
    // the pipelined 256 x 256 kernels from the same total tile count as a
    // single call (128 tiles of 256 x 256), when every problem can take them:
    // the 16 x 16 x 32 form for K in whole 64-deep stages and, with B not
    // transposed, N a multiple of 8 (8192^3 as 8 row blocks: 855.0-858.7 us
    // against 882.4-887.1 on the 32 x 32 x 16 form), else the 32 x 32 x 16 form
    const bool auto_pipe = config == -1 && t256 >= 128;
    if (config == kGroupedPipe16 || auto_pipe) {
        const tlg::TileConfig &tp = tlg::kPipeConfigs[tlg::PIPE16_256x256x64_A3_SP8];
        bool ok = t256 <= 0x7fffffff;
        for (int i = 0; i < n && ok; ++i)
            ok = (ps[i].K % tp.bk == 0 || config == kGroupedPipe16) &&
                 (trans_b ? offsets_ok_bt(ps[i], tp.bm, tp.bn) : ps[i].N % 8 == 0 && dma_ok(ps[i], tp.bm, tp.bn, tp.bk));
        if (ok) return tlg::launch_tiled_pipe16_grouped(ps, n, stream) == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
        if (config == kGroupedPipe16) return TLG_ERROR_NOT_SUPPORTED;
    }
    if (config == kGroupedPipe || auto_pipe) {
        const tlg::TileConfig &tp = tlg::kPipeConfigs[tlg::PIPE_256x256x64_W8_A3_EARLY];
        bool ok = t256 <= 0x7fffffff;
        for (int i = 0; i < n && ok; ++i)
            ok = trans_b ? offsets_ok_bt(ps[i], tp.bm, tp.bn) : dma_ok(ps[i], tp.bm, tp.bn, tp.bk);
        if (ok) return tlg::launch_tiled_pipe_grouped(ps, n, stream) == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
        if (config == kGroupedPipe) return TLG_ERROR_NOT_SUPPORTED;
    }
    const int cfg = config >= 0 ? config : dma_config_by_tiles(t256, t128);
    const tlg::TileConfig &tc = tlg::kDmaConfigs[cfg];
    int64_t tiles = 0;
    for (int i = 0; i < n; ++i) {
        const bool ok = trans_b ? offsets_ok_bt(ps[i], tc.bm, tc.bn) : dma_ok(ps[i], tc.bm, tc.bn, tc.bk);
        if (!ok) return TLG_ERROR_NOT_SUPPORTED;
        tiles += ceil_div(ps[i].M, tc.bm) * ceil_div(ps[i].N, tc.bn);
    }
    if (tiles > 0x7fffffff) return TLG_ERROR_NOT_SUPPORTED;
    return tlg::launch_tiled_dma_grouped(cfg, ps, n, stream) == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
}

// ---- block-scaled (MX) calls ----

int mx_codes_per_byte(int32_t format) { return format == TLG_MX_E2M1 ? 2 : 1; }

tlg_status check_args_mx(int32_t format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SA,
                         int64_t ldsa, const void *B, int64_t ldb, const void *SB, int64_t ldsb, const void *C,
                         int64_t ldc) {
    if (format != TLG_MX_E4M3 && format != TLG_MX_E5M2 && format != TLG_MX_E2M1) return TLG_ERROR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0 || K % TLG_MX_BLOCK) return TLG_ERROR_INVALID_VALUE;
    const int64_t kb = K / TLG_MX_BLOCK;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1) || ldc < (N > 1 ? N : 1)) return TLG_ERROR_INVALID_VALUE;
    if (ldsa < (kb > 1 ? kb : 1) || ldsb < (kb > 1 ? kb : 1)) return TLG_ERROR_INVALID_VALUE;
    if (format == TLG_MX_E2M1 && (lda % 2 || ldb % 2)) return TLG_ERROR_INVALID_VALUE;
    if (M == 0 || N == 0) return TLG_SUCCESS;
    if (!C || !aligned(C, 2)) return TLG_ERROR_INVALID_VALUE;
    if (K > 0 && (!A || !B || !SA || !SB)) return TLG_ERROR_INVALID_VALUE;
    return TLG_SUCCESS;
}

tlg_status plan_mx_select(const tlg::MxProblem &p, int32_t config, tlg_plan_info *o);
tlg_status plan_mx(const tlg::MxProblem &p, int32_t config, tlg_plan_info *o) {
    return grid_fits(plan_mx_select(p, config, o), o);
}
tlg_status plan_mx_select(const tlg::MxProblem &p, int32_t config, tlg_plan_info *o) {
    if (config < -1 || config >= tlg::MX_CONFIGS) return TLG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0) {
        fill_info(o, TLG_VARIANT_NOOP, 0, nullptr, 1, 0, 0, 0);
        return TLG_SUCCESS;
    }
    if (p.M > kMaxDim || p.N > kMaxDim || p.K > kMaxDim) return TLG_ERROR_NOT_SUPPORTED;
    if (p.K == 0) {
        fill_zero_info(o, p.M, p.N);
        return TLG_SUCCESS;
    }
    // stages of 128 codes (four scale blocks): K a multiple of 128; 16-byte
    // chunks wholly inside a row; scale dwords aligned
    const int epb = mx_codes_per_byte(p.format);
    if (p.K % 128) return TLG_ERROR_NOT_SUPPORTED;
    if (!aligned(p.A, 16) || !aligned(p.B, 16) || (p.lda / epb) % 16 || (p.ldb / epb) % 16)
        return TLG_ERROR_NOT_SUPPORTED;
    if (!aligned(p.SA, 4) || !aligned(p.SB, 4) || p.ldsa % 4 || p.ldsb % 4) return TLG_ERROR_NOT_SUPPORTED;
    // 256 x 256 tiles when there are more of them than half the CUs (measured:
    // 3072^3, 144 tiles: 53 vs 60 us MXFP8; 1024x8192x8192, 128 tiles: 127 vs
    // 114 us on 128 x 128 tiles)
    const int64_t t256 = ceil_div(p.M, 256) * ceil_div(p.N, 256);
    const int cfg = config >= 0 ? config : (t256 > 128 ? tlg::MX_256x256_W8 : tlg::MX_128x128_W4);
    // the four-wave pipelined form holds 8-bit fragments only (4-bit ones
    // would not stay in registers)
    if (cfg == tlg::MX_PIPE_256x256_W4 && p.format == TLG_MX_E2M1) return TLG_ERROR_NOT_SUPPORTED;
    const tlg::TileConfig &tc = tlg::kMxConfigs[cfg];
    if ((int64_t)tc.bm * (p.lda / epb) + 128 > kMaxOffset || (int64_t)tc.bn * (p.ldb / epb) + 128 > kMaxOffset ||
        (int64_t)tc.bm * p.ldsa > kMaxOffset || (int64_t)tc.bn * p.ldsb > kMaxOffset ||
        (int64_t)tc.bm * p.ldc * 2 + (int64_t)tc.bn * 2 > kMaxOffset)
        return TLG_ERROR_NOT_SUPPORTED;
    const int64_t tiles = ceil_div(p.M, tc.bm) * ceil_div(p.N, tc.bn);
    if (tiles > 0x7fffffff) return TLG_ERROR_NOT_SUPPORTED;
    fill_info(o, TLG_VARIANT_TILED_DMA, cfg, &tc, 1, 1, tiles, 0);
    o->block_k = tc.bk * epb;  // codes of K per stage
    return TLG_SUCCESS;
}

tlg::MxProblem make_mx_problem(int32_t format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                               const void *SA, int64_t ldsa, const void *B, int64_t ldb, const void *SB,
                               int64_t ldsb, const void *C, int64_t ldc) {
    tlg::MxProblem p;
    p.format = format;
    p.M = M;
    p.N = N;
    p.K = K;
    p.A = A;
    p.lda = lda;
    p.SA = SA;
    p.ldsa = ldsa;
    p.B = B;
    p.ldb = ldb;
    p.SB = SB;
    p.ldsb = ldsb;
    p.C = const_cast<void *>(C);
    p.ldc = ldc;
    return p;
}

tlg_status run_mx(tlg_handle h, int32_t config, const tlg::MxProblem &p, hipStream_t stream) {
    tlg_status st = device_ok(h);
    if (st != TLG_SUCCESS) return st;
    st = check_args_mx(p.format, p.M, p.N, p.K, p.A, p.lda, p.SA, p.ldsa, p.B, p.ldb, p.SB, p.ldsb, p.C, p.ldc);
    if (st != TLG_SUCCESS) return st;
    tlg_plan_info info;
    st = plan_mx(p, config, &info);
    if (st != TLG_SUCCESS) return st;
    hipError_t e = hipSuccess;
    switch (info.variant) {
        case TLG_VARIANT_NOOP: return TLG_SUCCESS;
        case TLG_VARIANT_FILL_ZERO: {
            tlg::Problem z = make_problem(p.M, p.N, 0, nullptr, 1, nullptr, p.N, p.C, p.ldc);
            e = tlg::launch_fill_zero(z, stream);
            break;
        }
        case TLG_VARIANT_TILED_DMA: e = tlg::launch_mx(info.config, p, stream); break;
        default: return TLG_ERROR_NOT_SUPPORTED;
    }
    return e == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
}

tlg_status run_mx_grouped(tlg_handle h, int32_t config, int32_t format, int32_t count, const tlg_mx_desc *descs,
                          hipStream_t stream) {
    tlg_status st = device_ok(h);
    if (st != TLG_SUCCESS) return st;
    if (count < 0 || count > TLG_GROUP_MAX) return TLG_ERROR_INVALID_VALUE;
    if (config != -1 && config != tlg::MX_256x256_W8 && config != tlg::MX_128x128_W4) return TLG_ERROR_INVALID_VALUE;
    if (format != TLG_MX_E4M3 && format != TLG_MX_E5M2 && format != TLG_MX_E2M1) return TLG_ERROR_INVALID_VALUE;
    if (count == 0) return TLG_SUCCESS;
    if (!descs) return TLG_ERROR_INVALID_VALUE;
    tlg::MxProblem ps[TLG_GROUP_MAX];
    int n = 0;
    int64_t t256 = 0;
    for (int i = 0; i < count; ++i) {
        const tlg_mx_desc &d = descs[i];
        st = check_args_mx(format, d.M, d.N, d.K, d.A, d.lda, d.SA, d.ldsa, d.B, d.ldb, d.SB, d.ldsb, d.C, d.ldc);
        if (st != TLG_SUCCESS) return st;
        if (d.M == 0 || d.N == 0) continue;
        if (d.K == 0) return TLG_ERROR_NOT_SUPPORTED;
        ps[n++] = make_mx_problem(format, d.M, d.N, d.K, d.A, d.lda, d.SA, d.ldsa, d.B, d.ldb, d.SB, d.ldsb, d.C,
                                  d.ldc);
        t256 += ceil_div(d.M, 256) * ceil_div(d.N, 256);
    }
    if (n == 0) return TLG_SUCCESS;
    const int cfg = config >= 0 ? config : (t256 > 128 ? tlg::MX_256x256_W8 : tlg::MX_128x128_W4);
    int64_t tiles = 0;
    for (int i = 0; i < n; ++i) {
        tlg_plan_info info;
        st = plan_mx(ps[i], cfg, &info);  // the single-problem checks (alignment, K % 128, offsets)
        if (st != TLG_SUCCESS) return st;
        tiles += info.grid;
    }
    if (tiles > 0x7fffffff) return TLG_ERROR_NOT_SUPPORTED;
    return tlg::launch_mx_grouped(cfg, ps, n, stream) == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
}

}  // namespace

extern "C" {

tlg_status tlg_check_args(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                          const void *C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return TLG_ERROR_INVALID_VALUE;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return TLG_ERROR_INVALID_VALUE;
    if (M == 0 || N == 0) return TLG_SUCCESS;  // nothing is read or written
    if (!C || !aligned(C, 2)) return TLG_ERROR_INVALID_VALUE;
    if (K > 0) {
        if (!A || !B || !aligned(A, 2) || !aligned(B, 2)) return TLG_ERROR_INVALID_VALUE;
    }
    return TLG_SUCCESS;
}

tlg_status tlg_plan(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                    const void *C, int64_t ldc, int32_t variant, int32_t config, int32_t splits,
                    int64_t workspace_cap_bytes,
                    tlg_plan_info *out) {
    if (!out) return TLG_ERROR_INVALID_VALUE;
    tlg_status st = tlg_check_args(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != TLG_SUCCESS) return st;
    tlg::Problem p = make_problem(M, N, K, A, lda, B, ldb, C, ldc);
    int64_t k_split = 0;
    return plan_impl(p, variant, config, splits, workspace_cap_bytes, kPlanCUs, out, &k_split);
}

const char *tlg_plan_config_name(int32_t variant, int32_t config) {
    switch (variant) {
        case TLG_VARIANT_TILED_DMA:
            return (config >= 0 && config < tlg::DMA_CONFIGS) ? tlg::kDmaConfigs[config].name : "";
        case TLG_VARIANT_TILED_GENERAL:
            return (config >= 0 && config < tlg::GEN_CONFIGS) ? tlg::kGenConfigs[config].name : "";
        case TLG_VARIANT_SPLITK:
            if (config == tlg::SPLIT_STREAMK_32x128x64) return tlg::kStreamKConfig.name;
            if (tlg::is_strip_config(config)) return tlg::kStripConfigs[config - tlg::SPLIT_WAVES_32x64x64].name;
            if (tlg::is_strip_sk_config(config))
                return tlg::kStripSkConfigs[config - tlg::SPLIT_STRIP_SK_32x64x64].name;
            return (config >= 0 && config < tlg::SPLIT_TWO_KERNEL_CONFIGS) ? tlg::kSplitConfigs[config].name : "";
        case TLG_VARIANT_TILED_PIPE:
            return (config >= 0 && config < tlg::PIPE_CONFIGS) ? tlg::kPipeConfigs[config].name : "";
        case TLG_VARIANT_PINGPONG:
            return (config >= 0 && config < tlg::PINGPONG_CONFIGS) ? tlg::kPingPongConfigs[config].name : "";
        case TLG_VARIANT_NAIVE: return "naive_16x16";
        case TLG_VARIANT_FILL_ZERO: return "fill_zero";
        case TLG_VARIANT_NOOP: return "noop";
        default: return "";
    }
}

int64_t tlg_workspace_bytes(void) { return kWorkspaceBytes; }

int32_t tlg_arch_supported(const char *name) {
    if (!name) return 0;
    // "gfx950" exactly, or followed by ':' feature flags
    return strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':') ? 1 : 0;
}

tlg_status tlg_create(tlg_handle *out) {
    if (!out) return TLG_ERROR_INVALID_VALUE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TLG_ERROR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TLG_ERROR_HIP;
    if (!tlg_arch_supported(prop.gcnArchName)) return TLG_ERROR_NOT_SUPPORTED;
    tlg_context *ctx = new (std::nothrow) tlg_context;
    if (!ctx) return TLG_ERROR_OUT_OF_MEMORY;
    ctx->device = dev;
    ctx->cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kPlanCUs;
    ctx->workspace_bytes = kWorkspaceBytes;
    ctx->workspace = nullptr;
    if (hipMalloc((void **)&ctx->workspace, (size_t)kWorkspaceBytes) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky allocation error
        delete ctx;
        return TLG_ERROR_OUT_OF_MEMORY;
    }
    // the stream-K counters start at zero (each call leaves them zero); the
    // clear runs on the null stream, so waiting on that stream is enough
    if (hipMemsetAsync(ctx->workspace, 0, (size_t)kCounterBytes, nullptr) != hipSuccess ||
        hipStreamSynchronize(nullptr) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(ctx->workspace);
        delete ctx;
        return TLG_ERROR_HIP;
    }
    *out = ctx;
    return TLG_SUCCESS;
}

tlg_status tlg_destroy(tlg_handle h) {
    if (!h) return TLG_SUCCESS;
    hipError_t e = hipSuccess;
    if (h->workspace) e = hipFree(h->workspace);
    delete h;
    return e == hipSuccess ? TLG_SUCCESS : TLG_ERROR_HIP;
}

tlg_status tlg_gemm_relu(tlg_handle h, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                         int64_t ldb, void *C, int64_t ldc, hipStream_t stream) {
    return run(h, TLG_VARIANT_AUTO, -1, 0, make_problem(M, N, K, A, lda, B, ldb, C, ldc), stream);
}

tlg_status tlg_gemm_relu_variant(tlg_handle h, int32_t variant, int32_t config, int32_t splits, int64_t M, int64_t N,
                                 int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                                 int64_t ldc, hipStream_t stream) {
    return run(h, variant, config, splits, make_problem(M, N, K, A, lda, B, ldb, C, ldc), stream);
}

const char *tlg_status_string(tlg_status s) {
    // a C caller may pass any int: read the argument's bytes as an int
    // instead of loading an enum value that may be out of its range
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case TLG_SUCCESS: return "TLG_SUCCESS";
        case TLG_ERROR_INVALID_VALUE: return "TLG_ERROR_INVALID_VALUE: an argument is out of range";
        case TLG_ERROR_NOT_SUPPORTED: return "TLG_ERROR_NOT_SUPPORTED: the device or request is not supported";
        case TLG_ERROR_OUT_OF_MEMORY: return "TLG_ERROR_OUT_OF_MEMORY: device memory allocation failed";
        case TLG_ERROR_HIP: return "TLG_ERROR_HIP: the HIP runtime reported an error";
        default: return "unknown tlg_status";
    }
}

int32_t tlg_version(void) { return kVersion; }

tlg_status tlg_gemm_relu_bt(tlg_handle h, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *Bt,
                            int64_t ldbt, void *C, int64_t ldc, hipStream_t stream) {
    return run_bt(h, TLG_VARIANT_AUTO, -1, make_problem(M, N, K, A, lda, Bt, ldbt, C, ldc), stream);
}

tlg_status tlg_gemm_relu_bt_variant(tlg_handle h, int32_t variant, int32_t config, int64_t M, int64_t N, int64_t K,
                                    const void *A, int64_t lda, const void *Bt, int64_t ldbt, void *C, int64_t ldc,
                                    hipStream_t stream) {
    return run_bt(h, variant, config, make_problem(M, N, K, A, lda, Bt, ldbt, C, ldc), stream);
}

tlg_status tlg_plan_bt(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *Bt, int64_t ldbt,
                       const void *C, int64_t ldc, int32_t variant, int32_t config, tlg_plan_info *out) {
    if (!out) return TLG_ERROR_INVALID_VALUE;
    tlg_status st = check_args_bt(M, N, K, A, lda, Bt, ldbt, C, ldc);
    if (st != TLG_SUCCESS) return st;
    tlg::Problem p = make_problem(M, N, K, A, lda, Bt, ldbt, C, ldc);
    p.trans_b = true;
    return plan_bt(p, variant, config, out);
}

tlg_status tlg_gemm_relu_grouped(tlg_handle h, int32_t count, const tlg_gemm_desc *descs, int32_t trans_b,
                                 hipStream_t stream) {
    return run_grouped(h, -1, count, descs, trans_b, stream);
}

tlg_status tlg_gemm_relu_grouped_variant(tlg_handle h, int32_t config, int32_t count, const tlg_gemm_desc *descs,
                                         int32_t trans_b, hipStream_t stream) {
    return run_grouped(h, config, count, descs, trans_b, stream);
}

tlg_status tlg_gemm_relu_mx(tlg_handle h, int32_t format, int64_t M, int64_t N, int64_t K, const void *A,
                            int64_t lda, const void *SA, int64_t ldsa, const void *B, int64_t ldb, const void *SB,
                            int64_t ldsb, void *C, int64_t ldc, hipStream_t stream) {
    return run_mx(h, -1, make_mx_problem(format, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, C, ldc), stream);
}

tlg_status tlg_gemm_relu_mx_variant(tlg_handle h, int32_t config, int32_t format, int64_t M, int64_t N, int64_t K,
                                    const void *A, int64_t lda, const void *SA, int64_t ldsa, const void *B,
                                    int64_t ldb, const void *SB, int64_t ldsb, void *C, int64_t ldc,
                                    hipStream_t stream) {
    return run_mx(h, config, make_mx_problem(format, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, C, ldc), stream);
}

tlg_status tlg_plan_mx(int32_t format, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *SA,
                       int64_t ldsa, const void *B, int64_t ldb, const void *SB, int64_t ldsb, const void *C,
                       int64_t ldc, int32_t config, tlg_plan_info *out) {
    if (!out) return TLG_ERROR_INVALID_VALUE;
    tlg_status st = check_args_mx(format, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, C, ldc);
    if (st != TLG_SUCCESS) return st;
    return plan_mx(make_mx_problem(format, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, C, ldc), config, out);
}

tlg_status tlg_gemm_relu_mx_grouped(tlg_handle h, int32_t format, int32_t count, const tlg_mx_desc *descs,
                                    hipStream_t stream) {
    return run_mx_grouped(h, -1, format, count, descs, stream);
}

tlg_status tlg_gemm_relu_mx_grouped_variant(tlg_handle h, int32_t config, int32_t format, int32_t count,
                                            const tlg_mx_desc *descs, hipStream_t stream) {
    return run_mx_grouped(h, config, format, count, descs, stream);
}

const char *tlg_plan_mx_config_name(int32_t config) {
    return (config >= 0 && config < tlg::MX_CONFIGS) ? tlg::kMxConfigs[config].name : "";
}

}  // extern "C"
