// gfx950 (MI355X, CDNA4) kernels for C = ReLU(A . B), fp16 in, fp32
// accumulation, fp16 out: the quick-start kernel of the TileLang article
// (aiwiki.ai/wiki/tilelang, "Programming model").
//
// What each kernel keeps of that kernel, and what it does differently:
//  * one work-group per BM x BN output tile over a ceil-divided grid, an fp32
//    accumulator cleared at the start, a K loop over LDS tiles of A and B,
//    ReLU applied to the fp32 accumulator, then the cast to fp16 (as in the
//    listing);
//  * the multi-stage pipeline (T.Pipelined in the listing) is built from
//    buffer_load_dwordx4 ... lds, which moves 16 bytes per lane from global
//    memory straight into LDS with no register staging; a stage's loads are
//    waited for with s_waitcnt vmcnt, so STAGES-1 tiles are in flight while
//    one is being multiplied;
//  * out-of-range rows, columns and k are zero-filled by giving those lanes
//    an out-of-range buffer offset (the hardware then writes zeros);
//  * LDS tiles are XOR-swizzled at 16-byte granularity (the bank-conflict
//    minimising layouts of the article's T.gemm), with swizzles chosen for
//    the 64-bank LDS of gfx950 (tile_layout.h);
//  * T.gemm becomes v_mfma_f32_32x32x16_f16; the B operand, which is
//    N-contiguous in memory, is transposed on the way out of LDS with
//    ds_read_b64_tr_b16;
//  * the grid order (T.use_swizzle in the article) is XCD-aware and grouped
//    along M so co-resident work-groups share A rows and B columns in L2;
//  * for skinny M a split-K variant (two stages: fp32 partials, then an
//    ordered reduce + ReLU + cast), the two-stage split-K the article reports
//    SGLang using for small-batch decoding ("Adoption by DeepSeek").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

// ---------------------------------------------------------------------------
// Tiled kernel fed by direct global->LDS loads. Requirements (checked on the
// host): every in-tile byte offset below kRange (2-byte aligned pointers and
// any leading dimension work; ragged K or N take the staged tail block).
// With SPLIT, blockIdx.y is the K split and fp32 partials go to W instead of
// C. BT: B is given transposed (N x K row-major, ldb >= K), its tile is
// loaded and read exactly like A's (BM == BN).
// ---------------------------------------------------------------------------
template <class S, bool SPLIT, bool BT>
__device__ __forceinline__ void tile_dma(const KArgs &a, int m0, int n0, int kbeg, int kend, LDS_PTR(char) lds) {
    static_assert(!BT || (S::BM == S::BN && !SPLIT), "transposed B: square tiles, no split");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int nk = kend > kbeg ? (kend - kbeg + S::BK - 1) / S::BK : 0;

    // Per-lane load descriptors (constant over the K loop): byte offset in
    // the stage's window, the k offset that decides whether the chunk is
    // inside K, and whether the row (or column) is inside M (N).
    uint32_t a_off[S::DMA_A];
    int a_col[S::DMA_A];
    bool a_ok[S::DMA_A];
#pragma unroll
    for (int i = 0; i < S::DMA_A; ++i) {
        ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        a_off[i] = (uint32_t)(c.row * a.lda * 2 + c.chunk * 16);
        a_col[i] = 8 * c.chunk;
        a_ok[i] = m0 + c.row < a.M;
    }
    uint32_t b_off[S::DMA_B];
    int b_k[S::DMA_B];
    bool b_ok[S::DMA_B];
#pragma unroll
    for (int i = 0; i < S::DMA_B; ++i) {
        if (BT) {  // rows n of the transposed B tile, as A's rows m
            ChunkRef c = dma_a_chunk<S>(wave, i, lane);
            b_off[i] = (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16);
            b_k[i] = 8 * c.chunk;
            b_ok[i] = n0 + c.row < a.N;
        } else {
            ChunkRef c = dma_b_chunk<S>(wave, i, lane);
            b_off[i] = (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16);
            b_k[i] = c.row;
            b_ok[i] = n0 + 8 * c.chunk < a.N;
        }
    }

    auto issue = [&](int kt, int buf) {
        const int k0 = kbeg + kt * S::BK;
        LDS_PTR(char) sA = lds + buf * S::STAGE_BYTES;
        LDS_PTR(char) sB = sA + S::A_BYTES;
        const int4_t ra = make_srd(a.A + (int64_t)m0 * a.lda + k0);
        const int4_t rb = make_srd(BT ? a.B + (int64_t)n0 * a.ldb + k0 : a.B + (int64_t)k0 * a.ldb + n0);
        const uint32_t la = (uint32_t)(uintptr_t)(sA + wave * S::DMA_A * 1024);
        const uint32_t lb = (uint32_t)(uintptr_t)(sB + wave * S::DMA_B * 1024);
#pragma unroll
        for (int i = 0; i < S::DMA_A; ++i) {
            uint32_t off = (a_ok[i] && k0 + a_col[i] < kend) ? a_off[i] : kOOB;
            dma16(ra, la + i * 1024, off);
        }
#pragma unroll
        for (int i = 0; i < S::DMA_B; ++i) {
            uint32_t off = (b_ok[i] && k0 + b_k[i] < kend) ? b_off[i] : kOOB;
            dma16(rb, lb + i * 1024, off);
        }
    };

    float16_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    constexpr int kLoadsPerStage = S::DMA_A + S::DMA_B;
#pragma unroll
    for (int s = 0; s < S::STAGES - 1; ++s)
        if (s < nk) issue(s, s);

    int buf = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // Tile kt has landed once at most the loads of the STAGES-2 later
        // tiles are still in flight.
        if (kt + S::STAGES - 2 < nk)
            wait_vmcnt<(S::STAGES - 2) * kLoadsPerStage>();
        else
            wait_vmcnt<0>();
        barrier_lds();  // every wave's loads of tile kt are in LDS; tile kt-1 is no longer read
        if (kt + S::STAGES - 1 < nk) {
            int nb = buf == 0 ? S::STAGES - 1 : buf - 1;  // the buffer tile kt-1 used
            issue(kt + S::STAGES - 1, nb);
        }
        LDS_PTR(const char) sA = lds + buf * S::STAGE_BYTES;
        mma_stage<S, BT>(sA, sA + S::A_BYTES, wm0, wn0, lane, acc);
        buf = buf + 1 == S::STAGES ? 0 : buf + 1;
    }

    // Rows kmain .. K-1 (ragged K or N): one zero-padded block staged element
    // by element into buffer 0 once every wave is done with the stages.
    if (!SPLIT && a.kmain < a.K) {
        barrier_lds();
        stage_tail<S, BT>(a, m0, n0, lds, lds + S::A_BYTES, tid);
        barrier_lds();
        mma_kstep<S, BT>(lds, lds + S::A_BYTES, 0, wm0, wn0, lane, acc);
    }

    // Epilogue: split-K partials go out as fp32 (a lane owns four consecutive
    // n of one row m per register quad); C goes through LDS.
    if (SPLIT) {
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            a.W + ((int64_t)blockIdx.y * a.M + m0) * a.N + n0, (short)0, (int)kRange, 0x00020000);
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < S::TM; ++tm) {
                const int mr = acc_m(wm0, tm, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nr = acc_n(wn0, tn, 4 * q, lane);
                    const bool ok = m0 + mr < a.M && n0 + nr < a.N;  // N % 8 == 0: n..n+3 all in range
                    const uint32_t off = ok ? (uint32_t)((mr * a.N + nr) * 4) : kOOB;
                    float4_t v = {acc[tn][tm][4 * q], acc[tn][tm][4 * q + 1], acc[tn][tm][4 * q + 2],
                                  acc[tn][tm][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, v), rw, off, 0, 0);
                }
            }
    } else {
        barrier_lds();  // every wave is done with the stages (and the tail block)
        store_c_tile_lds<S>(a, m0, n0, wave, lane, acc, lds);
    }
}

template <class S, bool SPLIT, bool BT>
__global__ __launch_bounds__(S::NT) void k_tiled_dma(const KArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[S::LDS_BYTES];
    const int nwg = a.tiles_m * a.tiles_n;
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, nwg), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    const int kbeg = SPLIT ? (int)blockIdx.y * a.k_split : 0;
    const int kend = SPLIT ? imin(a.K, kbeg + a.k_split) : a.kmain;
    tile_dma<S, SPLIT, BT>(a, tm_idx * S::BM, tn_idx * S::BN, kbeg, kend, (LDS_PTR(char))smem);
}

// Several independent problems in one launch: work-group ids are dealt to
// the XCDs as in the single-problem kernel, then split by problem in order
// (tile_start holds the running tile counts).
template <class S, bool BT>
__global__ __launch_bounds__(S::NT) void k_tiled_dma_grouped(const GroupArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem[S::LDS_BYTES];
    const int v = xcd_remap(blockIdx.x, g.tile_start[g.count]);
    int p = 0;
    while (p + 1 < g.count && v >= g.tile_start[p + 1]) ++p;
    const KArgs &a = g.p[p];
    int tm_idx, tn_idx;
    grouped_tile(v - g.tile_start[p], a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    tile_dma<S, false, BT>(a, tm_idx * S::BM, tn_idx * S::BN, 0, a.kmain, (LDS_PTR(char))smem);
}

// ---------------------------------------------------------------------------
// Tiled kernel fed through registers: any alignment, any leading dimension,
// any M, N, K. Each thread moves 16-byte chunks: a chunk wholly inside the
// matrix is one 16-byte buffer load (gfx950 buffer loads accept any 2-byte
// aligned offset, so odd leading dimensions and pointers need no special
// case; FAST = false drops this when in-tile offsets would not fit 32 bits),
// a chunk that crosses the M, N or K edge is gathered element by element with
// bounds checks (out-of-range elements are 0). Chunks are written to the same
// swizzled LDS layout as the direct-to-LDS kernels; two LDS buffers, the next
// tile's loads in flight during the current tile's MFMAs.
// ---------------------------------------------------------------------------
template <class S, bool FAST>
__global__ __launch_bounds__(S::NT) void k_tiled_general(const KArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * S::STAGE_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;

    const int nwg = a.tiles_m * a.tiles_n;
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, nwg), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    const int m0 = tm_idx * S::BM, n0 = tn_idx * S::BN;
    const int nk = (a.K + S::BK - 1) / S::BK;

    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    half8_t ra[S::JA], rb[S::JB];

    auto gload = [&](int kt) {
        const int k0 = kt * S::BK;
        const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.A + (int64_t)m0 * a.lda + k0), (short)0, (int)kRange, 0x00020000);
        const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.B + (int64_t)k0 * a.ldb + n0), (short)0, (int)kRange, 0x00020000);
#pragma unroll
        for (int j = 0; j < S::JA; ++j) {
            ChunkRef c = reg_a_chunk<S>(tid, j);
            const int m = m0 + c.row, k = k0 + 8 * c.chunk;
            if (FAST && m < a.M && k + 8 <= a.K) {
                ra[j] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rA, (uint32_t)((c.row * a.lda + 8 * c.chunk) * 2), 0, 0));
            } else {
                const _Float16 *p = a.A + (int64_t)m * a.lda + k;
#pragma unroll
                for (int e = 0; e < 8; ++e) ra[j][e] = (m < a.M && k + e < a.K) ? p[e] : (_Float16)0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < S::JB; ++j) {
            ChunkRef c = reg_b_chunk<S>(tid, j);
            const int k = k0 + c.row, n = n0 + 8 * c.chunk;
            if (FAST && k < a.K && n + 8 <= a.N) {
                rb[j] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rB, (uint32_t)((c.row * a.ldb + 8 * c.chunk) * 2), 0, 0));
            } else {
                const _Float16 *p = a.B + (int64_t)k * a.ldb + n;
#pragma unroll
                for (int e = 0; e < 8; ++e) rb[j][e] = (k < a.K && n + e < a.N) ? p[e] : (_Float16)0.0f;
            }
        }
    };
    auto swrite = [&](int buf) {
        LDS_PTR(char) sA = lds + buf * S::STAGE_BYTES;
        LDS_PTR(char) sB = sA + S::A_BYTES;
#pragma unroll
        for (int j = 0; j < S::JA; ++j) {
            ChunkRef c = reg_a_chunk<S>(tid, j);
            *(LDS_PTR(half8_t))(sA + lds_a_offset<S>(c.row, c.chunk)) = ra[j];
        }
#pragma unroll
        for (int j = 0; j < S::JB; ++j) {
            ChunkRef c = reg_b_chunk<S>(tid, j);
            *(LDS_PTR(half8_t))(sB + lds_b_offset<S>(c.row, c.chunk)) = rb[j];
        }
    };

    float16_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        gload(0);
        swrite(0);
        barrier_lds();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        LDS_PTR(const char) sA = lds + buf * S::STAGE_BYTES;
        mma_stage<S>(sA, sA + S::A_BYTES, wm0, wn0, lane, acc);
        if (kt + 1 < nk) swrite(buf ^ 1);
        barrier_lds();
    }

#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const int m = m0 + acc_m(wm0, tm, lane);
            if (m >= a.M) continue;
            _Float16 *crow = a.C + (int64_t)m * a.ldc;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = n0 + acc_n(wn0, tn, r, lane);
                if (n < a.N) crow[n] = relu_to_half(acc[tn][tm][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// Split-K stage 2: C[m][n] = rne16(relu(sum over s ascending of W[s][m][n])).
// Four consecutive n per thread; N % 4 == 0, ldc % 4 == 0, C 8-byte aligned.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ W, int splits, int M, int N,
                                                       _Float16 *__restrict__ C, int64_t ldc) {
    const int64_t mn = (int64_t)M * N;
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (idx >= mn) return;
    float4_t acc = *(const float4_t *)(W + idx);
    for (int s = 1; s < splits; ++s) {
        float4_t v = *(const float4_t *)(W + s * mn + idx);
        acc[0] = acc[0] + v[0];
        acc[1] = acc[1] + v[1];
        acc[2] = acc[2] + v[2];
        acc[3] = acc[3] + v[3];
    }
    const int m = (int)(idx / N), n = (int)(idx % N);
    half4_t h = {relu_to_half(acc[0]), relu_to_half(acc[1]), relu_to_half(acc[2]), relu_to_half(acc[3])};
    *(half4_t *)(C + (int64_t)m * ldc + n) = h;
}

// ---------------------------------------------------------------------------
// Cross-check kernel: one thread per output, k ascending, fp32 accumulator.
// fp16 x fp16 products are exact in fp32, so a fused or unfused multiply-add
// gives the same bits and this kernel reproduces the sequential definition
// exactly.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_naive(const KArgs a) {
    const int n = blockIdx.x * 16 + (threadIdx.x & 15);
    const int m = blockIdx.y * 16 + (threadIdx.x >> 4);
    if (m >= a.M || n >= a.N) return;
    const _Float16 *arow = a.A + (int64_t)m * a.lda;
    float acc = 0.0f;
    for (int k = 0; k < a.K; ++k) acc = __builtin_fmaf((float)arow[k], (float)a.B[(int64_t)k * a.ldb + n], acc);
    a.C[(int64_t)m * a.ldc + n] = relu_to_half(acc);
}

// K == 0: the empty sum is +0 and ReLU keeps it.
__global__ __launch_bounds__(256) void k_fill_zero(_Float16 *C, int M, int N, int64_t ldc) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
        C[(i / N) * ldc + (i % N)] = (_Float16)0.0f;
}

// ---------------------------------------------------------------------------
// Configurations and launchers
// ---------------------------------------------------------------------------
using Dma256 = TileShape<256, 256, 32, 2, 2, 4>;
using Dma128 = TileShape<128, 128, 32, 2, 2, 4>;
using Dma64 = TileShape<64, 64, 64, 2, 2, 3>;
using Dma256w8 = TileShape<256, 256, 64, 2, 4, 2>;
using Dma256w8x32 = TileShape<256, 256, 32, 2, 4, 4>;
using Gen128 = TileShape<128, 128, 32, 2, 2, 2>;
using Gen64 = TileShape<64, 64, 32, 2, 2, 2>;
using Split32x128 = TileShape<32, 128, 64, 1, 4, 4>;
using Split32x256 = TileShape<32, 256, 64, 1, 4, 3>;

const TileConfig kDmaConfigs[DMA_CONFIGS] = {
    {Dma256::BM, Dma256::BN, Dma256::BK, Dma256::NT, Dma256::STAGES, "dma_256x256x32_w2x2_s4"},
    {Dma128::BM, Dma128::BN, Dma128::BK, Dma128::NT, Dma128::STAGES, "dma_128x128x32_w2x2_s4"},
    {Dma64::BM, Dma64::BN, Dma64::BK, Dma64::NT, Dma64::STAGES, "dma_64x64x64_w2x2_s3"},
    {Dma256w8::BM, Dma256w8::BN, Dma256w8::BK, Dma256w8::NT, Dma256w8::STAGES, "dma_256x256x64_w2x4_s2"},
    {Dma256w8x32::BM, Dma256w8x32::BN, Dma256w8x32::BK, Dma256w8x32::NT, Dma256w8x32::STAGES,
     "dma_256x256x32_w2x4_s4"},
};
const TileConfig kGenConfigs[GEN_CONFIGS] = {
    {Gen128::BM, Gen128::BN, Gen128::BK, Gen128::NT, 2, "gen_128x128x32_w2x2"},
    {Gen64::BM, Gen64::BN, Gen64::BK, Gen64::NT, 2, "gen_64x64x32_w2x2"},
};
const TileConfig kSplitConfigs[SPLIT_TWO_KERNEL_CONFIGS] = {
    {Split32x128::BM, Split32x128::BN, Split32x128::BK, Split32x128::NT, Split32x128::STAGES,
     "splitk_32x128x64_w1x4_s4"},
    {Split32x256::BM, Split32x256::BN, Split32x256::BK, Split32x256::NT, Split32x256::STAGES,
     "splitk_32x256x64_w1x4_s3"},
};

static KArgs make_args(const Problem &p, bool bt = false) {
    KArgs a;
    a.A = (const _Float16 *)p.A;
    a.B = (const _Float16 *)p.B;
    a.C = (_Float16 *)p.C;
    a.W = nullptr;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.group_m = 4;
    a.k_split = (int)p.K;
    // direct-to-LDS loads stop at the last multiple of 8 below K when a
    // 16-byte chunk could cross the end of a row (K-contiguous A or
    // transposed B: K % 8; N-contiguous B: N % 8)
    const bool whole = p.K % 8 == 0 && (bt || p.N % 8 == 0);
    a.kmain = whole ? (int)p.K : (int)(8 * ((p.K - 1) / 8));
    return a;
}

template <class S, bool SPLIT, bool BT = false>
static hipError_t launch_dma_t(KArgs a, int splits, hipStream_t stream) {
    a.tiles_m = (a.M + S::BM - 1) / S::BM;
    a.tiles_n = (a.N + S::BN - 1) / S::BN;
    dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)splits);
    hipLaunchKernelGGL((k_tiled_dma<S, SPLIT, BT>), grid, dim3(S::NT), 0, stream, a);
    return hipGetLastError();
}

template <class S, bool BT>
static hipError_t launch_grouped_t(const Problem *ps, int count, hipStream_t stream) {
    GroupArgs g;
    g.count = count;
    g.tile_start[0] = 0;
    for (int i = 0; i < count; ++i) {
        KArgs a = make_args(ps[i], BT);
        a.tiles_m = (a.M + S::BM - 1) / S::BM;
        a.tiles_n = (a.N + S::BN - 1) / S::BN;
        g.p[i] = a;
        g.tile_start[i + 1] = g.tile_start[i] + a.tiles_m * a.tiles_n;
    }
    if (g.tile_start[count] == 0) return hipSuccess;
    hipLaunchKernelGGL((k_tiled_dma_grouped<S, BT>), dim3((unsigned)g.tile_start[count]), dim3(S::NT), 0, stream, g);
    return hipGetLastError();
}

template <class S>
static hipError_t launch_gen_t(KArgs a, hipStream_t stream) {
    a.tiles_m = (a.M + S::BM - 1) / S::BM;
    a.tiles_n = (a.N + S::BN - 1) / S::BN;
    // the 16-byte loads address a tile through 32-bit offsets
    const bool fast = (int64_t)S::BM * a.lda * 2 < (int64_t)kRange && (int64_t)S::BK * a.ldb * 2 < (int64_t)kRange;
    if (fast)
        hipLaunchKernelGGL((k_tiled_general<S, true>), dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(S::NT), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((k_tiled_general<S, false>), dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(S::NT), 0,
                           stream, a);
    return hipGetLastError();
}

hipError_t launch_tiled_dma(int config, const Problem &p, hipStream_t stream) {
    KArgs a = make_args(p, p.trans_b);
    if (p.trans_b) {
        switch (config) {
            case DMA_256x256x32: return launch_dma_t<Dma256, false, true>(a, 1, stream);
            case DMA_128x128x32: return launch_dma_t<Dma128, false, true>(a, 1, stream);
            case DMA_64x64x64: return launch_dma_t<Dma64, false, true>(a, 1, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (config) {
        case DMA_256x256x32: return launch_dma_t<Dma256, false>(a, 1, stream);
        case DMA_128x128x32: return launch_dma_t<Dma128, false>(a, 1, stream);
        case DMA_64x64x64: return launch_dma_t<Dma64, false>(a, 1, stream);
        case DMA_256x256x64_W8: return launch_dma_t<Dma256w8, false>(a, 1, stream);
        case DMA_256x256x32_W8: return launch_dma_t<Dma256w8x32, false>(a, 1, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_tiled_dma_grouped(int config, const Problem *ps, int count, hipStream_t stream) {
    static_assert(sizeof(GroupArgs) <= 4096, "kernel arguments");
    if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
    const bool bt = ps[0].trans_b;
    for (int i = 1; i < count; ++i)
        if (ps[i].trans_b != bt) return hipErrorInvalidValue;
    switch (config) {
        case DMA_256x256x32:
            return bt ? launch_grouped_t<Dma256, true>(ps, count, stream) : launch_grouped_t<Dma256, false>(ps, count, stream);
        case DMA_128x128x32:
            return bt ? launch_grouped_t<Dma128, true>(ps, count, stream) : launch_grouped_t<Dma128, false>(ps, count, stream);
        case DMA_64x64x64:
            return bt ? launch_grouped_t<Dma64, true>(ps, count, stream) : launch_grouped_t<Dma64, false>(ps, count, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_tiled_general(int config, const Problem &p, hipStream_t stream) {
    KArgs a = make_args(p);
    switch (config) {
        case GEN_128x128x32: return launch_gen_t<Gen128>(a, stream);
        case GEN_64x64x32: return launch_gen_t<Gen64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_splitk(int config, int splits, int64_t k_split, const Problem &p, float *workspace,
                         hipStream_t stream) {
    KArgs a = make_args(p);
    a.W = workspace;
    a.k_split = (int)k_split;
    hipError_t e;
    switch (config) {
        case SPLIT_32x128x64: e = launch_dma_t<Split32x128, true>(a, splits, stream); break;
        case SPLIT_32x256x64: e = launch_dma_t<Split32x256, true>(a, splits, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t quads = (p.M * p.N) / 4;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream,
                       (const float *)workspace, splits, (int)p.M, (int)p.N, (_Float16 *)p.C, p.ldc);
    return hipGetLastError();
}

hipError_t launch_naive(const Problem &p, hipStream_t stream) {
    KArgs a = make_args(p);
    dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.M + 15) / 16));
    hipLaunchKernelGGL(k_naive, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(const Problem &p, hipStream_t stream) {
    const int64_t total = p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, (_Float16 *)p.C, (int)p.M,
                       (int)p.N, p.ldc);
    return hipGetLastError();
}

}  // namespace tlg
