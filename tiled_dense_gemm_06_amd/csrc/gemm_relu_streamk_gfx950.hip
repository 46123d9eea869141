// Stream-K split of the K loop for skinny problems (few output tiles, long K):
// the two-stage split-K that the TileLang article reports SGLang using for
// small-batch decoding (aiwiki.ai/wiki/tilelang, "Adoption by DeepSeek"),
// arranged for one MI355X.
//
// The output tiles' K iterations form one sequence (tile-major, k ascending
// inside a tile). Work-group g of G takes the contiguous range
// [g*total/G, (g+1)*total/G) of it, so every work-group streams the same
// number of B bytes and the grid is sized to the number of work-groups the
// CUs hold at once: no tile quantisation and no second round. Inside its range
// a work-group runs the direct-to-LDS pipeline of k_tiled_dma without a break
// at tile boundaries.
//
// A tile covered whole by one work-group gets ReLU + fp16 written directly.
// A tile split between work-groups is finished in the same kernel: each part
// stores its fp32 partial tile in a private slot of the workspace with
// device-scope stores (the sc1 cache policy: written through to the level
// shared by all XCDs), and once every store of the work-group has completed
// it adds its iteration count to the tile's counter with a device-scope
// atomic. The work-group that completes the count reads the tile's partials
// with device-scope loads, sums them in ascending k order (so the result does
// not depend on which work-group finishes last), applies ReLU and the fp16
// cast, writes C and resets the counter to zero for the next call. Only these
// few accesses carry the device scope; a fence would instead write back and
// invalidate a whole XCD's L2. No work-group ever waits for another, so no
// co-residency is assumed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

struct SKArgs {
    const _Float16 *A;
    const _Float16 *B;
    _Float16 *C;
    float *P;    // partial slots: [G][2][BM * BN] fp32
    int *cnt;    // per-tile iteration counters, zero between calls
    int M, N, K;
    int64_t lda, ldb, ldc;
    int tiles_m;
    int ipt;        // K iterations per tile
    int total;      // tiles * ipt
};

// Cache policy of the partial-tile stores and loads: sc1, device scope.
// Partials from work-groups on different XCDs meet through these bits alone.
// On gfx950 an sc1 load or store is coherent at device scope (it is how the
// compiler implements a relaxed agent-scope atomic load or store), so each
// partial lives in one device-wide modification order and no XCD's L2 holds
// a stale copy of it. The order between a part's partials and its count
// comes from the wait for store completion (vmcnt(0) in every thread, then
// the work-group barrier) before the count's atomic is issued; the reading
// part issues its partial loads only after its own count has returned the
// total. Nothing else is read across work-groups, so the L2 write-back and
// invalidate that an agent-scope release/acquire pair adds (measured: 5 to
// 40 % longer calls on the split shapes) are not needed.
constexpr int kDeviceScope = 16;

template <class S>
__global__ __launch_bounds__(S::NT) void k_streamk(const SKArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[S::LDS_BYTES];
    constexpr int LOADS = S::DMA_A + S::DMA_B;
    constexpr int TILE = S::BM * S::BN;
    static_assert(S::STAGES == 4, "waits written for four stages");
    static_assert(TILE % (4 * S::NT) == 0, "reduction reads whole float4s");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int g = blockIdx.x, G = gridDim.x;
    const int beg = (int)sk_begin(g, a.total, G), end = (int)sk_begin(g + 1, a.total, G);

    LDS_PTR(char) lds = (LDS_PTR(char))smem;

    // Issue the loads of iteration kt of tile t into LDS buffer buf.
    auto issue = [&](int t, int kt, int buf) {
        const int k0 = kt * S::BK;
        const int m0 = (t % a.tiles_m) * S::BM, n0 = (t / a.tiles_m) * S::BN;
        const int4_t ra = make_srd(a.A + (int64_t)m0 * a.lda + k0);
        const int4_t rb = make_srd(a.B + (int64_t)k0 * a.ldb + n0);
        LDS_PTR(char) sA = lds + buf * S::STAGE_BYTES;
        const uint32_t la = (uint32_t)(uintptr_t)(sA + wave * S::DMA_A * 1024);
        const uint32_t lb = (uint32_t)(uintptr_t)(sA + S::A_BYTES + wave * S::DMA_B * 1024);
#pragma unroll
        for (int i = 0; i < S::DMA_A; ++i) {
            const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
            const bool in = m0 + c.row < a.M && k0 + 8 * c.chunk < a.K;
            dma16(ra, la + i * 1024, in ? (uint32_t)(c.row * a.lda * 2 + c.chunk * 16) : kOOB);
        }
#pragma unroll
        for (int i = 0; i < S::DMA_B; ++i) {
            const ChunkRef c = dma_b_chunk<S>(wave, i, lane);
            const bool in = n0 + 8 * c.chunk < a.N && k0 + c.row < a.K;
            dma16(rb, lb + i * 1024, in ? (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16) : kOOB);
        }
    };

    float16_t acc[S::TN][S::TM];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < S::TN; ++i)
#pragma unroll
            for (int j = 0; j < S::TM; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    };

    // ReLU + fp16 stores of a finished tile (rows >= M and columns >= N dropped
    // by the buffer range check).
    auto store_c = [&](int t) {
        const int m0 = (t % a.tiles_m) * S::BM, n0 = (t / a.tiles_m) * S::BN;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(a.C + (int64_t)m0 * a.ldc + n0, (short)0,
                                                                            (int)kRange, 0x00020000);
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < S::TM; ++tm) {
                const int mr = acc_m(wm0, tm, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nr = acc_n(wn0, tn, 4 * q, lane);
                    const bool in = m0 + mr < a.M && n0 + nr < a.N;
                    const uint32_t o = in ? (uint32_t)((mr * a.ldc + nr) * 2) : kOOB;
                    half4_t h = {relu_to_half(acc[tn][tm][4 * q]), relu_to_half(acc[tn][tm][4 * q + 1]),
                                 relu_to_half(acc[tn][tm][4 * q + 2]), relu_to_half(acc[tn][tm][4 * q + 3])};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(int2_t, h), rc, o, 0, 0);
                }
            }
    };

    // fp32 partial of a split tile into this work-group's slot (rows >= M skipped).
    auto store_partial = [&](int t, int slot) {
        const int m0 = (t % a.tiles_m) * S::BM;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            a.P + ((int64_t)g * 2 + slot) * TILE, (short)0, (int)kRange, 0x00020000);
        // (stored with the device-scope policy: read by another work-group)
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < S::TM; ++tm) {
                const int mr = acc_m(wm0, tm, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nr = acc_n(wn0, tn, 4 * q, lane);
                    const uint32_t o = m0 + mr < a.M ? (uint32_t)((mr * S::BN + nr) * 4) : kOOB;
                    float4_t v = {acc[tn][tm][4 * q], acc[tn][tm][4 * q + 1], acc[tn][tm][4 * q + 2],
                                  acc[tn][tm][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, v), rp, o, 0, kDeviceScope);
                }
            }
    };

    // The split tiles of this range: at most the first and the last tile it touches.
    int part_tile[2] = {-1, -1};
    int part_len[2] = {0, 0};

    // (tile, k iteration) of the next load to issue and of the next product,
    // advanced one iteration at a time (no division in the loop)
    int t_ld = beg / a.ipt, k_ld = beg - t_ld * a.ipt;
    int t_mm = t_ld, k_mm = k_ld;
    auto advance = [&](int &t, int &k) {
        if (++k == a.ipt) {
            k = 0;
            ++t;
        }
    };

    zero_acc();
#pragma unroll
    for (int s = 0; s < S::STAGES - 1; ++s)
        if (beg + s < end) {
            issue(t_ld, k_ld, s);
            advance(t_ld, k_ld);
        }

    int buf = 0;
    int seg_lo = beg;
    for (int i = beg; i < end; ++i) {
        const int after = end - 1 - i;  // iterations of this range after i
        if (after >= 2)
            wait_vmcnt<2 * LOADS>();
        else if (after == 1)
            wait_vmcnt<LOADS>();
        else
            wait_vmcnt<0>();
        barrier_lds();  // iteration i is in LDS for every wave; iteration i-1's buffer is free
        if (i + S::STAGES - 1 < end) {
            issue(t_ld, k_ld, buf == 0 ? S::STAGES - 1 : buf - 1);
            advance(t_ld, k_ld);
        }
        LDS_PTR(const char) sA = lds + buf * S::STAGE_BYTES;
        mma_stage<S>(sA, sA + S::A_BYTES, wm0, wn0, lane, acc);
        buf = buf + 1 == S::STAGES ? 0 : buf + 1;

        if (k_mm + 1 == a.ipt || i + 1 == end) {
            const int t = t_mm;
            if (seg_lo == t * a.ipt && k_mm + 1 == a.ipt) {
                store_c(t);
            } else {
                const int slot = seg_lo == beg ? 0 : 1;
                store_partial(t, slot);
                part_tile[slot] = t;
                part_len[slot] = i + 1 - seg_lo;
            }
            zero_acc();
            seg_lo = i + 1;
        }
        advance(t_mm, k_mm);
    }

    if (part_tile[0] < 0 && part_tile[1] < 0) return;

    // Count this range's partials into their tiles once all its stores have
    // completed. The loads are all done too, so the first bytes of the stage
    // buffers carry the "this work-group finishes the tile" flags (keeping LDS
    // at two work-groups per CU).
    int *s_last = (int *)smem;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every store of this thread is done
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s_last[s] = 0;
            if (part_tile[s] >= 0) {
                const int old = __hip_atomic_fetch_add(&a.cnt[part_tile[s]], part_len[s], __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                s_last[s] = old + part_len[s] == a.ipt;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if (!s_last[s]) continue;
        const int t = part_tile[s];
        const int m0 = (t % a.tiles_m) * S::BM, n0 = (t / a.tiles_m) * S::BN;
        const int first = t * a.ipt;
        const int g0 = sk_owner(first, a.total, G), g1 = sk_owner(first + a.ipt - 1, a.total, G);
        // Each thread finishes 4 consecutive columns of TILE / (4 * NT) rows.
#pragma unroll
        for (int e0 = 0; e0 < TILE; e0 += 4 * S::NT) {
            const int e = e0 + 4 * tid;
            const int m = e / S::BN, n = e % S::BN;
            if (m0 + m >= a.M || n0 + n >= a.N) continue;
            float4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int gg = g0; gg <= g1; ++gg) {
                const int64_t gb = sk_begin(gg, a.total, G);
                if (sk_begin(gg + 1, a.total, G) == gb) continue;  // an empty range owns nothing
                const int slot = gb >= first ? 0 : 1;
                const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                    a.P + ((int64_t)gg * 2 + slot) * TILE, (short)0, (int)kRange, 0x00020000);
                const float4_t v = __builtin_bit_cast(
                    float4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(e * 4), 0, kDeviceScope));
                sum[0] = sum[0] + v[0];
                sum[1] = sum[1] + v[1];
                sum[2] = sum[2] + v[2];
                sum[3] = sum[3] + v[3];
            }
            half4_t h = {relu_to_half(sum[0]), relu_to_half(sum[1]), relu_to_half(sum[2]), relu_to_half(sum[3])};
            *(half4_t *)(a.C + (int64_t)(m0 + m) * a.ldc + n0 + n) = h;
        }
        if (tid == 0) __hip_atomic_store(&a.cnt[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

using SK32x128 = TileShape<32, 128, 64, 1, 4, 4>;

const TileConfig kStreamKConfig = {SK32x128::BM, SK32x128::BN, SK32x128::BK, SK32x128::NT, SK32x128::STAGES,
                                   "streamk_32x128x64_w1x4_s4"};

hipError_t launch_streamk(const Problem &p, int grid, float *partials, int *counters, hipStream_t stream) {
    SKArgs a;
    a.A = (const _Float16 *)p.A;
    a.B = (const _Float16 *)p.B;
    a.C = (_Float16 *)p.C;
    a.P = partials;
    a.cnt = counters;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.tiles_m = (int)((p.M + SK32x128::BM - 1) / SK32x128::BM);
    const int64_t tiles_n = (p.N + SK32x128::BN - 1) / SK32x128::BN;
    a.ipt = (int)((p.K + SK32x128::BK - 1) / SK32x128::BK);
    a.total = (int)((int64_t)a.tiles_m * tiles_n * a.ipt);
    static_assert(SK32x128::LDS_BYTES * kStreamKBlocksPerCU <= 160 * 1024, "occupancy assumed by the planner");
    hipLaunchKernelGGL(k_streamk<SK32x128>, dim3((unsigned)grid), dim3(SK32x128::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tlg
