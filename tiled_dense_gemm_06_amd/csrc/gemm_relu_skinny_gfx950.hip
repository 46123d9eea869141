// Skinny problems (M <= 64, many columns): split-K inside one work-group.
//
// The two-stage split-K of the TileLang article (aiwiki.ai/wiki/tilelang,
// "Adoption by DeepSeek": K partitioned for small-batch decoding, partial
// results reduced afterwards), arranged so that the reduction never leaves a
// work-group. With M this small the kernel is bound by reading B once from
// HBM, so it is built for memory-level parallelism rather than for the
// matrix cores:
//  * one work-group per 64-column strip of B and C;
//  * its waves split the strip's K blocks (wave w of W takes blocks w,
//    w + W, ...), each with a private ring of direct-to-LDS loads, so no wave
//    ever waits for another inside the K loop and W x STAGES blocks per
//    work-group are in flight;
//  * each wave multiplies its blocks with v_mfma_f32_32x32x16_f16 (B
//    transposed on the way out of LDS by ds_read_b64_tr_b16, M padded to 32
//    with zero rows that cost no memory traffic);
//  * at the end the waves' partial tiles meet in LDS and are summed in wave
//    order (a fixed order, so results are deterministic), then ReLU and the
//    round-to-nearest-even fp16 cast.
// Block depth, stage count and waves were chosen by measurement on MI355X
// (64-deep blocks keep every row piece of B a whole 128-byte line).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

// Direct-to-LDS 16-byte load of B with the non-temporal policy: every byte
// of B is read once, and the hint measured about 1 % faster here
// (16 x 14336 x 4096: 24.51 vs 24.76 us; sc1, or sc1 with nt, no better).
__device__ __forceinline__ void dma16_nt(int4_t srd, uint32_t lds_base, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(lds_base),
        "v"(voff), "s"(srd)
        : "memory", "m0");
}

// Wait until at most `n` blocks of this wave are still loading (n < STAGES).
template <int LOADS, int STAGES>
__device__ __forceinline__ void wait_blocks(int n) {
    static_assert(STAGES <= 4, "waits written for up to four stages");
    if (STAGES > 3 && n >= 3)
        wait_vmcnt<(STAGES > 3 ? 3 : 0) * LOADS>();
    else if (STAGES > 2 && n >= 2)
        wait_vmcnt<(STAGES > 2 ? 2 : 0) * LOADS>();
    else if (n >= 1)
        wait_vmcnt<LOADS>();
    else
        wait_vmcnt<0>();
}

// Cache policy of the partial-strip stores and loads: sc1, device scope
// (the same combining scheme, and the same ordering argument, as the
// stream-K tiles' partials, kDeviceScope).
constexpr int kPartialScope = 16;

// Grid: strips x parts (a.k_split parts per strip, adjacent work-groups share
// a strip). Part p takes the strip's K blocks [p*nkb/parts, (p+1)*nkb/parts).
// BT (B given transposed, N x K): a block of B is BN rows n of 64 k, loaded
// and read the way A's rows are.
template <class S, int W, bool BT = false>
__global__ __launch_bounds__(W * 64) void k_skinny_strip(const KArgs a) {
    static_assert(S::WAVES == 1, "one wave per ring");
    constexpr int LOADS = S::DMA_A + S::DMA_B;  // loads per block per wave
    constexpr int RING = S::STAGES * S::STAGE_BYTES;
    constexpr int TILE = S::BM * S::BN;
    static_assert(TILE * 4 <= RING, "partials fit in the rings");
    __shared__ __attribute__((aligned(1024))) char smem[W * RING];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int parts = a.k_split, strip = blockIdx.x / parts, part = blockIdx.x - strip * parts;
    const int n0 = strip * S::BN;
    const int nkb = (a.K + S::BK - 1) / S::BK;                         // K blocks of the strip
    const int kb0 = (int)((int64_t)part * nkb / parts);                // this part's blocks [kb0, kb1)
    const int kb1 = (int)((int64_t)(part + 1) * nkb / parts);
    const int nmine = kb1 - kb0;
    const int mine = nmine > wave ? (nmine - wave + W - 1) / W : 0;    // this wave's blocks

    LDS_PTR(char) ring = (LDS_PTR(char))smem + wave * RING;

    // Block j of this wave (block kb0 + wave + W j of the strip) into stage buffer buf.
    static_assert(!BT || S::BN * S::BK * 2 == S::DMA_B * 1024, "a transposed B block is whole loads of A's kind");
    auto issue = [&](int j, int buf) {
        const int k0 = (kb0 + wave + W * j) * S::BK;
        const int4_t ra = make_srd(a.A + k0);
        const int4_t rb = make_srd(BT ? a.B + (int64_t)n0 * a.ldb + k0 : a.B + (int64_t)k0 * a.ldb + n0);
        LDS_PTR(char) st = ring + buf * S::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < S::DMA_A; ++i) {
            const ChunkRef c = dma_a_chunk<S>(0, i, lane);
            const bool in = c.row < a.M && k0 + 8 * c.chunk < a.K;
            dma16(ra, (uint32_t)(uintptr_t)(st + i * 1024), in ? (uint32_t)(c.row * a.lda * 2 + c.chunk * 16) : kOOB);
        }
#pragma unroll
        for (int i = 0; i < S::DMA_B; ++i) {
            const ChunkRef c = BT ? dma_a_chunk<S>(0, i, lane) : dma_b_chunk<S>(0, i, lane);
            const bool in = BT ? n0 + c.row < a.N && k0 + 8 * c.chunk < a.K
                               : n0 + 8 * c.chunk < a.N && k0 + c.row < a.K;
            dma16_nt(rb, (uint32_t)(uintptr_t)(st + S::A_BYTES + i * 1024),
                     in ? (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16) : kOOB);
        }
    };

    float16_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
    for (int s = 0; s < S::STAGES; ++s)
        if (s < mine) issue(s, s);
    int buf = 0;
    for (int j = 0; j < mine; ++j) {
        // this wave's blocks still in flight behind block j may keep loading
        wait_blocks<LOADS, S::STAGES>(imin(S::STAGES - 1, mine - 1 - j));
        LDS_PTR(const char) st = ring + buf * S::STAGE_BYTES;
        mma_stage<S, BT>(st, st + S::A_BYTES, 0, 0, lane, acc);
        // every read of this buffer is complete before the block STAGES ahead
        // is loaded into it (compiler-visible lgkmcnt(0))
        __builtin_amdgcn_s_waitcnt(0xC07F);
        if (j + S::STAGES < mine) issue(j + S::STAGES, buf);
        buf = buf + 1 == S::STAGES ? 0 : buf + 1;
    }

    // The waves' partial tiles meet in LDS (the rings are no longer used),
    // laid out [wave][m][n] fp32.
    __syncthreads();
    float *lds_part = (float *)smem;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const int mr = acc_m(0, tm, lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nr = acc_n(0, tn, 4 * q, lane);
                float4_t v = {acc[tn][tm][4 * q], acc[tn][tm][4 * q + 1], acc[tn][tm][4 * q + 2],
                              acc[tn][tm][4 * q + 3]};
                *(float4_t *)(lds_part + wave * TILE + mr * S::BN + nr) = v;
            }
        }
    __syncthreads();
    // Thread t owns groups of four consecutive columns: sum over the waves in order.
    constexpr int GROUPS = TILE / (4 * W * 64);
    static_assert(TILE % (4 * W * 64) == 0, "whole groups per thread");
    float4_t sum[GROUPS];
#pragma unroll
    for (int r = 0; r < GROUPS; ++r) {
        const int e = 4 * (tid + r * W * 64);
        float4_t s = *(const float4_t *)(lds_part + e);
#pragma unroll
        for (int w = 1; w < W; ++w) {
            const float4_t v = *(const float4_t *)(lds_part + w * TILE + e);
            s[0] = s[0] + v[0];
            s[1] = s[1] + v[1];
            s[2] = s[2] + v[2];
            s[3] = s[3] + v[3];
        }
        sum[r] = s;
    }
    auto store_groups = [&](const float4_t (&v)[GROUPS]) {
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) {
            const int e = 4 * (tid + r * W * 64);
            const int m = e / S::BN, n = e % S::BN;
            if (m >= a.M || n0 + n >= a.N) continue;
            half4_t h = {relu_to_half(v[r][0]), relu_to_half(v[r][1]), relu_to_half(v[r][2]), relu_to_half(v[r][3])};
            *(half4_t *)(a.C + (int64_t)m * a.ldc + n0 + n) = h;
        }
    };
    if (parts == 1) {
        store_groups(sum);
        return;
    }

    // Split strip: this part's sum goes to its slot (device-scope stores),
    // then, once every store of the work-group is done, it is counted in;
    // the part that completes the count adds the slots in part order
    // (its own from registers), applies ReLU and the cast, and resets the
    // counter for the next call.
    float *slots = a.W + (int64_t)strip * parts * TILE;
    {
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(slots + (int64_t)part * TILE, (short)0,
                                                                            (int)kRange, 0x00020000);
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) {
            const int e = 4 * (tid + r * W * 64);
            if (e / S::BN >= a.M) continue;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, sum[r]), rp, (uint32_t)(e * 4), 0,
                                                   kPartialScope);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
    __syncthreads();
    int *s_last = (int *)smem;  // LDS is free: the sums are in registers
    if (tid == 0)
        s_last[0] = __hip_atomic_fetch_add(&a.cnt[strip], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    parts - 1;
    __syncthreads();
    if (!s_last[0]) return;
    float4_t tot[GROUPS];
#pragma unroll
    for (int r = 0; r < GROUPS; ++r) tot[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = 0; q < parts; ++q) {
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(slots + (int64_t)q * TILE, (short)0,
                                                                            (int)kRange, 0x00020000);
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) {
            const int e = 4 * (tid + r * W * 64);
            float4_t v = sum[r];
            if (q != part)
                v = __builtin_bit_cast(float4_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(e * 4), 0, kPartialScope));
            tot[r][0] = tot[r][0] + v[0];
            tot[r][1] = tot[r][1] + v[1];
            tot[r][2] = tot[r][2] + v[2];
            tot[r][3] = tot[r][3] + v[3];
        }
    }
    store_groups(tot);
    if (tid == 0) __hip_atomic_store(&a.cnt[strip], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stream-K over strips: with fewer strips than work-groups the CUs can hold,
// one work-group per strip leaves CUs idle (16 x 14336: 224 strips on 256
// CUs). Here the strips' K blocks form one sequence (strip-major, K
// ascending inside a strip) and work-group g of G takes the contiguous range
// [g*T/G, (g+1)*T/G) of it, so every work-group streams the same number of B
// bytes. With G >= strips a range is at most one strip long and touches at
// most two strips. The waves keep their private rings across the strip
// boundary: a wave whose next block belongs to the second strip parks its
// partial of the first strip in LDS and starts a new one, so the load
// pipeline never drains inside a range.
// A strip covered whole by one range is written directly. A strip split
// between ranges is finished in the same kernel: each range stores its fp32
// partial in its own slot (slot 0: its first strip, slot 1: its second) with
// device-scope stores, then counts its blocks into the strip's counter with
// a device-scope atomic; the range that completes the count adds the slots in
// ascending K order, applies ReLU and the cast, and resets the counter. No
// work-group ever waits for another.
template <class S, int W>
__global__ __launch_bounds__(W * 64) void k_skinny_sk(const KArgs a) {
    static_assert(S::WAVES == 1, "one wave per ring");
    constexpr int LOADS = S::DMA_A + S::DMA_B;
    constexpr int RING = S::STAGES * S::STAGE_BYTES;
    constexpr int TILE = S::BM * S::BN;
    static_assert(TILE * 4 <= RING, "partials fit in the rings");
    // rings, then the parked partials of the first strip ([wave][m][n] fp32)
    __shared__ __attribute__((aligned(1024))) char smem[W * RING + W * TILE * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, g = blockIdx.x;
    const int nkb = (a.K + S::BK - 1) / S::BK;  // K blocks per strip
    const int64_t T = (int64_t)a.tiles_n * nkb;
    const int64_t beg = sk_begin(g, T, G), end = sk_begin(g + 1, T, G);
    if (beg == end) return;  // (whole work-group: before any barrier)
    const StripSegments sg = strip_segments(beg, end, nkb);
    const int s0 = sg.s0;                             // first strip of the range
    const int64_t bound = sg.bound;                   // first block of the next strip
    const bool two = sg.two;                          // the range reaches a second strip
    const int len = (int)(end - beg);
    const int mine = len > wave ? (len - wave + W - 1) / W : 0;  // this wave's blocks

    LDS_PTR(char) ring = (LDS_PTR(char))smem + wave * RING;
    float *parked = (float *)(smem + W * RING);

    // Block j of this wave (block beg + wave + W j of the sequence) into stage buffer buf.
    auto issue = [&](int j, int buf) {
        const int64_t u = beg + wave + (int64_t)W * j;
        const int strip = u >= bound ? s0 + 1 : s0;
        const int k0 = (int)(u - (int64_t)strip * nkb) * S::BK;
        const int n0 = strip * S::BN;
        const int4_t ra = make_srd(a.A + k0);
        const int4_t rb = make_srd(a.B + (int64_t)k0 * a.ldb + n0);
        LDS_PTR(char) st = ring + buf * S::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < S::DMA_A; ++i) {
            const ChunkRef c = dma_a_chunk<S>(0, i, lane);
            const bool in = c.row < a.M && k0 + 8 * c.chunk < a.K;
            dma16(ra, (uint32_t)(uintptr_t)(st + i * 1024), in ? (uint32_t)(c.row * a.lda * 2 + c.chunk * 16) : kOOB);
        }
#pragma unroll
        for (int i = 0; i < S::DMA_B; ++i) {
            const ChunkRef c = dma_b_chunk<S>(0, i, lane);
            const bool in = n0 + 8 * c.chunk < a.N && k0 + c.row < a.K;
            dma16_nt(rb, (uint32_t)(uintptr_t)(st + S::A_BYTES + i * 1024),
                     in ? (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16) : kOOB);
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
    // this wave's partial tile into LDS at dst ([m][n] fp32)
    auto acc_to_lds = [&](float *dst) {
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < S::TM; ++tm) {
                const int mr = acc_m(0, tm, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nr = acc_n(0, tn, 4 * q, lane);
                    float4_t v = {acc[tn][tm][4 * q], acc[tn][tm][4 * q + 1], acc[tn][tm][4 * q + 2],
                                  acc[tn][tm][4 * q + 3]};
                    *(float4_t *)(dst + mr * S::BN + nr) = v;
                }
            }
    };

    zero_acc();
#pragma unroll
    for (int s = 0; s < S::STAGES; ++s)
        if (s < mine) issue(s, s);
    bool parked_first = false;
    int buf = 0;
    for (int j = 0; j < mine; ++j) {
        wait_blocks<LOADS, S::STAGES>(imin(S::STAGES - 1, mine - 1 - j));
        if (two && !parked_first && beg + wave + (int64_t)W * j >= bound) {
            acc_to_lds(parked + wave * TILE);  // this wave's part of the first strip is complete
            zero_acc();
            parked_first = true;
        }
        LDS_PTR(const char) st = ring + buf * S::STAGE_BYTES;
        mma_stage<S>(st, st + S::A_BYTES, 0, 0, lane, acc);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // reads of this buffer done before it is reloaded
        if (j + S::STAGES < mine) issue(j + S::STAGES, buf);
        buf = buf + 1 == S::STAGES ? 0 : buf + 1;
    }
    if (two && !parked_first) {  // no block of the second strip fell to this wave
        acc_to_lds(parked + wave * TILE);
        zero_acc();
    }

    // the last strip's partials meet in the (now idle) rings; sums in wave order
    __syncthreads();
    float *lds_part = (float *)smem;
    acc_to_lds(lds_part + wave * TILE);
    __syncthreads();
    constexpr int GROUPS = TILE / (4 * W * 64);
    static_assert(TILE % (4 * W * 64) == 0, "whole groups per thread");
    float4_t sum[2][GROUPS];  // [0]: first strip of the range, [1]: second
    auto wave_sum = [&](const float *src, float4_t(&dst)[GROUPS]) {
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) {
            const int e = 4 * (tid + r * W * 64);
            float4_t s = *(const float4_t *)(src + e);
#pragma unroll
            for (int w = 1; w < W; ++w) {
                const float4_t v = *(const float4_t *)(src + w * TILE + e);
                s[0] = s[0] + v[0];
                s[1] = s[1] + v[1];
                s[2] = s[2] + v[2];
                s[3] = s[3] + v[3];
            }
            dst[r] = s;
        }
    };
    if (two) {
        wave_sum(parked, sum[0]);
        wave_sum(lds_part, sum[1]);
    } else {
        wave_sum(lds_part, sum[0]);
    }
    auto store_groups = [&](const float4_t(&v)[GROUPS], int strip) {
        const int n0 = strip * S::BN;
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) {
            const int e = 4 * (tid + r * W * 64);
            const int m = e / S::BN, n = e % S::BN;
            if (m >= a.M || n0 + n >= a.N) continue;
            half4_t h = {relu_to_half(v[r][0]), relu_to_half(v[r][1]), relu_to_half(v[r][2]), relu_to_half(v[r][3])};
            *(half4_t *)(a.C + (int64_t)m * a.ldc + n0 + n) = h;
        }
    };

    // segments: 0 = [beg, min(end, bound)) of strip s0; 1 = [bound, end) of strip s0 + 1
    const int nseg = two ? 2 : 1;
    bool split[2];
    split[0] = !strip_part_whole(sg, beg, end, nkb, 0);
    split[1] = !strip_part_whole(sg, beg, end, nkb, 1);
    bool any_split = false;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (q >= nseg) continue;
        if (!split[q]) store_groups(sum[q], s0 + q);
        any_split = any_split || split[q];
    }
    if (!any_split) return;

    // split strips: partials to this range's slots, then counted in
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (q >= nseg || !split[q]) continue;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            a.W + ((int64_t)g * 2 + q) * TILE, (short)0, (int)kRange, 0x00020000);
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) {
            const int e = 4 * (tid + r * W * 64);
            if (e / S::BN >= a.M) continue;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4_t, sum[q][r]), rp, (uint32_t)(e * 4), 0,
                                                   kPartialScope);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
    __syncthreads();
    int *s_last = (int *)smem;  // LDS is free: the sums are in registers
    if (tid == 0) {
        for (int q = 0; q < 2; ++q) {
            s_last[q] = 0;
            if (q < nseg && split[q]) {
                const int cnt = (int)strip_part_blocks(sg, beg, end, q);
                const int old =
                    __hip_atomic_fetch_add(&a.cnt[s0 + q], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_last[q] = old + cnt == nkb;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (q >= nseg || !s_last[q]) continue;
        const int strip = s0 + q;
        const int64_t first = (int64_t)strip * nkb;
        const int g0 = sk_owner(first, T, G), g1 = sk_owner(first + nkb - 1, T, G);
        float4_t tot[GROUPS];
#pragma unroll
        for (int r = 0; r < GROUPS; ++r) tot[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int gg = g0; gg <= g1; ++gg) {  // ascending K
            const int64_t gb = sk_begin(gg, T, G);
            if (sk_begin(gg + 1, T, G) == gb) continue;  // an empty range owns nothing
            const int slot = gb >= first ? 0 : 1;
            const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                a.W + ((int64_t)gg * 2 + slot) * TILE, (short)0, (int)kRange, 0x00020000);
#pragma unroll
            for (int r = 0; r < GROUPS; ++r) {
                const int e = 4 * (tid + r * W * 64);
                float4_t v = sum[q][r];
                if (gg != g)
                    v = __builtin_bit_cast(
                        float4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(e * 4), 0, kPartialScope));
                tot[r][0] = tot[r][0] + v[0];
                tot[r][1] = tot[r][1] + v[1];
                tot[r][2] = tot[r][2] + v[2];
                tot[r][3] = tot[r][3] + v[3];
            }
        }
        store_groups(tot, strip);
        if (tid == 0) __hip_atomic_store(&a.cnt[strip], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Strip configurations: one wave per ring, W rings per work-group. Index
// 0 is the default; the others trade more bytes in flight per work-group
// (four waves, four stages) or wider strips (whole 256- or 512-byte row
// pieces of B per request, with more parts per strip) for LDS. The 64-row
// strip serves 32 < M <= 64 with one pass over B (32-row tiles would read
// each strip of B twice).
using Strip32x64 = TileShape<32, 64, 64, 1, 1, 3>;
using Strip32x64S4 = TileShape<32, 64, 64, 1, 1, 4>;
using Strip32x64S2 = TileShape<32, 64, 64, 1, 1, 2>;
using Strip32x128 = TileShape<32, 128, 64, 1, 1, 3>;
using Strip32x128S2 = TileShape<32, 128, 64, 1, 1, 2>;
using Strip32x256 = TileShape<32, 256, 32, 1, 1, 3>;
using Strip64x64 = TileShape<64, 64, 64, 1, 1, 3>;

#define TLG_STRIP_CFG(S, W, name) {S::BM, S::BN, S::BK, (W) * 64, S::STAGES, name}
const TileConfig kStripConfigs[STRIP_CONFIGS] = {
    TLG_STRIP_CFG(Strip32x64, 2, "splitk_waves_32x64x64_w2_s3"),
    TLG_STRIP_CFG(Strip32x64, 4, "splitk_waves_32x64x64_w4_s3"),
    TLG_STRIP_CFG(Strip32x64S4, 2, "splitk_waves_32x64x64_w2_s4"),
    TLG_STRIP_CFG(Strip32x128, 2, "splitk_waves_32x128x64_w2_s3"),
    TLG_STRIP_CFG(Strip32x128S2, 4, "splitk_waves_32x128x64_w4_s2"),
    TLG_STRIP_CFG(Strip32x256, 2, "splitk_waves_32x256x32_w2_s3"),
    TLG_STRIP_CFG(Strip64x64, 2, "splitk_waves_64x64x64_w2_s3"),
};
#undef TLG_STRIP_CFG
const TileConfig &kStripConfig = kStripConfigs[0];

template <class S, int W>
static hipError_t launch_strip_t(const Problem &p, int parts, float *partials, int *counters, hipStream_t stream) {
    static_assert(S::BN * S::BK * 2 == S::DMA_B * 1024, "strip blocks are whole loads");
    static_assert(W * S::STAGES * S::STAGE_BYTES <= 160 * 1024, "rings fit the LDS");
    KArgs a;
    a.A = (const _Float16 *)p.A;
    a.B = (const _Float16 *)p.B;
    a.C = (_Float16 *)p.C;
    a.W = partials;
    a.cnt = counters;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.tiles_m = 1;
    a.tiles_n = (int)((p.N + S::BN - 1) / S::BN);
    a.group_m = 1;
    a.k_split = parts;
    a.kmain = (int)p.K;
    if (p.trans_b)
        hipLaunchKernelGGL((k_skinny_strip<S, W, true>), dim3((unsigned)(a.tiles_n * parts)), dim3(W * 64), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((k_skinny_strip<S, W>), dim3((unsigned)(a.tiles_n * parts)), dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

template <class S, int W>
static hipError_t launch_strip_sk_t(const Problem &p, int grid, float *partials, int *counters, hipStream_t stream) {
    static_assert(W * S::STAGES * S::STAGE_BYTES + W * S::BM * S::BN * 4 <= 160 * 1024, "rings fit the LDS");
    KArgs a;
    a.A = (const _Float16 *)p.A;
    a.B = (const _Float16 *)p.B;
    a.C = (_Float16 *)p.C;
    a.W = partials;
    a.cnt = counters;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.tiles_m = 1;
    a.tiles_n = (int)((p.N + S::BN - 1) / S::BN);
    a.group_m = 1;
    a.k_split = 1;
    a.kmain = (int)p.K;
    hipLaunchKernelGGL((k_skinny_sk<S, W>), dim3((unsigned)grid), dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

const TileConfig kStripSkConfigs[STRIP_SK_CONFIGS] = {
    {Strip32x64::BM, Strip32x64::BN, Strip32x64::BK, 2 * 64, Strip32x64::STAGES, "strip_sk_32x64x64_w2_s3"},
    {Strip32x64S2::BM, Strip32x64S2::BN, Strip32x64S2::BK, 2 * 64, Strip32x64S2::STAGES, "strip_sk_32x64x64_w2_s2"},
};

hipError_t launch_skinny_strip_sk(int config, const Problem &p, int grid, float *partials, int *counters,
                                  hipStream_t stream) {
    switch (config) {
        case 0: return launch_strip_sk_t<Strip32x64, 2>(p, grid, partials, counters, stream);
        case 1: return launch_strip_sk_t<Strip32x64S2, 2>(p, grid, partials, counters, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_skinny_strip(int config, const Problem &p, int parts, float *partials, int *counters,
                               hipStream_t stream) {
    switch (config) {
        case 0: return launch_strip_t<Strip32x64, 2>(p, parts, partials, counters, stream);
        case 1: return launch_strip_t<Strip32x64, 4>(p, parts, partials, counters, stream);
        case 2: return launch_strip_t<Strip32x64S4, 2>(p, parts, partials, counters, stream);
        case 3: return launch_strip_t<Strip32x128, 2>(p, parts, partials, counters, stream);
        case 4: return launch_strip_t<Strip32x128S2, 4>(p, parts, partials, counters, stream);
        case 5: return launch_strip_t<Strip32x256, 2>(p, parts, partials, counters, stream);
        case 6: return launch_strip_t<Strip64x64, 2>(p, parts, partials, counters, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tlg
