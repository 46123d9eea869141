// gfx950 wave-role ("ping-pong") schedule for C = ReLU(A . B), fp16 in,
// fp32 accumulation, fp16 out: the quick-start kernel of the TileLang
// article (aiwiki.ai/wiki/tilelang, "Programming model"), with the
// producer/consumer wave specialisation that the article's "Compiler and
// scheduling automation" section describes TileLang doing automatically
// (and that the forum post "TileLang: Writing Near-Hardware-Limit GPU
// Kernels in 70 Lines of Python", "Key Technical Milestones", lists), re-cut
// for CDNA4.
//
// A 256 x 256 output tile, eight waves, two per SIMD: waves 0-3 (group 0,
// rows 0..127 of the tile) and waves 4-7 (group 1, rows 128..255), one of
// each on every SIMD. The K loop is a sequence of slots separated by
// work-group barriers; in every slot one group is the "memory" group and the
// other the "math" group, and they swap each slot:
//
//   slot      2u               2u+1
//   group 0   read stage u     MFMAs of stage u
//   group 1   MFMAs of u-1     read stage u
//
// "read stage u" issues the wave's share of the direct-to-LDS loads of stage
// u+STAGES-1, reads all of the wave's operand fragments of stage u into
// registers, and waits for the wave's loads of stage u+1; "MFMAs" runs the
// stage's 16 MFMAs of the wave back to back from those registers, at raised
// wave priority. So on each SIMD one wave keeps the matrix core busy while
// the other moves data, and the two swap roles every slot; the barrier at
// the end of each slot publishes the loads and fragment reads it depends on.
// (Group 1 spends the first slot idle and group 0 the last, so both pass the
// same number of barriers.)
//
// Buffer reuse: stage u's buffer is last read by group 1 in slot 2u+1; the
// loads of stage u+STAGES go out in slots 2u+2 (group 0) and 2u+3 (group 1),
// after that slot's barrier. Loads of stage v complete before the barrier
// that ends slot 2v-1, which precedes every read of stage v.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

template <class S, bool BT>
__global__ __launch_bounds__(S::NT) void k_pingpong(const KArgs a) {
    static_assert(S::WAVES == 8 && S::WM == 2, "two groups of four waves, one row half each");
    static_assert(S::KSTEPS == 2, "a stage is one 32-deep slot of MFMAs");
    static_assert(!BT || S::BM == S::BN, "transposed B is held like A");
    __shared__ __attribute__((aligned(1024))) char smem[S::LDS_BYTES];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const int nwg = a.tiles_m * a.tiles_n;
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, nwg), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    const int m0 = tm_idx * S::BM, n0 = tn_idx * S::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave / S::WN;
    const int wm0 = group * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int kend = a.kmain;
    const int nk = (kend + S::BK - 1) / S::BK;

    uint32_t a_off[S::DMA_A], b_off[S::DMA_B];
    int a_col[S::DMA_A], b_k[S::DMA_B];
    bool a_ok[S::DMA_A], b_ok[S::DMA_B];
#pragma unroll
    for (int i = 0; i < S::DMA_A; ++i) {
        const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        a_off[i] = (uint32_t)(c.row * a.lda * 2 + c.chunk * 16);
        a_col[i] = 8 * c.chunk;
        a_ok[i] = m0 + c.row < a.M;
    }
#pragma unroll
    for (int i = 0; i < S::DMA_B; ++i) {
        if (BT) {
            const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
            b_off[i] = (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16);
            b_k[i] = 8 * c.chunk;
            b_ok[i] = n0 + c.row < a.N;
        } else {
            const ChunkRef c = dma_b_chunk<S>(wave, i, lane);
            b_off[i] = (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16);
            b_k[i] = c.row;
            b_ok[i] = n0 + 8 * c.chunk < a.N;
        }
    }
    auto issue = [&](int kt) {
        const int k0 = kt * S::BK;
        LDS_PTR(char) sA = lds + (kt % S::STAGES) * S::STAGE_BYTES;
        LDS_PTR(char) sB = sA + S::A_BYTES;
        const int4_t ra = make_srd(a.A + (int64_t)m0 * a.lda + k0);
        const int4_t rb = make_srd(BT ? a.B + (int64_t)n0 * a.ldb + k0 : a.B + (int64_t)k0 * a.ldb + n0);
        const uint32_t la = (uint32_t)(uintptr_t)(sA + wave * S::DMA_A * 1024);
        const uint32_t lb = (uint32_t)(uintptr_t)(sB + wave * S::DMA_B * 1024);
#pragma unroll
        for (int i = 0; i < S::DMA_A; ++i) dma16(ra, la + i * 1024, (a_ok[i] && k0 + a_col[i] < kend) ? a_off[i] : kOOB);
#pragma unroll
        for (int i = 0; i < S::DMA_B; ++i) dma16(rb, lb + i * 1024, (b_ok[i] && k0 + b_k[i] < kend) ? b_off[i] : kOOB);
    };
    constexpr int kLoads = S::DMA_A + S::DMA_B;

    float16_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    half8_t af[S::KSTEPS][S::TM], bf[S::KSTEPS][S::TN];

    // prologue: stages 0 .. STAGES-2 in flight, stage 0 landed everywhere
#pragma unroll
    for (int s = 0; s < S::STAGES - 1; ++s)
        if (s < nk) issue(s);
    if (nk >= S::STAGES - 1)
        wait_vmcnt<(S::STAGES - 2) * kLoads>();
    else
        wait_vmcnt<0>();
    barrier_lds();
    if (group == 1) barrier_lds();  // group 1 starts one slot behind

    for (int u = 0; u < nk; ++u) {
        // ---- memory slot: loads of stage u+STAGES-1, fragments of stage u
        __builtin_amdgcn_sched_barrier(0);
        if (u + S::STAGES - 1 < nk) issue(u + S::STAGES - 1);
        {
            LDS_PTR(const char) sA = lds + (u % S::STAGES) * S::STAGE_BYTES;
            LDS_PTR(const char) sB = sA + S::A_BYTES;
#pragma unroll
            for (int s = 0; s < S::KSTEPS; ++s) {
#pragma unroll
                for (int tn = 0; tn < S::TN; ++tn)
                    bf[s][tn] = BT ? *(LDS_PTR(const half8_t))(sB + frag_a_offset<S>(wn0, tn, s, lane))
                                   : read_b_frag(sB, frag_b_offset<S>(wn0, tn, s, 0, lane),
                                                 frag_b_offset<S>(wn0, tn, s, 1, lane));
#pragma unroll
                for (int tm = 0; tm < S::TM; ++tm)
                    af[s][tm] = *(LDS_PTR(const half8_t))(sA + frag_a_offset<S>(wm0, tm, s, lane));
            }
        }
        // this wave's loads of stage u+1 have landed (later stages may still fly)
        if (u + S::STAGES - 1 < nk)
            wait_vmcnt<(S::STAGES - 2) * kLoads>();
        else
            wait_vmcnt<0>();
        barrier_lds();
        __builtin_amdgcn_sched_barrier(0);
        // ---- math slot: the stage's MFMAs from registers
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < S::KSTEPS; ++s)
#pragma unroll
            for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < S::TM; ++tm)
                    acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[s][tn], af[s][tm], acc[tn][tm], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        barrier_lds();
    }
    if (group == 0) barrier_lds();  // group 0 ends one slot ahead

    // rows kmain .. K-1 (ragged K or N): one zero-padded block staged element
    // by element into buffer 0, every wave done with the stages
    if (a.kmain < a.K) {
        stage_tail<S, BT>(a, m0, n0, lds, lds + S::A_BYTES, tid);
        barrier_lds();
        mma_kstep<S, BT>(lds, lds + S::A_BYTES, 0, wm0, wn0, lane, acc);
        barrier_lds();
    }
    store_c_tile_lds<S>(a, m0, n0, wave, lane, acc, lds);
}

using PingPong256x32 = TileShape<256, 256, 32, 2, 4, 4>;  // four 32 KiB stages (128 KiB)

const TileConfig kPingPongConfigs[PINGPONG_CONFIGS] = {
    {256, 256, 32, PingPong256x32::NT, PingPong256x32::STAGES, "pingpong_256x256x32_w2x4_s4"},
};

template <class S, bool BT>
static hipError_t launch_pp_t(const Problem &p, hipStream_t stream) {
    KArgs a;
    a.A = (const _Float16 *)p.A;
    a.B = (const _Float16 *)p.B;
    a.C = (_Float16 *)p.C;
    a.W = nullptr;
    a.cnt = nullptr;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.lda = p.lda;
    a.ldb = p.ldb;
    a.ldc = p.ldc;
    a.group_m = 4;
    a.k_split = (int)p.K;
    // loads stop at the last multiple of 8 below K when a 16-byte chunk
    // could cross the end of a row (K % 8; N % 8 too for an N-contiguous B)
    const bool whole = p.K % 8 == 0 && (BT || p.N % 8 == 0);
    a.kmain = whole ? (int)p.K : (int)(8 * ((p.K - 1) / 8));
    a.tiles_m = (a.M + S::BM - 1) / S::BM;
    a.tiles_n = (a.N + S::BN - 1) / S::BN;
    hipLaunchKernelGGL((k_pingpong<S, BT>), dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(S::NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_pingpong(int config, const Problem &p, hipStream_t stream) {
    if (config != PINGPONG_256x256x32) return hipErrorInvalidValue;
    return p.trans_b ? launch_pp_t<PingPong256x32, true>(p, stream) : launch_pp_t<PingPong256x32, false>(p, stream);
}

}  // namespace tlg
