// Software-pipelined gfx950 kernel for C = ReLU(A . B) on large, aligned
// problems: the quick-start kernel of the TileLang article
// (aiwiki.ai/wiki/tilelang, "Programming model") with its T.Pipelined K loop
// scheduled by hand for one 64-wide wave per SIMD.
//
// Data movement and layouts are those of k_tiled_dma (direct global->LDS
// loads, XOR-swizzled LDS stages, ds_read_b64_tr_b16 for the N-contiguous B
// operand, v_mfma_f32_32x32x16_f16 with fp32 accumulators). What changes is
// the order of work inside one K step of a wave. The MFMA pipe of a SIMD has
// no other wave to switch to, so every instruction that is not an MFMA is
// slotted between MFMAs, where it costs no matrix-core time: the LDS reads of
// the next k-step's operand fragments, one or two after each MFMA, and the
// direct-to-LDS loads of the stage three steps ahead, one every two to four
// MFMAs (so the load unit is never flooded). One barrier per K step publishes
// the next stage; the loop is arranged so that nothing is pending in LDS at
// that point and the first MFMAs after it still have operands in registers.
//
// The stream of loads is uniform: stages past the end of K are issued with
// every lane out of range, which writes zeros into a buffer no wave reads.
// So every step waits for the same load count and the loop has no branch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

// Operand fragments of one k-step: TM A fragments (second MFMA operand, one
// ds_read_b128 each) and TN B fragments (first operand, two transposing
// 8-byte reads each).
template <class S>
struct Frags {
    half8_t a[S::TM];
    short4_t blo[S::TN], bhi[S::TN];
};

// LDS reads of one k-step's fragments, numbered in the order the MFMAs use
// them (tile i uses b[i / TM] and a[i % TM]): b[0] (two reads), a[0..TM-1],
// then b[1..TN-1] (two reads each). BT (B given transposed, its tile held
// like A's): one 16-byte read per B fragment, b[0], a[0..TM-1], b[1..TN-1].
template <class S, bool BT = false>
constexpr int kFragReads = S::TM + (BT ? 1 : 2) * S::TN;

template <class S, bool BT>
__device__ __forceinline__ void frag_read(Frags<S> &f, LDS_PTR(const char) sA, LDS_PTR(const char) sB,
                                          int wm0, int wn0, int s, int lane, int r) {
    if (BT) {
        if (r >= 1 && r < 1 + S::TM) {
            f.a[r - 1] = *(LDS_PTR(const half8_t))(sA + frag_a_offset<S>(wm0, r - 1, s, lane));
        } else {
            const int tn = r == 0 ? 0 : r - S::TM;
            const short8_t v = *(LDS_PTR(const short8_t))(sB + frag_a_offset<S>(wn0, tn, s, lane));
            f.blo[tn] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
            f.bhi[tn] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
        }
        return;
    }
    if (r < 2) {
        LDS_PTR(short4_t) p = (LDS_PTR(short4_t))(sB + frag_b_offset<S>(wn0, 0, s, r, lane));
        if (r == 0)
            f.blo[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
        else
            f.bhi[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    } else if (r < 2 + S::TM) {
        const int tm = r - 2;
        f.a[tm] = *(LDS_PTR(const half8_t))(sA + frag_a_offset<S>(wm0, tm, s, lane));
    } else {
        const int tn = 1 + (r - 2 - S::TM) / 2, h = (r - 2 - S::TM) % 2;
        LDS_PTR(short4_t) p = (LDS_PTR(short4_t))(sB + frag_b_offset<S>(wn0, tn, s, h, lane));
        if (h == 0)
            f.blo[tn] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
        else
            f.bhi[tn] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    }
}

template <class S>
__device__ __forceinline__ void mfma_tile(const Frags<S> &f, int i, float16_t (&acc)[S::TN][S::TM]) {
    const int tn = i / S::TM, tm = i % S::TM;
    const half8_t b = __builtin_bit_cast(half8_t, __builtin_shufflevector(f.blo[tn], f.bhi[tn], 0, 1, 2, 3, 4, 5,
                                                                           6, 7));
    acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, f.a[tm], acc[tn][tm], 0, 0, 0);
}

// Nothing may be scheduled across this point (keeps the hand-written order).
#define TLG_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// One K step of the loop is a fixed sequence of KSTEPS*T MFMA slots, T =
// TM*TN the wave's MFMA tiles (16 for four waves of 128 x 128, 8 for eight
// waves of 128 x 64), H = T/2:
//   slots 0..H-1      MFMAs H..T-1 of the previous stage's last k-step (held
//                     in f[1]); after them the LDS reads of this stage's
//                     k-step-0 fragments into f[0], two per slot;
//   next T per ks     k-steps 0..KSTEPS-2: T MFMAs on f[ks & 1], with the
//                     reads of k-step ks+1 into f[(ks+1) & 1], one per slot;
//   last H slots      MFMAs 0..H-1 of the last k-step (f[1]).
// With eight waves two share each SIMD and the hardware interleaves their
// slots, which covers one wave's waits with the other's MFMAs.
// The LOADS direct-to-LDS loads go after slots DOFF, DOFF+SPACING, ...: the
// B tile of stage kt+STAGES-1 and the A tile of stage kt+ASTAGES-1 (A may
// have one LDS buffer more than B, which gives its loads a step more to
// arrive; they are then issued after the B loads). Then this wave's loads of
// stage kt+1 are waited for and the barrier publishes it (and retires stage
// kt). The C tile leaves through LDS (store_c_tile_lds).
// EARLY (the default eight-wave form): the wait and the barrier come before
// the last H slots instead of after them. Those slots read no LDS of stage
// kt (the last k-step's fragments were read during the k-step before), so
// the barrier can already publish stage kt+1 there, and the reads of its
// k-step-0 fragments into f[0] move from the next stage's first H slots into
// these, half a k-step earlier than they are needed.
template <class S, int ASTAGES>
constexpr int pipe_lds_bytes() {
    return ASTAGES * S::A_BYTES + S::STAGES * S::B_BYTES;  // A buffers first, then the B buffers
}

// One output tile (tm_idx, tn_idx) of problem a, with the work-group's LDS.
// Whether a load reads memory is decided per stage, on the scalar unit, by
// the buffer descriptor's range (0 bytes past the end of K); each lane's
// offset is fixed for the whole loop. This keeps a chain of vector compares
// and selects out of the slot program, where with one wave per SIMD it would
// hold up the next MFMA's issue. FULLK: kmain is a multiple of BK, every
// stage wholly inside K or wholly past it; else the last stage inside K takes
// a second set of offsets, fixed too, that also drop what lies past kmain.
template <class S, int SPACING, int DOFF, int ASTAGES, bool BT, bool EARLY, bool FULLK>
__device__ __forceinline__ void pipe_tile(const KArgs &a, int tm_idx, int tn_idx, LDS_PTR(char) lds) {
    constexpr int T = S::TM * S::TN;  // MFMA tiles of a wave (MFMAs per k-step)
    constexpr int H = T / 2;
    static_assert(T % 2 == 0 && S::KSTEPS % 2 == 0, "the last k-step of a stage must use f[1]");
    constexpr int READS = kFragReads<S, BT>;
    static_assert(READS <= T && READS <= 2 * H, "fragment reads must fit under the MFMAs of a k-step");
    static_assert(!BT || S::BM == S::BN, "transposed B is held in the A layout");
    constexpr int LOADS = S::DMA_A + S::DMA_B;  // direct-to-LDS loads per wave per stage
    constexpr int AHEAD = S::STAGES - 1;        // B stages in flight beyond the one being multiplied
    constexpr int AHEAD_A = ASTAGES - 1;        // A stages likewise
    static_assert(ASTAGES >= S::STAGES - 1 && ASTAGES <= S::STAGES + 1, "A and B differ by at most one buffer");
    // Within a step the loads of the operand loaded fewer stages ahead go
    // first, so the loads still allowed in flight at the step's wait are
    // exactly the latest ones (the WAIT count below).
    constexpr bool B_FIRST = ASTAGES > S::STAGES;  // B loads of a step before its A loads
    // loads issued after the last one of the next stage: those of later stages
    constexpr int WAIT = (AHEAD_A - 1) * S::DMA_A + (AHEAD - 1) * S::DMA_B;
    constexpr int SLOTS = S::KSTEPS * T;
    static_assert(AHEAD >= 1 && AHEAD_A >= 1 && WAIT < 64, "vmcnt range");
    static_assert(DOFF + (LOADS - 1) * SPACING < SLOTS, "loads must fit in one K step");
    constexpr int B_REGION = ASTAGES * S::A_BYTES;  // A buffers first, then the B buffers
    static_assert(pipe_lds_bytes<S, ASTAGES>() <= 160 * 1024, "LDS of one work-group");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int m0 = tm_idx * S::BM, n0 = tn_idx * S::BN;
    const int nk = (a.kmain + S::BK - 1) / S::BK;

    // Per-lane load descriptors (constant over the K loop): byte offset in the
    // stage's window, the column (A) or row (B) inside the stage that decides
    // whether the chunk is inside K, and whether the row/column is inside M/N.
    uint32_t off[LOADS];
    int kin[LOADS];
    bool ok[LOADS];
#pragma unroll
    for (int i = 0; i < S::DMA_A; ++i) {
        ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        off[i] = (uint32_t)(c.row * a.lda * 2 + c.chunk * 16);
        kin[i] = 8 * c.chunk;
        ok[i] = m0 + c.row < a.M;
    }
#pragma unroll
    for (int i = 0; i < S::DMA_B; ++i) {
        ChunkRef c = BT ? dma_a_chunk<S>(wave, i, lane) : dma_b_chunk<S>(wave, i, lane);
        off[S::DMA_A + i] = (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16);
        kin[S::DMA_A + i] = BT ? 8 * c.chunk : c.row;          // transposed B: rows n, chunks along K
        ok[S::DMA_A + i] = BT ? n0 + c.row < a.N : n0 + 8 * c.chunk < a.N;
    }

    const _Float16 *a_tile = a.A + (int64_t)m0 * a.lda;
    const _Float16 *b_tile = BT ? a.B + (int64_t)n0 * a.ldb : a.B + n0;
    uint32_t voff[LOADS];  // the offset, or kOOB for a row or column outside M or N
#pragma unroll
    for (int i = 0; i < LOADS; ++i) voff[i] = ok[i] ? off[i] : kOOB;
    // (!FULLK) the last stage, nk - 1, ends inside K: its offsets also drop
    // the chunks at or past kmain. Every earlier stage lies wholly inside K,
    // so one select per load, on a scalar condition, is all the slot program
    // carries for a ragged K (against a compare chain per load in every
    // stage: 3008 x 2049 x 1536 29.5 vs 31.3 us, 4096 x 4100 x 4096 187.4 vs
    // 192.3 us).
    uint32_t vlast[FULLK ? 1 : LOADS];
    if (!FULLK) {
        const int klast = (nk - 1) * S::BK;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) vlast[i] = ok[i] && klast + kin[i] < a.kmain ? off[i] : kOOB;
    }

    // Load j of stage kt into LDS buffer buf of its operand (stages past K
    // load zeros); j < DMA_A loads A, the others B.
    auto dma = [&](int j, int kt, int buf) {
        const int k0 = kt * S::BK;
        int4_t r = j < S::DMA_A ? make_srd(a_tile + k0) : make_srd(BT ? b_tile + k0 : b_tile + (int64_t)k0 * a.ldb);
        if (kt >= nk) r[2] = 0;  // past the end of K: every lane out of range, zeros
        const uint32_t l = j < S::DMA_A ? (uint32_t)(uintptr_t)(lds + buf * S::A_BYTES + (wave * S::DMA_A + j) * 1024)
                                        : (uint32_t)(uintptr_t)(lds + B_REGION + buf * S::B_BYTES +
                                                                (wave * S::DMA_B + (j - S::DMA_A)) * 1024);
        if (FULLK)
            dma16(r, l, voff[j]);
        else
            dma16(r, l, kt == nk - 1 ? vlast[FULLK ? 0 : j] : voff[j]);
    };

    float16_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // f[1] starts at zero: the first step's slots 0..7 add 0 * 0.
    Frags<S> f[2];
#pragma unroll
    for (int t = 0; t < S::TN; ++t) {
        f[1].blo[t] = short4_t{0, 0, 0, 0};
        f[1].bhi[t] = short4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < S::TM; ++t) f[1].a[t] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};

#pragma unroll
    for (int s = 0; s < (AHEAD_A > AHEAD ? AHEAD_A : AHEAD); ++s) {
        if (s < AHEAD_A)
#pragma unroll
            for (int j = 0; j < S::DMA_A; ++j) dma(j, s, s);
        if (s < AHEAD)
#pragma unroll
            for (int j = S::DMA_A; j < LOADS; ++j) dma(j, s, s);
    }
    wait_vmcnt<WAIT>();
    barrier_lds();
    if (EARLY) {
#pragma unroll
        for (int r = 0; r < READS; ++r) frag_read<S, BT>(f[0], lds, lds + B_REGION, wm0, wn0, 0, lane, r);
    }

    int bbuf = 0, abuf = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt+AHEAD of B (kt+AHEAD_A of A) goes where stage kt-1 was
        const int nbbuf = bbuf == 0 ? S::STAGES - 1 : bbuf - 1;
        const int nabuf = abuf == 0 ? ASTAGES - 1 : abuf - 1;
        LDS_PTR(const char) sA = lds + abuf * S::A_BYTES;
        LDS_PTR(const char) sB = lds + B_REGION + bbuf * S::B_BYTES;
        // (EARLY) stage kt+1's buffers
        LDS_PTR(const char) sA1 = lds + (abuf == ASTAGES - 1 ? 0 : abuf + 1) * S::A_BYTES;
        LDS_PTR(const char) sB1 = lds + B_REGION + (bbuf == S::STAGES - 1 ? 0 : bbuf + 1) * S::B_BYTES;
        TLG_SCHED_FENCE();
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) {
            if (q < H) {
                mfma_tile<S>(f[1], H + q, acc);
                if (!EARLY) {
#pragma unroll
                    for (int r = 2 * q; r < 2 * q + 2; ++r)
                        if (r < READS) frag_read<S, BT>(f[0], sA, sB, wm0, wn0, 0, lane, r);
                }
            } else if (q < H + (S::KSTEPS - 1) * T) {
                const int ks = (q - H) / T, i = (q - H) % T;
                mfma_tile<S>(f[ks & 1], i, acc);
                if (i < READS) frag_read<S, BT>(f[(ks + 1) & 1], sA, sB, wm0, wn0, ks + 1, lane, i);
            } else {
                const int u = q - H - (S::KSTEPS - 1) * T;
                if (EARLY && u == 0) {
                    wait_vmcnt<WAIT>();  // this wave's loads of stage kt+1 are in LDS
                    barrier_lds();       // ... and every wave's; no wave reads stage kt any more
                }
                mfma_tile<S>(f[1], u, acc);
                if (EARLY) {
#pragma unroll
                    for (int r = 2 * u; r < 2 * u + 2; ++r)
                        if (r < READS) frag_read<S, BT>(f[0], sA1, sB1, wm0, wn0, 0, lane, r);
                }
            }
            if (q >= DOFF && (q - DOFF) % SPACING == 0 && (q - DOFF) / SPACING < LOADS) {
                const int n = (q - DOFF) / SPACING;
                const int j = !B_FIRST ? n : n < S::DMA_B ? S::DMA_A + n : n - S::DMA_B;
                if (j < S::DMA_A)
                    dma(j, kt + AHEAD_A, nabuf);
                else
                    dma(j, kt + AHEAD, nbbuf);
            }
            TLG_SCHED_FENCE();
        }
        if (!EARLY) {
            wait_vmcnt<WAIT>();  // this wave's loads of stage kt+1 are in LDS
            barrier_lds();       // ... and every wave's; stage kt is no longer read
        }
        bbuf = bbuf == S::STAGES - 1 ? 0 : bbuf + 1;
        abuf = abuf == ASTAGES - 1 ? 0 : abuf + 1;
    }
#pragma unroll
    for (int i = H; i < T; ++i) mfma_tile<S>(f[1], i, acc);
    // No load may still be writing LDS when the work-group ends.
    wait_vmcnt<0>();

    // Rows kmain .. K-1 (ragged K or N): one zero-padded block staged element
    // by element into buffer 0 once every wave is done with the stages.
    if (a.kmain < a.K) {
        barrier_lds();
        stage_tail<S, BT>(a, m0, n0, lds, lds + B_REGION, tid);
        barrier_lds();
        mma_kstep<S, BT>(lds, lds + B_REGION, 0, wm0, wn0, lane, acc);
    }

    barrier_lds();  // every wave is done with the stages (and the tail block)
    store_c_tile_lds<S>(a, m0, n0, wave, lane, acc, lds);
}

template <class S, int SPACING, int DOFF, int ASTAGES, bool BT, bool EARLY, bool FULLK>
__global__ __launch_bounds__(S::NT) void k_tiled_pipe(const KArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[pipe_lds_bytes<S, ASTAGES>()];
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    pipe_tile<S, SPACING, DOFF, ASTAGES, BT, EARLY, FULLK>(a, tm_idx, tn_idx, (LDS_PTR(char))smem);
}

// Grouped problems in one launch: after the XCD renumbering, work-group ids
// tile_start[p] .. tile_start[p+1]-1 take problem p's tiles in its grouped
// order (the table travels as the kernel argument).
template <class S, int SPACING, int DOFF, int ASTAGES, bool BT, bool EARLY, bool FULLK>
__global__ __launch_bounds__(S::NT) void k_tiled_pipe_grouped(const GroupArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem[pipe_lds_bytes<S, ASTAGES>()];
    const int v = xcd_remap(blockIdx.x, g.tile_start[g.count]);
    int p = 0;
    while (p + 1 < g.count && v >= g.tile_start[p + 1]) ++p;
    const KArgs &a = g.p[p];
    int tm_idx, tn_idx;
    grouped_tile(v - g.tile_start[p], a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    pipe_tile<S, SPACING, DOFF, ASTAGES, BT, EARLY, FULLK>(a, tm_idx, tn_idx, (LDS_PTR(char))smem);
}

using Pipe256x32 = TileShape<256, 256, 32, 2, 2, 4>;
using Pipe256x64 = TileShape<256, 256, 64, 2, 2, 2>;
using Pipe256x64w8 = TileShape<256, 256, 64, 2, 4, 2>;  // eight waves, two per SIMD
// three B buffers beside two A buffers (B, whose lines are shared by fewer
// work-groups of an XCD, is loaded two steps ahead)
using Pipe256x64B3 = TileShape<256, 256, 64, 2, 2, 3>;
using Pipe256x64w8B3 = TileShape<256, 256, 64, 2, 4, 3>;
// half tiles (four waves of 128 x 64, three stages): twice the tiles of
// 256 x 256 for problems that leave CUs idle at that size
using Pipe256x128 = TileShape<256, 128, 64, 2, 2, 3>;
using Pipe128x256 = TileShape<128, 256, 64, 1, 4, 3>;

const TileConfig kPipeConfigs[PIPE_CONFIGS] = {
    {Pipe256x32::BM, Pipe256x32::BN, Pipe256x32::BK, Pipe256x32::NT, Pipe256x32::STAGES, "pipe_256x256x32_w2x2_s4"},
    {Pipe256x64::BM, Pipe256x64::BN, Pipe256x64::BK, Pipe256x64::NT, Pipe256x64::STAGES, "pipe_256x256x64_w2x2_s2"},
    {Pipe256x64::BM, Pipe256x64::BN, Pipe256x64::BK, Pipe256x64::NT, Pipe256x64::STAGES, "pipe_256x256x64_w2x2_s2_a3"},
    {Pipe256x64w8::BM, Pipe256x64w8::BN, Pipe256x64w8::BK, Pipe256x64w8::NT, Pipe256x64w8::STAGES,
     "pipe_256x256x64_w2x4_s2"},
    {Pipe256x64w8::BM, Pipe256x64w8::BN, Pipe256x64w8::BK, Pipe256x64w8::NT, Pipe256x64w8::STAGES,
     "pipe_256x256x64_w2x4_s2_a3"},
    {Pipe256x128::BM, Pipe256x128::BN, Pipe256x128::BK, Pipe256x128::NT, Pipe256x128::STAGES,
     "pipe_256x128x64_w2x2_s3"},
    {Pipe128x256::BM, Pipe128x256::BN, Pipe128x256::BK, Pipe128x256::NT, Pipe128x256::STAGES,
     "pipe_128x256x64_w1x4_s3"},
    {Pipe256x64w8::BM, Pipe256x64w8::BN, Pipe256x64w8::BK, Pipe256x64w8::NT, Pipe256x64w8::STAGES,
     "pipe_256x256x64_w2x4_s2_a3_early"},
    {Pipe256x64w8B3::BM, Pipe256x64w8B3::BN, Pipe256x64w8B3::BK, Pipe256x64w8B3::NT, Pipe256x64w8B3::STAGES,
     "pipe_256x256x64_w2x4_s3_a2_early"},
    {Pipe256x64B3::BM, Pipe256x64B3::BN, Pipe256x64B3::BK, Pipe256x64B3::NT, Pipe256x64B3::STAGES,
     "pipe_256x256x64_w2x2_s3_a2"},
    // 16 x 16 x 32 MFMA tiles, four waves (gemm_relu_pipe16_gfx950.hip)
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_early"},
    {256, 256, 64, 256, 3, "pipe16_256x256x64_w2x2_s3_a2"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_sp2"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_sp6"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_early_sp2"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_sp7"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_sp8"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_sp6_d5"},
    {256, 256, 64, 256, 3, "pipe16_256x256x64_w2x2_s3_a2_sp6"},
    {256, 256, 64, 256, 2, "pipe16_256x256x64_w2x2_s2_a3_early_sp6"},
    {128, 256, 64, 256, 3, "pipe16_128x256x64_w1x4_s3_a3"},
    {128, 256, 64, 256, 3, "pipe16_128x256x64_w1x4_s3_a4"},
    {256, 256, 64, 512, 2, "pipe16_256x256x64_w2x4_s2_a3_sp8"},
    {256, 256, 64, 512, 2, "pipe16_256x256x64_w2x4_s2_a3_sp4"},
    {256, 256, 64, 512, 2, "pipe16_256x256x64_w2x4_s2_a3_early_sp6"},
    {192, 256, 64, 256, 2, "pipe16_192x256x64_w2x2_s2_a3_sp6"},
    {192, 256, 64, 256, 2, "pipe16_192x256x64_w2x2_s2_a3_sp7"},
};

template <class S, bool BT>
static KArgs pipe_args(const Problem &p) {
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
    // loads stop at the last multiple of 8 below K when a 16-byte chunk
    // could cross the end of a row (K % 8; N % 8 too for an N-contiguous B)
    const bool whole = p.K % 8 == 0 && (BT || p.N % 8 == 0);
    a.kmain = whole ? (int)p.K : (int)(8 * ((p.K - 1) / 8));
    a.tiles_m = (a.M + S::BM - 1) / S::BM;
    a.tiles_n = (a.N + S::BN - 1) / S::BN;
    return a;
}

template <class S, int SPACING, int DOFF, int ASTAGES, bool BT = false, bool EARLY = false>
static hipError_t launch_pipe_t(const Problem &p, hipStream_t stream) {
    const KArgs a = pipe_args<S, BT>(p);
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
    if (a.kmain % S::BK == 0)
        hipLaunchKernelGGL((k_tiled_pipe<S, SPACING, DOFF, ASTAGES, BT, EARLY, true>), grid, dim3(S::NT), 0, stream, a);
    else
        hipLaunchKernelGGL((k_tiled_pipe<S, SPACING, DOFF, ASTAGES, BT, EARLY, false>), grid, dim3(S::NT), 0, stream,
                           a);
    return hipGetLastError();
}

template <bool BT>
static hipError_t launch_pipe_grouped_t(const Problem *ps, int count, hipStream_t stream) {
    using S = Pipe256x64w8;
    GroupArgs g;
    g.count = count;
    g.tile_start[0] = 0;
    for (int i = 0; i < count; ++i) {
        g.p[i] = pipe_args<S, BT>(ps[i]);
        g.tile_start[i + 1] = g.tile_start[i] + g.p[i].tiles_m * g.p[i].tiles_n;
    }
    if (g.tile_start[count] == 0) return hipSuccess;
    bool fullk = true;
    for (int i = 0; i < count; ++i) fullk = fullk && g.p[i].kmain % S::BK == 0;
    const dim3 grid((unsigned)g.tile_start[count]);
    if (fullk)
        hipLaunchKernelGGL((k_tiled_pipe_grouped<S, 2, 1, 3, BT, true, true>), grid, dim3(S::NT), 0, stream, g);
    else
        hipLaunchKernelGGL((k_tiled_pipe_grouped<S, 2, 1, 3, BT, true, false>), grid, dim3(S::NT), 0, stream, g);
    return hipGetLastError();
}

// The eight-wave early-barrier configuration over up to kGroupMax problems
// (all with the same trans_b).
hipError_t launch_tiled_pipe_grouped(const Problem *ps, int count, hipStream_t stream) {
    static_assert(sizeof(GroupArgs) <= 4096, "kernel arguments");
    if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
    const bool bt = ps[0].trans_b;
    for (int i = 1; i < count; ++i)
        if (ps[i].trans_b != bt) return hipErrorInvalidValue;
    return bt ? launch_pipe_grouped_t<true>(ps, count, stream) : launch_pipe_grouped_t<false>(ps, count, stream);
}

hipError_t launch_tiled_pipe(int config, const Problem &p, hipStream_t stream) {
    if (config >= PIPE16_FIRST) return launch_tiled_pipe16(config, p, stream);
    if (p.trans_b) {
        switch (config) {
            case PIPE_256x256x64_A3: return launch_pipe_t<Pipe256x64, 2, 1, 3, true>(p, stream);
            case PIPE_256x256x64_W8_A3: return launch_pipe_t<Pipe256x64w8, 2, 1, 3, true>(p, stream);
            case PIPE_256x256x64_W8_A3_EARLY: return launch_pipe_t<Pipe256x64w8, 2, 1, 3, true, true>(p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (config) {
        // four 32-deep stages: loads every 4 slots across the step
        case PIPE_256x256x32: return launch_pipe_t<Pipe256x32, 4, 3, 4>(p, stream);
        // two 64-deep stages: the next stage's 16 loads go in early, every 2 slots
        case PIPE_256x256x64: return launch_pipe_t<Pipe256x64, 2, 1, 2>(p, stream);
        // the same with a third A buffer (160 KiB of LDS): A is loaded two steps ahead
        case PIPE_256x256x64_A3: return launch_pipe_t<Pipe256x64, 2, 1, 3>(p, stream);
        // eight waves (two per SIMD, 128 x 64 each): 8 loads per wave and stage
        case PIPE_256x256x64_W8: return launch_pipe_t<Pipe256x64w8, 2, 1, 2>(p, stream);
        case PIPE_256x256x64_W8_A3: return launch_pipe_t<Pipe256x64w8, 2, 1, 3>(p, stream);
        // half tiles: 12 loads per wave and stage, every 2 slots
        case PIPE_256x128x64: return launch_pipe_t<Pipe256x128, 2, 1, 3>(p, stream);
        case PIPE_128x256x64: return launch_pipe_t<Pipe128x256, 2, 1, 3>(p, stream);
        // eight waves, the stage barrier before the last half k-step (the default)
        case PIPE_256x256x64_W8_A3_EARLY: return launch_pipe_t<Pipe256x64w8, 2, 1, 3, false, true>(p, stream);
        // two A buffers and three B buffers
        case PIPE_256x256x64_W8_B3_EARLY: return launch_pipe_t<Pipe256x64w8B3, 2, 1, 2, false, true>(p, stream);
        case PIPE_256x256x64_B3: return launch_pipe_t<Pipe256x64B3, 2, 1, 2>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tlg
