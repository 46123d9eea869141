// gfx950 (MI355X, CDNA4) kernel for the block-scaled variant of
// C = ReLU(A . B): 8-bit (E4M3, E5M2) or 4-bit (E2M1) element codes, one
// E8M0 scale per 32 elements along K, fp32 accumulation on the matrix cores,
// ReLU and the fp16 copy-out of the quick-start kernel (TileLang article,
// aiwiki.ai/wiki/tilelang, "Programming model"). The project page "TileLang:
// a tile-level DSL for writing GPU kernels in Python" (hysenlabs.com,
// "Three backends under one language dialect") names FP4 E2M1 matrix cores
// on CDNA4 (gfx950) and a block-scaled MMA path; the forum post "TileLang:
// Writing Near-Hardware-Limit GPU Kernels in 70 Lines of Python"
// (zhichai.net, "Key Technical Milestones") names MXFP8 grouped GEMM with
// block scaling and a transposed B.
//
// Design (gfx950 first):
//  * the product is v_mfma_scale_f32_32x32x64_f8f6f4: 64 k per instruction,
//    each lane supplies one scale byte for the 32 values of one block
//    (block 2j + l/32 of a 64-deep step j: measured on the device, lane l's
//    scale multiplies bytes 0..15 of lanes l%32 and l%32+32 for 8-bit codes,
//    i.e. an 8-bit operand lane holds k = 16*(l/32) + e and
//    32 + 16*(l/32) + e (e = 0..15); a 4-bit lane holds 32 consecutive k,
//    k = 32*(l/32) + e);
//  * B is taken transposed (N x K), so both operands and both scale arrays
//    are K-contiguous; A's and B's tiles are loaded and read the same way;
//  * a stage holds 128 bytes of K per row (128 8-bit or 256 4-bit codes):
//    the byte layout, the direct-to-LDS loads (buffer_load_dwordx4 ... lds)
//    and the XOR swizzle are those of the fp16 kernels' A tile with a 64-deep
//    fp16 K step; the scale bytes of the stage (4 or 8 per row) come along
//    with buffer_load_dword ... lds, one dword per lane;
//  * every wave issues the same number of loads per stage, so one vmcnt
//    wait per stage covers tiles and scales;
//  * the epilogue (ReLU, fp16 round to nearest even, C written through LDS
//    as 16-byte row segments) is the fp16 kernels' own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

typedef int int8v_t __attribute__((ext_vector_type(8)));

// Nothing may be scheduled across this point (keeps the hand-written order).
#define TLG_MX_FENCE() __builtin_amdgcn_sched_barrier(0)

struct MxArgs {
    const uint8_t *A;   // M x K codes, lda bytes per row
    const uint8_t *B;   // N x K codes (B transposed), ldb bytes per row
    const uint8_t *SA;  // M x K/32 scale bytes, ldsa bytes per row
    const uint8_t *SB;  // N x K/32 scale bytes, ldsb bytes per row
    _Float16 *C;
    int M, N, K;        // K in elements, a multiple of 128
    int64_t lda, ldb, ldsa, ldsb, ldc;
    int tiles_m, tiles_n, group_m;
};

// 4 bytes per lane from buffer offset `voff` into LDS at lds_base + 4*lane
// (same contract as dma16: zeros for an out-of-range offset, counted in vmcnt).
__device__ __forceinline__ void dma4(int4_t srd, uint32_t lds_base, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_base),
        "v"(voff), "s"(srd)
        : "memory", "m0");
}

// Per-format constants. FMT is the matrix-core format code (0 E4M3, 1 E5M2,
// 4 E2M1).
template <class S, int FMT>
struct MxShape {
    static constexpr int EPB = FMT == 4 ? 2 : 1;             // codes per byte
    static constexpr int KPS = S::RA * EPB;                  // k per stage (row bytes RA = 128)
    static constexpr int SBR = KPS / 32;                     // scale bytes per row per stage
    static constexpr int KSTEPS = KPS / 64;                  // 64-deep MFMA steps per stage
    static constexpr int SC_A = S::BM * SBR, SC_B = S::BN * SBR;
    static constexpr int STAGE = S::STAGE_BYTES + SC_A + SC_B;
    static constexpr int NSA = SC_A / 256, NSB = SC_B / 256;  // 256-byte scale slabs
    static constexpr int SPW = (NSA + NSB) / S::WAVES;       // scale slabs per wave
    static constexpr int LOADS = S::DMA_A + S::DMA_B + SPW;  // loads per wave per stage
    static_assert(S::RA == 128, "a stage holds 128 bytes of K per row");
    static_assert(S::BM == S::BN && S::A_BYTES == S::B_BYTES, "A and B tiles are alike");
    static_assert((NSA + NSB) % S::WAVES == 0 && SPW >= 1 && NSA % SPW == 0, "scale slabs split evenly");
};

// One 64-deep step J of a stage: operand fragments from LDS, the lane's
// scale bytes, then every MFMA tile of the wave. sa/sb hold the lane's
// scale dwords of the stage shifted right by 8*(l/32), so byte 2*(J%2) of
// dword J/2 (4-bit) or byte 2J (8-bit) is the scale of block 2J + l/32.
template <class S, int FMT, int J>
__device__ __forceinline__ void mx_kstep(LDS_PTR(const char) sA, LDS_PTR(const char) sB, int wm0, int wn0, int lane,
                                         const uint32_t (&sa)[S::TM][MxShape<S, FMT>::SBR / 4],
                                         const uint32_t (&sb)[S::TN][MxShape<S, FMT>::SBR / 4],
                                         float16_t (&acc)[S::TN][S::TM]) {
    constexpr bool B8 = FMT != 4;
    constexpr int OPSEL = B8 ? 2 * J : 2 * (J % 2);
    constexpr int DW = B8 ? 0 : J / 2;
    const int half = lane / 32;
    int8v_t af[S::TM], bf[S::TN];
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm) {
        const int r = wm0 + 32 * tm + lane % 32;
        if (B8) {
            const int4_t x = *(LDS_PTR(const int4_t))(sA + lds_a_offset<S>(r, 4 * J + half));
            const int4_t y = *(LDS_PTR(const int4_t))(sA + lds_a_offset<S>(r, 4 * J + 2 + half));
            af[tm] = int8v_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        } else {
            const int4_t x = *(LDS_PTR(const int4_t))(sA + lds_a_offset<S>(r, 2 * J + half));
            af[tm] = int8v_t{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn) {
        const int r = wn0 + 32 * tn + lane % 32;
        if (B8) {
            const int4_t x = *(LDS_PTR(const int4_t))(sB + lds_a_offset<S>(r, 4 * J + half));
            const int4_t y = *(LDS_PTR(const int4_t))(sB + lds_a_offset<S>(r, 4 * J + 2 + half));
            bf[tn] = int8v_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        } else {
            const int4_t x = *(LDS_PTR(const int4_t))(sB + lds_a_offset<S>(r, 2 * J + half));
            bf[tn] = int8v_t{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        }
    }
    // D = B^T A^T as in the fp16 kernels: the first operand (and its scale)
    // is the B tile (output columns), the second the A tile (output rows)
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[tn], af[tm], acc[tn][tm], FMT, FMT, OPSEL,
                                                                          (int)sb[tn][DW], OPSEL, (int)sa[tm][DW]);
}

// mid() runs between the first and the second k-step (the kernel issues
// part of the next stage's loads there).
template <class S, int FMT, class MID>
__device__ __forceinline__ void mx_stage(LDS_PTR(const char) st, int wm0, int wn0, int lane,
                                         float16_t (&acc)[S::TN][S::TM], MID &&mid) {
    using X = MxShape<S, FMT>;
    LDS_PTR(const char) sA = st;
    LDS_PTR(const char) sB = st + S::A_BYTES;
    LDS_PTR(const char) cA = st + S::STAGE_BYTES;
    LDS_PTR(const char) cB = cA + X::SC_A;
    const int sh = 8 * (lane / 32);
    uint32_t sa[S::TM][X::SBR / 4], sb[S::TN][X::SBR / 4];
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm)
#pragma unroll
        for (int d = 0; d < X::SBR / 4; ++d)
            sa[tm][d] = *(LDS_PTR(const uint32_t))(cA + (wm0 + 32 * tm + lane % 32) * X::SBR + 4 * d) >> sh;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int d = 0; d < X::SBR / 4; ++d)
            sb[tn][d] = *(LDS_PTR(const uint32_t))(cB + (wn0 + 32 * tn + lane % 32) * X::SBR + 4 * d) >> sh;
    mx_kstep<S, FMT, 0>(sA, sB, wm0, wn0, lane, sa, sb, acc);
    mid();
    mx_kstep<S, FMT, 1>(sA, sB, wm0, wn0, lane, sa, sb, acc);
    if constexpr (X::KSTEPS == 4) {
        mx_kstep<S, FMT, 2>(sA, sB, wm0, wn0, lane, sa, sb, acc);
        mx_kstep<S, FMT, 3>(sA, sB, wm0, wn0, lane, sa, sb, acc);
    }
}

// One work-group per BM x BN output tile; STAGES LDS stages of tiles and
// scales; out-of-range rows, columns, k chunks and scale dwords read zeros
// (a zero scale byte is 2^-127 and multiplies only zero codes there).
template <class S, int FMT>
__device__ __forceinline__ void mx_tile(const MxArgs &a, int m0, int n0, LDS_PTR(char) lds) {
    using X = MxShape<S, FMT>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int nk = (a.K + X::KPS - 1) / X::KPS;
    const int nkb = a.K / 32;

    // tile loads: chunk c of a row holds codes k0 + 16*EPB*c .. +16*EPB-1
    uint32_t a_off[S::DMA_A], b_off[S::DMA_B];
    int a_k[S::DMA_A], b_k[S::DMA_B];
    bool a_ok[S::DMA_A], b_ok[S::DMA_B];
#pragma unroll
    for (int i = 0; i < S::DMA_A; ++i) {
        const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        a_off[i] = (uint32_t)(c.row * a.lda + 16 * c.chunk);
        a_k[i] = 16 * X::EPB * c.chunk;
        a_ok[i] = m0 + c.row < a.M;
    }
#pragma unroll
    for (int i = 0; i < S::DMA_B; ++i) {
        const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        b_off[i] = (uint32_t)(c.row * a.ldb + 16 * c.chunk);
        b_k[i] = 16 * X::EPB * c.chunk;
        b_ok[i] = n0 + c.row < a.N;
    }
    // scale loads: this wave's slabs are all A's or all B's; dword q of a
    // slab run is row q / (SBR/4), bytes 4*(q % (SBR/4)) .. +3 of the stage
    const int slab0 = wave * X::SPW;
    const bool sc_b = slab0 >= X::NSA;
    const int64_t lds_s = sc_b ? a.ldsb : a.ldsa;
    const int lim_s = sc_b ? a.N - n0 : a.M - m0;
    uint32_t s_off[X::SPW];
    int s_kb[X::SPW];
    bool s_ok[X::SPW];
#pragma unroll
    for (int i = 0; i < X::SPW; ++i) {
        const int q = ((slab0 + i) % X::NSA) * 64 + lane;
        const int row = q / (X::SBR / 4), d = q % (X::SBR / 4);
        s_off[i] = (uint32_t)(row * lds_s + 4 * d);
        s_kb[i] = 4 * d;
        s_ok[i] = row < lim_s;
    }

    auto issue = [&](int kt, int buf, int part) {  // part: 0 A tile, 1 B tile and scales, 2 all
        const int k0 = kt * X::KPS;
        const int64_t k0b = k0 / X::EPB;
        const int kb0 = k0 / 32;
        LDS_PTR(char) st = lds + buf * X::STAGE;
        const int4_t ra = make_srd(a.A + (int64_t)m0 * a.lda + k0b);
        const int4_t rb = make_srd(a.B + (int64_t)n0 * a.ldb + k0b);
        const int4_t rs = make_srd(sc_b ? a.SB + (int64_t)n0 * a.ldsb + kb0 : a.SA + (int64_t)m0 * a.ldsa + kb0);
        const uint32_t la = (uint32_t)(uintptr_t)(st + wave * S::DMA_A * 1024);
        const uint32_t lb = (uint32_t)(uintptr_t)(st + S::A_BYTES + wave * S::DMA_B * 1024);
        const uint32_t ls = (uint32_t)(uintptr_t)(st + S::STAGE_BYTES + (sc_b ? X::SC_A : 0) +
                                                  ((slab0 % X::NSA) * 256));
        if (part != 1) {
#pragma unroll
            for (int i = 0; i < S::DMA_A; ++i)
                dma16(ra, la + i * 1024, (a_ok[i] && k0 + a_k[i] < a.K) ? a_off[i] : kOOB);
        }
        if (part != 0) {
#pragma unroll
            for (int i = 0; i < S::DMA_B; ++i)
                dma16(rb, lb + i * 1024, (b_ok[i] && k0 + b_k[i] < a.K) ? b_off[i] : kOOB);
#pragma unroll
            for (int i = 0; i < X::SPW; ++i)
                dma4(rs, ls + i * 256, (s_ok[i] && kb0 + s_kb[i] < nkb) ? s_off[i] : kOOB);
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
    for (int s = 0; s < S::STAGES - 1; ++s)
        if (s < nk) issue(s, s, 2);

    int buf = 0;
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once at most the loads of the STAGES-2 later
        // stages are still in flight
        if (kt + S::STAGES - 2 < nk)
            wait_vmcnt<(S::STAGES - 2) * X::LOADS>();
        else
            wait_vmcnt<0>();
        barrier_lds();  // every wave's loads of stage kt are in LDS; stage kt-1 is no longer read
        // With two stages the next stage's loads go in two halves: the A
        // tile now, the B tile and the scales after the first k-step (one
        // burst of every load of all eight waves at the barrier measured
        // 1.2-2.5 % slower at 8192^3). With three stages the loads have two
        // stages to land and one burst measured 2 % faster.
        constexpr bool SPLIT = S::STAGES == 2;
        const bool more = kt + S::STAGES - 1 < nk;
        const int nb = buf == 0 ? S::STAGES - 1 : buf - 1;  // the buffer stage kt-1 used
        if (more) issue(kt + S::STAGES - 1, nb, SPLIT ? 0 : 2);
        mx_stage<S, FMT>(lds + buf * X::STAGE, wm0, wn0, lane, acc, [&]() {
            if (SPLIT && more) issue(kt + S::STAGES - 1, nb, 1);
        });
        buf = buf + 1 == S::STAGES ? 0 : buf + 1;
    }

    barrier_lds();  // every wave is done with the stages
    KArgs c{};
    c.C = a.C;
    c.M = a.M;
    c.N = a.N;
    c.ldc = a.ldc;
    store_c_tile_lds<S>(c, m0, n0, wave, lane, acc, lds);
}

template <class S, int FMT>
__global__ __launch_bounds__(S::NT) void k_mx(const MxArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[S::STAGES * MxShape<S, FMT>::STAGE];
    const int nwg = a.tiles_m * a.tiles_n;
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, nwg), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    mx_tile<S, FMT>(a, tm_idx * S::BM, tn_idx * S::BN, (LDS_PTR(char))smem);
}

// Several independent block-scaled problems in one launch: work-group ids
// are dealt to the XCDs as in the single-problem kernel, then split by
// problem in order (tile_start holds the running tile counts).
struct MxGroupArgs {
    int count;
    int tile_start[kGroupMax + 1];
    MxArgs p[kGroupMax];
};

template <class S, int FMT>
__global__ __launch_bounds__(S::NT) void k_mx_grouped(const MxGroupArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem[S::STAGES * MxShape<S, FMT>::STAGE];
    const int v = xcd_remap(blockIdx.x, g.tile_start[g.count]);
    int p = 0;
    while (p + 1 < g.count && v >= g.tile_start[p + 1]) ++p;
    const MxArgs &a = g.p[p];
    int tm_idx, tn_idx;
    grouped_tile(v - g.tile_start[p], a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    mx_tile<S, FMT>(a, tm_idx * S::BM, tn_idx * S::BN, (LDS_PTR(char))smem);
}

// ---------------------------------------------------------------------------
// Software-pipelined form: the slot program of the fp16 pipelined kernel
// (one K step = KSTEPS*T MFMA slots, T = TM*TN tiles of the wave, H = T/2):
// the first H slots finish the previous stage's last 64-deep step (tiles
// H..T-1) while this stage's first fragments and its scale dwords are read;
// each later step's fragments are read under the MFMAs of the step before;
// the direct-to-LDS loads of the next stage (tiles and scales) go out every
// SPACING slots; one vmcnt wait and one barrier per stage. Scales of the
// stage being finished ("prev") and of the new one ("cur") are both held,
// and cur becomes prev at the end of the step.
// ---------------------------------------------------------------------------

template <class S, int FMT>
struct MxFrags {
    int8v_t a[S::TM], b[S::TN];
};

template <class S, int FMT>
struct MxScales {
    uint32_t a[S::TM][MxShape<S, FMT>::SBR / 4], b[S::TN][MxShape<S, FMT>::SBR / 4];
};

// Reads of one 64-deep step J: 8-bit codes take two 16-byte reads per
// fragment (r even: bytes 0..15, odd: 16..31), 4-bit codes one; fragments
// in the order the MFMAs use them: b[0], a[0..TM-1], b[1..TN-1].
template <class S, int FMT>
constexpr int kMxFragReads = (FMT == 4 ? 1 : 2) * (S::TM + S::TN);

template <class S, int FMT>
__device__ __forceinline__ void mx_frag_read(MxFrags<S, FMT> &f, LDS_PTR(const char) sA, LDS_PTR(const char) sB,
                                             int wm0, int wn0, int J, int lane, int r) {
    constexpr bool B8 = FMT != 4;
    constexpr int PER = B8 ? 2 : 1;
    const int fi = r / PER, part = r % PER, half = lane / 32;
    const bool is_a = fi >= 1 && fi < 1 + S::TM;
    const int t = is_a ? fi - 1 : (fi == 0 ? 0 : fi - S::TM);
    const int row = (is_a ? wm0 : wn0) + 32 * t + lane % 32;
    const int chunk = B8 ? 4 * J + 2 * part + half : 2 * J + half;
    const int4_t x = *(LDS_PTR(const int4_t))((is_a ? sA : sB) + lds_a_offset<S>(row, chunk));
    int8v_t &d = is_a ? f.a[t] : f.b[t];
    if (!B8) {
        d = int8v_t{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    } else if (part == 0) {
        d[0] = x[0], d[1] = x[1], d[2] = x[2], d[3] = x[3];
    } else {
        d[4] = x[0], d[5] = x[1], d[6] = x[2], d[7] = x[3];
    }
}

// Scale dwords of one row (A: r < TM) or column (B) of the wave for a stage,
// shifted so that byte 0 is block l/32 of each 64-deep step pair.
template <class S, int FMT>
__device__ __forceinline__ void mx_scale_read(MxScales<S, FMT> &c, LDS_PTR(const char) st, int wm0, int wn0,
                                              int lane, int r) {
    using X = MxShape<S, FMT>;
    const int sh = 8 * (lane / 32);
    const bool is_a = r < S::TM;
    const int t = is_a ? r : r - S::TM;
    LDS_PTR(const char) base = st + S::STAGE_BYTES + (is_a ? 0 : X::SC_A) +
                               ((is_a ? wm0 : wn0) + 32 * t + lane % 32) * X::SBR;
    if (X::SBR == 4) {
        const uint32_t v = *(LDS_PTR(const uint32_t))base;
        (is_a ? c.a[t] : c.b[t])[0] = v >> sh;
    } else {
        const int2_t v = *(LDS_PTR(const int2_t))base;
        (is_a ? c.a[t] : c.b[t])[0] = (uint32_t)v[0] >> sh;
        (is_a ? c.a[t] : c.b[t])[X::SBR / 4 - 1] = (uint32_t)v[1] >> sh;
    }
}

// MFMA tile i of 64-deep step J from fragments f and scales c.
template <class S, int FMT>
__device__ __forceinline__ void mx_mfma_tile(const MxFrags<S, FMT> &f, const MxScales<S, FMT> &c, int J, int i,
                                             float16_t (&acc)[S::TN][S::TM]) {
    constexpr bool B8 = FMT != 4;
    const int tn = i / S::TM, tm = i % S::TM;
    const int dw = B8 ? 0 : J / 2;
    const int sb = (int)c.b[tn][dw], sa = (int)c.a[tm][dw];
    if ((B8 ? J : J % 2) == 0)
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[tn], f.a[tm], acc[tn][tm], FMT, FMT, 0, sb,
                                                                      0, sa);
    else
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[tn], f.a[tm], acc[tn][tm], FMT, FMT, 2, sb,
                                                                      2, sa);
}

template <class S, int FMT>
__global__ __launch_bounds__(S::NT) void k_mx_pipe(const MxArgs a) {
    using X = MxShape<S, FMT>;
    constexpr int T = S::TM * S::TN, H = T / 2;
    constexpr int KS = X::KSTEPS;
    constexpr int READS = kMxFragReads<S, FMT>;
    constexpr int SREADS = S::TM + S::TN;        // scale reads per stage
    constexpr int R0 = READS + SREADS;           // reads under the first H slots
    constexpr int PER0 = (R0 + H - 1) / H;       // ... per slot
    constexpr int PER = (READS + T - 1) / T;     // reads per slot under a full step
    constexpr int SLOTS = KS * T;
    constexpr int LOADS = X::LOADS;
    constexpr int SPACING = SLOTS >= 2 * LOADS + 2 ? 2 : 1;
    constexpr int DOFF = 1;
    static_assert(S::STAGES == 2 && KS % 2 == 0 && T % 2 == 0, "two stages; the last step uses f[1]");
    static_assert(DOFF + (LOADS - 1) * SPACING < SLOTS, "loads must fit in one K step");
    __shared__ __attribute__((aligned(1024))) char smem[S::STAGES * X::STAGE];
    LDS_PTR(char) lds = (LDS_PTR(char))smem;
    const int nwg = a.tiles_m * a.tiles_n;
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, nwg), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    const int m0 = tm_idx * S::BM, n0 = tn_idx * S::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int nk = (a.K + X::KPS - 1) / X::KPS;
    const int nkb = a.K / 32;

    // load j of a stage: j < DMA_A an A chunk, then B chunks, then scale dwords
    uint32_t off[LOADS];
    int kin[LOADS];
    bool ok[LOADS];
#pragma unroll
    for (int i = 0; i < S::DMA_A; ++i) {
        const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        off[i] = (uint32_t)(c.row * a.lda + 16 * c.chunk);
        kin[i] = 16 * X::EPB * c.chunk;
        ok[i] = m0 + c.row < a.M;
    }
#pragma unroll
    for (int i = 0; i < S::DMA_B; ++i) {
        const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
        off[S::DMA_A + i] = (uint32_t)(c.row * a.ldb + 16 * c.chunk);
        kin[S::DMA_A + i] = 16 * X::EPB * c.chunk;
        ok[S::DMA_A + i] = n0 + c.row < a.N;
    }
    const int slab0 = wave * X::SPW;
    const bool sc_b = slab0 >= X::NSA;
    const int64_t lds_s = sc_b ? a.ldsb : a.ldsa;
    const int lim_s = sc_b ? a.N - n0 : a.M - m0;
#pragma unroll
    for (int i = 0; i < X::SPW; ++i) {
        const int q = ((slab0 + i) % X::NSA) * 64 + lane;
        const int row = q / (X::SBR / 4), d = q % (X::SBR / 4);
        off[S::DMA_A + S::DMA_B + i] = (uint32_t)(row * lds_s + 4 * d);
        kin[S::DMA_A + S::DMA_B + i] = 4 * d;  // blocks, not codes
        ok[S::DMA_A + S::DMA_B + i] = row < lim_s;
    }
    auto dma = [&](int j, int kt) {
        const int k0 = kt * X::KPS;
        const int64_t k0b = k0 / X::EPB;
        const int kb0 = k0 / 32;
        LDS_PTR(char) st = lds + (kt & 1) * X::STAGE;
        if (j < S::DMA_A) {
            const int4_t r = make_srd(a.A + (int64_t)m0 * a.lda + k0b);
            dma16(r, (uint32_t)(uintptr_t)(st + (wave * S::DMA_A + j) * 1024),
                  ok[j] && k0 + kin[j] < a.K ? off[j] : kOOB);
        } else if (j < S::DMA_A + S::DMA_B) {
            const int4_t r = make_srd(a.B + (int64_t)n0 * a.ldb + k0b);
            dma16(r, (uint32_t)(uintptr_t)(st + S::A_BYTES + (wave * S::DMA_B + j - S::DMA_A) * 1024),
                  ok[j] && k0 + kin[j] < a.K ? off[j] : kOOB);
        } else {
            const int i = j - S::DMA_A - S::DMA_B;
            const int4_t r = make_srd(sc_b ? a.SB + (int64_t)n0 * a.ldsb + kb0 : a.SA + (int64_t)m0 * a.ldsa + kb0);
            dma4(r, (uint32_t)(uintptr_t)(st + S::STAGE_BYTES + (sc_b ? X::SC_A : 0) + ((slab0 + i) % X::NSA) * 256),
                 ok[j] && kb0 + kin[j] < nkb ? off[j] : kOOB);
        }
    };

    float16_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    MxFrags<S, FMT> f[2];
    MxScales<S, FMT> prev, cur;
#pragma unroll
    for (int t = 0; t < S::TN; ++t) {
        f[1].b[t] = int8v_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int d = 0; d < X::SBR / 4; ++d) prev.b[t][d] = 0;
    }
#pragma unroll
    for (int t = 0; t < S::TM; ++t) {
        f[1].a[t] = int8v_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int d = 0; d < X::SBR / 4; ++d) prev.a[t][d] = 0;
    }

#pragma unroll
    for (int j = 0; j < LOADS; ++j) dma(j, 0);
    wait_vmcnt<0>();
    barrier_lds();

    for (int kt = 0; kt < nk; ++kt) {
        LDS_PTR(const char) st = lds + (kt & 1) * X::STAGE;
        LDS_PTR(const char) sA = st;
        LDS_PTR(const char) sB = st + S::A_BYTES;
        TLG_MX_FENCE();
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) {
            if (q < H) {
                mx_mfma_tile<S, FMT>(f[1], prev, KS - 1, H + q, acc);
#pragma unroll
                for (int r = PER0 * q; r < PER0 * q + PER0; ++r) {
                    if (r < SREADS)
                        mx_scale_read<S, FMT>(cur, st, wm0, wn0, lane, r);
                    else if (r < R0)
                        mx_frag_read<S, FMT>(f[0], sA, sB, wm0, wn0, 0, lane, r - SREADS);
                }
            } else if (q < H + (KS - 1) * T) {
                const int ks = (q - H) / T, i = (q - H) % T;
                mx_mfma_tile<S, FMT>(f[ks & 1], cur, ks, i, acc);
#pragma unroll
                for (int r = PER * i; r < PER * i + PER; ++r)
                    if (r < READS) mx_frag_read<S, FMT>(f[(ks + 1) & 1], sA, sB, wm0, wn0, ks + 1, lane, r);
            } else {
                mx_mfma_tile<S, FMT>(f[1], cur, KS - 1, q - H - (KS - 1) * T, acc);
            }
            if (q >= DOFF && (q - DOFF) % SPACING == 0 && (q - DOFF) / SPACING < LOADS)
                dma((q - DOFF) / SPACING, kt + 1);
            TLG_MX_FENCE();
        }
        wait_vmcnt<0>();  // this wave's loads of stage kt+1 are in LDS
        barrier_lds();    // ... and every wave's; stage kt is no longer read
        prev = cur;
    }
#pragma unroll
    for (int i = H; i < T; ++i) mx_mfma_tile<S, FMT>(f[1], prev, KS - 1, i, acc);

    barrier_lds();
    KArgs c{};
    c.C = a.C;
    c.M = a.M;
    c.N = a.N;
    c.ldc = a.ldc;
    store_c_tile_lds<S>(c, m0, n0, wave, lane, acc, lds);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

using Mx256 = TileShape<256, 256, 64, 2, 4, 2>;  // eight waves (two per SIMD), 128 x 64 each
using Mx128 = TileShape<128, 128, 64, 2, 2, 3>;  // four waves, 64 x 64 each

using Mx256w4 = TileShape<256, 256, 64, 2, 2, 2>;  // four waves, 128 x 128 each

const TileConfig kMxConfigs[MX_CONFIGS] = {
    {256, 256, 128, Mx256::NT, Mx256::STAGES, "mx_256x256_w2x4_s2"},
    {128, 128, 128, Mx128::NT, Mx128::STAGES, "mx_128x128_w2x2_s3"},
    {256, 256, 128, Mx256::NT, Mx256::STAGES, "mx_pipe_256x256_w2x4_s2"},
    {256, 256, 128, Mx256w4::NT, Mx256w4::STAGES, "mx_pipe_256x256_w2x2_s2"},
};

template <class S, int FMT>
static hipError_t launch_mx_t(const MxArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((k_mx<S, FMT>), dim3(a.tiles_m * a.tiles_n), dim3(S::NT), 0, stream, a);
    return hipGetLastError();
}

template <class S, int FMT>
static hipError_t launch_mx_pipe_t(const MxArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((k_mx_pipe<S, FMT>), dim3(a.tiles_m * a.tiles_n), dim3(S::NT), 0, stream, a);
    return hipGetLastError();
}

template <class S, int FMT, bool PIPE>
static hipError_t launch_mx_kind(const MxArgs &a, hipStream_t stream) {
    if constexpr (PIPE)
        return launch_mx_pipe_t<S, FMT>(a, stream);
    else
        return launch_mx_t<S, FMT>(a, stream);
}

template <class S, bool PIPE>
static hipError_t launch_mx_fmt(int hw_format, const MxArgs &a, hipStream_t stream) {
    switch (hw_format) {
        case 0: return launch_mx_kind<S, 0, PIPE>(a, stream);
        case 1: return launch_mx_kind<S, 1, PIPE>(a, stream);
        case 4: return launch_mx_kind<S, 4, PIPE>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

static int mx_hw_format(int format) { return format == 1 ? 0 : format == 2 ? 1 : format == 3 ? 4 : -1; }

static MxArgs mx_args(const TileConfig &tc, const MxProblem &p) {
    const int epb = mx_hw_format(p.format) == 4 ? 2 : 1;
    MxArgs a;
    a.A = (const uint8_t *)p.A;
    a.B = (const uint8_t *)p.B;
    a.SA = (const uint8_t *)p.SA;
    a.SB = (const uint8_t *)p.SB;
    a.C = (_Float16 *)p.C;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.lda = p.lda / epb;
    a.ldb = p.ldb / epb;
    a.ldsa = p.ldsa;
    a.ldsb = p.ldsb;
    a.ldc = p.ldc;
    a.tiles_m = (int)((p.M + tc.bm - 1) / tc.bm);
    a.tiles_n = (int)((p.N + tc.bn - 1) / tc.bn);
    a.group_m = 4;
    return a;
}

template <class S, int FMT>
static hipError_t launch_mx_grouped_t(const MxGroupArgs &g, hipStream_t stream) {
    hipLaunchKernelGGL((k_mx_grouped<S, FMT>), dim3(g.tile_start[g.count]), dim3(S::NT), 0, stream, g);
    return hipGetLastError();
}

template <class S>
static hipError_t launch_mx_grouped_fmt(int hw_format, const MxGroupArgs &g, hipStream_t stream) {
    switch (hw_format) {
        case 0: return launch_mx_grouped_t<S, 0>(g, stream);
        case 1: return launch_mx_grouped_t<S, 1>(g, stream);
        case 4: return launch_mx_grouped_t<S, 4>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mx_grouped(int config, const MxProblem *ps, int count, hipStream_t stream) {
    if ((config != MX_256x256_W8 && config != MX_128x128_W4) || count < 1 || count > kGroupMax)
        return hipErrorInvalidValue;
    const TileConfig &tc = kMxConfigs[config];
    MxGroupArgs g;
    g.count = count;
    g.tile_start[0] = 0;
    for (int i = 0; i < count; ++i) {
        if (ps[i].format != ps[0].format) return hipErrorInvalidValue;
        g.p[i] = mx_args(tc, ps[i]);
        g.tile_start[i + 1] = g.tile_start[i] + g.p[i].tiles_m * g.p[i].tiles_n;
    }
    const int hw = mx_hw_format(ps[0].format);
    return config == MX_256x256_W8 ? launch_mx_grouped_fmt<Mx256>(hw, g, stream)
                                   : launch_mx_grouped_fmt<Mx128>(hw, g, stream);
}

hipError_t launch_mx(int config, const MxProblem &p, hipStream_t stream) {
    if (config < 0 || config >= MX_CONFIGS) return hipErrorInvalidValue;
    const int hw = mx_hw_format(p.format);
    const MxArgs a = mx_args(kMxConfigs[config], p);
    switch (config) {
        case MX_256x256_W8: return launch_mx_fmt<Mx256, false>(hw, a, stream);
        case MX_128x128_W4: return launch_mx_fmt<Mx128, false>(hw, a, stream);
        case MX_PIPE_256x256_W8: return launch_mx_fmt<Mx256, true>(hw, a, stream);
        default: return launch_mx_fmt<Mx256w4, true>(hw, a, stream);
    }
}

}  // namespace tlg
