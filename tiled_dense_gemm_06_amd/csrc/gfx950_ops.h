// Device-side building blocks shared by the gfx950 GEMM+ReLU kernels: vector
// types, buffer descriptors, the direct global->LDS load, wait and barrier
// helpers, the transposing B-fragment read and the ReLU + fp16 epilogue.
#ifndef TLG_GFX950_OPS_H
#define TLG_GFX950_OPS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_layout.h"

namespace tlg {


typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(T) __attribute__((address_space(3))) T *

// Every buffer descriptor covers offsets [0, kRange); a lane given offset
// kOOB reads zeros. Host code guarantees every real offset is below kRange.
constexpr uint32_t kRange = 0x7ffffff0u;
constexpr uint32_t kOOB = 0x7ffffff0u;

struct KArgs {
    const _Float16 *A;
    const _Float16 *B;
    _Float16 *C;
    float *W;          // split-K partials (split-K kernels only)
    int *cnt;          // per-tile counters of the skinny kernel's split strips (zero between calls)
    int M, N, K;
    int64_t lda, ldb, ldc;
    int tiles_m, tiles_n, group_m;
    int k_split;       // K elements per split, a multiple of BK
    // K rows the direct-to-LDS loads cover (tiled and pipelined kernels): K
    // when K and N are multiples of 8; otherwise the largest multiple of 8
    // below K, and the last 1..8 rows are added from a zero-padded block
    // staged element by element (see stage_tail).
    int kmain;
};

// Arguments of a grouped launch: problem p owns work-group ids (after the
// XCD renumbering) tile_start[p] .. tile_start[p+1]-1.
struct GroupArgs {
    int count;
    int tile_start[17];
    KArgs p[16];
};

typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));

// Buffer descriptor: base address, stride 0, kRange bytes, word 3 = 0x00020000
// (raw, untyped buffer on gfx9-class parts).
__device__ __forceinline__ int4_t make_srd(const void *base) {
    const uint64_t p = (uint64_t)base;
    int4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));
    r[2] = (int)kRange;
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_base + 16*lane.
// Issued through inline assembly: the compiler does not see an LDS write here,
// so it does not add its own conservative vmcnt(0) wait before every later
// LDS read. The kernels wait for these loads themselves (wait_vmcnt) before
// the barrier that publishes a stage. M0 needs one wait state after its write.
__device__ __forceinline__ void dma16(int4_t srd, uint32_t lds_base, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base),
        "v"(voff), "s"(srd)
        : "memory", "m0");
}

// The same with a scalar offset added to every lane's (the instruction's
// soffset operand).
__device__ __forceinline__ void dma16_soff(int4_t srd, uint32_t lds_base, uint32_t voff, uint32_t soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_base),
        "v"(voff), "s"(srd), "s"(soff)
        : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// All LDS operations of this wave are complete, then the work-group barrier.
// The wait is the compiler's own s_waitcnt (lgkmcnt(0), encoding 0xC07F on
// gfx9-class parts: vmcnt and expcnt left at their maxima), so the compiler
// knows that no LDS read is pending afterwards and adds no wait of its own
// for them. The barrier is inline assembly with a "memory" clobber, which
// keeps the compiler from moving memory accesses across it; it repeats the
// wait so that nothing the compiler might place between the two is left
// pending at the barrier (the repeated wait costs nothing).
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ReLU on the fp32 accumulator (everything not > 0 becomes +0, so -0 and NaN
// give +0), then the fp16 conversion, which rounds to nearest even.
__device__ __forceinline__ _Float16 relu_to_half(float x) { return (_Float16)(x > 0.0f ? x : 0.0f); }

__device__ __forceinline__ half8_t read_b_frag(LDS_PTR(const char) base, int off_lo, int off_hi) {
    short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(short4_t))(base + off_lo));
    short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(short4_t))(base + off_hi));
    short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(half8_t, v);
}

// One 16-wide k-step s of an LDS stage: read the operand fragments of every
// MFMA tile of this wave and accumulate. BT: the B tile is held like the A
// tile (rows n, K-contiguous; B given transposed), so its fragments are read
// the way A's are.
template <class S, bool BT = false>
__device__ __forceinline__ void mma_kstep(LDS_PTR(const char) sA, LDS_PTR(const char) sB, int s, int wm0, int wn0,
                                          int lane, float16_t (&acc)[S::TN][S::TM]) {
    half8_t bf[S::TN], af[S::TM];
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
        bf[tn] = BT ? *(LDS_PTR(const half8_t))(sB + frag_a_offset<S>(wn0, tn, s, lane))
                    : read_b_frag(sB, frag_b_offset<S>(wn0, tn, s, 0, lane), frag_b_offset<S>(wn0, tn, s, 1, lane));
#pragma unroll
    for (int tm = 0; tm < S::TM; ++tm) af[tm] = *(LDS_PTR(const half8_t))(sA + frag_a_offset<S>(wm0, tm, s, lane));
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[tn], af[tm], acc[tn][tm], 0, 0, 0);
}

// The tile product of one LDS stage.
template <class S, bool BT = false>
__device__ __forceinline__ void mma_stage(LDS_PTR(const char) sA, LDS_PTR(const char) sB, int wm0, int wn0, int lane,
                                          float16_t (&acc)[S::TN][S::TM]) {
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) mma_kstep<S, BT>(sA, sB, s, wm0, wn0, lane, acc);
}

// Rows kmain .. K-1 of the sum (1 to 8 of them) as one 16-deep block in the
// stage layout of LDS buffer (sA, sB): element-wise loads with bounds checks,
// zeros outside the matrices, so one MFMA k-step adds them. Used when K or N
// is not a multiple of 8: the direct-to-LDS loads then stop at kmain, so no
// 16-byte chunk they fetch crosses the K edge of A, and a chunk crossing the
// N edge of B reads at most into the next row of B (needs ldb >= 8), whose
// values only reach output columns >= N, which are never stored.
// BT (B given transposed, N x K): the B block is staged like the A block,
// rows n, k = kmain .. kmain+15 (needs BM == BN).
template <class S, bool BT = false>
__device__ __forceinline__ void stage_tail(const KArgs &a, int m0, int n0, LDS_PTR(char) sA, LDS_PTR(char) sB,
                                           int tid) {
    for (int q = tid; q < S::BM * 2; q += S::NT) {
        const int row = q / 2, chunk = q % 2;
        const int m = m0 + row, k = a.kmain + 8 * chunk;
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (m < a.M && k + e < a.K) ? a.A[(int64_t)m * a.lda + k + e] : (_Float16)0.0f;
        *(LDS_PTR(half8_t))(sA + lds_a_offset<S>(row, chunk)) = v;
    }
    if (BT) {
        static_assert(!BT || S::BM == S::BN, "transposed B is staged in the A layout");
        for (int q = tid; q < S::BN * 2; q += S::NT) {
            const int row = q / 2, chunk = q % 2;
            const int n = n0 + row, k = a.kmain + 8 * chunk;
            half8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (n < a.N && k + e < a.K) ? a.B[(int64_t)n * a.ldb + k + e] : (_Float16)0.0f;
            *(LDS_PTR(half8_t))(sB + lds_a_offset<S>(row, chunk)) = v;
        }
        return;
    }
    for (int q = tid; q < 16 * S::CB; q += S::NT) {
        const int row = q / S::CB, chunk = q % S::CB;
        const int k = a.kmain + row, n = n0 + 8 * chunk;
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (k < a.K && n + e < a.N) ? a.B[(int64_t)k * a.ldb + n + e] : (_Float16)0.0f;
        *(LDS_PTR(half8_t))(sB + lds_b_offset<S>(row, chunk)) = v;
    }
}

// Epilogue of an output tile: ReLU, round to nearest even, 8-byte stores of
// the four consecutive n a lane holds per register quad (any 2-byte aligned
// address works); a quad that crosses column N is stored element by element;
// lanes outside the window get offset kOOB and the hardware drops their
// stores.
template <class S>
__device__ __forceinline__ void store_c_tile(const KArgs &a, int m0, int n0, int wm0, int wn0, int lane,
                                             const float16_t (&acc)[S::TN][S::TM]) {
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(a.C + (int64_t)m0 * a.ldc + n0, (short)0, (int)kRange, 0x00020000);
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const int mr = acc_m(wm0, tm, lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nr = acc_n(wn0, tn, 4 * q, lane);
                const bool row_in = m0 + mr < a.M;
                half4_t h = {relu_to_half(acc[tn][tm][4 * q]), relu_to_half(acc[tn][tm][4 * q + 1]),
                             relu_to_half(acc[tn][tm][4 * q + 2]), relu_to_half(acc[tn][tm][4 * q + 3])};
                const uint32_t base = (uint32_t)((mr * a.ldc + nr) * 2);
                if (n0 + nr + 4 <= a.N || !row_in) {
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(int2_t, h), rc, row_in ? base : kOOB, 0, 0);
                } else {
                    // each element converted and stored on its own (the 16-bit
                    // buffer-store builtin fed from an odd element of a half
                    // vector was observed to store the even element instead)
                    _Float16 *crow = a.C + (int64_t)(m0 + mr) * a.ldc + n0 + nr;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n0 + nr + e < a.N) crow[e] = relu_to_half(acc[tn][tm][4 * q + e]);
                }
            }
        }
}

// Epilogue through LDS: ReLU and the fp16 conversion, then the two 8-byte
// halves of each 16-byte row piece, held by lanes l and l+32, are brought
// into one lane (v_permlane32_swap exchanges the upper 32 lanes of its first
// operand with the lower 32 lanes of its second), the pieces go to this
// wave's WTM x WTN block of LDS (layout: epi_lds_offset, conflict-free for
// every 16 lanes), and come back as whole row segments of the wave block for
// 16-byte buffer stores (rows >= M dropped by the range check, a piece
// crossing column N stored element by element). The caller makes sure no
// wave still reads or loads into the first BM*BN*2 bytes of LDS.
template <class S>
__device__ __forceinline__ void store_c_tile_lds(const KArgs &a, int m0, int n0, int wave, int lane,
                                                 const float16_t (&acc)[S::TN][S::TM], LDS_PTR(char) lds) {
    constexpr int PITCH = S::WTN * 2, CH = S::WTN / 8;
    static_assert(CH == 4 || CH == 8 || CH == 16, "wave blocks 32, 64 or 128 columns wide");
    static_assert(S::WAVES * S::WTM * PITCH <= S::STAGES * S::STAGE_BYTES, "C tile must fit the stages' LDS");
    LDS_PTR(char) q = lds + wave * S::WTM * PITCH;
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            uint32_t d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const half2_t h = {relu_to_half(acc[tn][tm][2 * i]), relu_to_half(acc[tn][tm][2 * i + 1])};
                d[i] = __builtin_bit_cast(uint32_t, h);
            }
            const int row = epi_piece_row(tm, lane);
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                // quads 2*pr and 2*pr+1 (registers 4 apart): lane l < 32 ends up
                // with columns 16*pr + 0..7 of its row, lane l+32 with 16*pr + 8..15
                const auto s0 = __builtin_amdgcn_permlane32_swap(d[4 * pr], d[4 * pr + 2], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(d[4 * pr + 1], d[4 * pr + 3], false, false);
                const int4_t v = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
                *(LDS_PTR(int4_t))(q + epi_lds_offset<S>(row, epi_piece_index(tn, pr, lane))) = v;
            }
        }
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(a.C + (int64_t)m0 * a.ldc + n0, (short)0, (int)kRange, 0x00020000);
    constexpr int ROWS = 64 / CH;  // rows per wave instruction
#pragma unroll
    for (int k = 0; k < S::WTM / ROWS; ++k) {
        const int row = epi_read_row<S>(k, lane), c = epi_read_piece<S>(lane);
        const int4_t v = *(LDS_PTR(const int4_t))(q + epi_lds_offset<S>(row, c));
        const int mr = wm0 + row, nr = wn0 + 8 * c;
        const bool row_in = m0 + mr < a.M;
        if (n0 + nr + 8 <= a.N || !row_in) {
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, row_in ? (uint32_t)((mr * a.ldc + nr) * 2) : kOOB, 0, 0);
        } else {
            const half8_t h = __builtin_bit_cast(half8_t, v);
            _Float16 *crow = a.C + (int64_t)(m0 + mr) * a.ldc + n0 + nr;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n0 + nr + e < a.N) crow[e] = h[e];
        }
    }
}

}  // namespace tlg

#endif
