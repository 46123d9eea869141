// Software-pipelined gfx950 kernel for C = ReLU(A . B) on 16 x 16 x 32 MFMA
// tiles: the quick-start kernel of the TileLang article
// (aiwiki.ai/wiki/tilelang, "Programming model") with its T.Pipelined K loop
// scheduled by hand.
//
// Why a second MFMA shape. These parts run matrix-heavy kernels at a
// power-limited clock, so what a GEMM can sustain is set by the energy it
// spends per FLOP. Measured on one MI355X with nothing but MFMAs on random
// fp16 operands, two waves per SIMD, equal matrix-core occupancy (0.92):
// v_mfma_f32_16x16x32_f16 held 1.93 GHz and 1.88 PFLOP/s where
// v_mfma_f32_32x32x16_f16 held 1.67 GHz and 1.62 PFLOP/s. (Per FLOP the
// 16 x 16 form moves about a fifth fewer operand and accumulator registers:
// 16 + 16 against 8 + 32 per 32768 FLOP.)
//
// Layout and schedule. A 256 x 256 output tile per work-group of four waves,
// one per SIMD, each wave 128 x 128 = 8 x 8 MFMA tiles with their 256 fp32
// accumulators; 64-deep LDS stages fed by direct global->LDS loads (A
// K-contiguous, B N-contiguous and read back transposed by
// ds_read_b64_tr_b16), XOR-swizzled so every fragment read is free of bank
// conflicts. One K step is a fixed sequence of 128 MFMA slots (two 32-deep
// k-steps of 64 MFMAs); between MFMAs sit the LDS reads of the next k-step's
// fragments and, every SPACING slots, one direct-to-LDS load of a later
// stage, so a lone wave per SIMD never waits on an operand. The loop runs
// over whole stages only, so every stage in it is wholly inside K and no load
// in the slot program needs a range check; the rows of K past the last whole
// stage are added after the loop (one stage loaded with per-lane ranges, then
// a zero-padded block staged element by element). The C tile leaves through
// LDS as whole 256-byte row segments.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_ops.h"
#include "kernels.h"
#include "tile_layout.h"

namespace tlg {

// Operand fragments of one 32-deep k-step: TM A fragments (one ds_read_b128
// each) and TN B fragments (two transposing 8-byte reads each).
template <class S>
struct Frags16 {
    half8_t a[S::TM];
    short4_t blo[S::TN], bhi[S::TN];
};

// The fragment reads of one k-step, in the order the MFMAs use them (tile i
// uses b[i / TM] and a[i % TM]): b[0] (two reads), a[0..TM-1], then
// b[1..TN-1] (two reads each). BT (B given transposed, N x K): the B tile is
// held like the A tile and each B fragment is one 16-byte read.
template <class S, bool BT = false>
constexpr int kFragReads16 = S::TM + (BT ? 1 : 2) * S::TN;

// Per-lane parts of the fragment addresses (frag_a16_lane, frag_b16_lane):
// A for each k-step parity, B for each fragment column (BT: b[0], b[1] for
// each k-step parity, as for A); the rest of each address is a constant in
// the read's offset field.
template <class S>
struct FragLanes16 {
    uint32_t a[2];
    uint32_t b[S::TN];
};

template <class S, bool BT = false>
__device__ __forceinline__ void frag_read16(Frags16<S> &f, LDS_PTR(const char) sA, LDS_PTR(const char) sB,
                                            const FragLanes16<S> &o, int s, int r) {
    if constexpr (BT) {
        if (r == 0 || r > S::TM) {
            const int tn = r == 0 ? 0 : r - S::TM;
            const short8_t v = *(LDS_PTR(const short8_t))(sB + o.b[s & 1] + tn * 16 * S::RA);
            f.blo[tn] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
            f.bhi[tn] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
        } else {
            f.a[r - 1] = *(LDS_PTR(const half8_t))(sA + o.a[s & 1] + (r - 1) * 16 * S::RA);
        }
        return;
    }
    if (r < 2) {
        LDS_PTR(short4_t) p = (LDS_PTR(short4_t))(sB + o.b[0] + (32 * s + 4 * r) * S::RB);
        if (r == 0)
            f.blo[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
        else
            f.bhi[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    } else if (r < 2 + S::TM) {
        const int tm = r - 2;
        f.a[tm] = *(LDS_PTR(const half8_t))(sA + o.a[s & 1] + tm * 16 * S::RA);
    } else {
        const int tn = 1 + (r - 2 - S::TM) / 2, h = (r - 2 - S::TM) % 2;
        LDS_PTR(short4_t) p = (LDS_PTR(short4_t))(sB + o.b[tn] + (32 * s + 4 * h) * S::RB);
        if (h == 0)
            f.blo[tn] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
        else
            f.bhi[tn] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    }
}

// The MFMA is written out so that each accumulator tuple stays in its own
// four AGPRs and is accumulated in place: with 256 accumulators, 128
// fragment registers and the addresses live at once, the compiler's own
// register assignment for the builtin copies accumulators between AGPRs and
// VGPRs around every MFMA. Register hazards the compiler cannot see here are
// excluded by the schedule: a fragment register is rewritten, and an
// accumulator used again, only 64 MFMA slots after its last use, and the
// epilogue waits explicitly before it reads the accumulators
// (mfma16_results_ready). The compiler still makes every MFMA wait for the
// LDS reads of its operands.
template <class S>
__device__ __forceinline__ void mfma16_tile(const Frags16<S> &f, int i, float4_t (&acc)[S::TN][S::TM]) {
    const int tn = i / S::TM, tm = i % S::TM;
    const half8_t b =
        __builtin_bit_cast(half8_t, __builtin_shufflevector(f.blo[tn], f.bhi[tn], 0, 1, 2, 3, 4, 5, 6, 7));
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[tn][tm]) : "v"(b), "v"(f.a[tm]));
}

// Wait states between the last MFMAs and any other instruction reading
// their results (more than the 18 a 16 x 16 x 32 f16 MFMA needs).
__device__ __forceinline__ void mfma16_results_ready() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

#define TLG_SCHED_FENCE16() __builtin_amdgcn_sched_barrier(0)

template <class S, int ASTAGES>
constexpr int pipe16_lds_bytes() {
    return ASTAGES * S::A_BYTES + S::STAGES * S::B_BYTES;  // A buffers first, then the B buffers
}

// Epilogue: ReLU and the fp16 conversion of each lane's four consecutive n of
// one row, written as 8-byte pieces into this wave's WTM x WTN block of LDS
// (epi16_offset), then read back as whole row segments for 16-byte stores
// (rows >= M dropped by the buffer range check; a piece crossing column N is
// stored element by element). The caller makes sure no wave still reads or
// loads into the first WAVES * WTM * WTN * 2 bytes of LDS.
template <class S>
__device__ __forceinline__ void store_c_tile16_lds(const KArgs &a, int m0, int n0, int wave, int lane,
                                                   const float4_t (&acc)[S::TN][S::TM], LDS_PTR(char) lds) {
    constexpr int PIECES = S::WTN / 8;  // 16-byte pieces per row of the wave block (8 or 16)
    LDS_PTR(char) q = lds + wave * S::WTM * S::WTN * 2;
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const half4_t h = {relu_to_half(acc[tn][tm][0]), relu_to_half(acc[tn][tm][1]),
                               relu_to_half(acc[tn][tm][2]), relu_to_half(acc[tn][tm][3])};
            const int row = 16 * tm + lane % 16, col = 16 * tn + 4 * (lane / 16);
            *(LDS_PTR(half4_t))(q + epi16_offset<S>(row, col / 8) + 2 * (col % 8)) = h;
        }
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(a.C + (int64_t)m0 * a.ldc + n0, (short)0, (int)kRange, 0x00020000);
#pragma unroll
    for (int k = 0; k < S::WTM / (64 / PIECES); ++k) {
        const int row = k * (64 / PIECES) + lane / PIECES, piece = lane % PIECES;
        const int4_t v = *(LDS_PTR(const int4_t))(q + epi16_offset<S>(row, piece));
        const int mr = wm0 + row, nr = wn0 + 8 * piece;
        const bool row_in = m0 + mr < a.M;
        if (n0 + nr + 8 <= a.N || !row_in) {
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, row_in ? (uint32_t)((mr * a.ldc + nr) * 2) : kOOB, 0, 0);
        } else {
            const half8_t hv = __builtin_bit_cast(half8_t, v);
            _Float16 *crow = a.C + (int64_t)(m0 + mr) * a.ldc + n0 + nr;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n0 + nr + e < a.N) crow[e] = hv[e];
        }
    }
}

// Direct-to-LDS loads that leave five wait states between any earlier
// instruction and the load. With B transposed the kernel runs with more
// scalar registers spilled, and the compiler may reload a descriptor word
// (v_readlane, a vector-ALU write of a scalar register) right before the
// inline-assembly load, which reads the descriptor, and must not read it
// within five wait states of that write. The K tail of those instantiations
// and the loop of their tile that holds row N (BROWS) take these; the loop
// of the tiles inside N keeps the plain loads (the test of the generated
// assembly finds no such reload there, and the wait would cost 2 %).
__device__ __forceinline__ void dma16_settled(int4_t srd, uint32_t lds_base, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base),
        "v"(voff), "s"(srd)
        : "memory", "m0");
}
__device__ __forceinline__ void dma16_soff_settled(int4_t srd, uint32_t lds_base, uint32_t voff, uint32_t soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_base),
        "v"(voff), "s"(srd), "s"(soff)
        : "memory", "m0");
}
template <bool SETTLED>
__device__ __forceinline__ void p16_dma(int4_t srd, uint32_t lds_base, uint32_t voff) {
    if constexpr (SETTLED)
        dma16_settled(srd, lds_base, voff);
    else
        dma16(srd, lds_base, voff);
}
template <bool SETTLED>
__device__ __forceinline__ void p16_dma_soff(int4_t srd, uint32_t lds_base, uint32_t voff, uint32_t soff) {
    if constexpr (SETTLED)
        dma16_soff_settled(srd, lds_base, voff, soff);
    else
        dma16_soff(srd, lds_base, voff, soff);
}

// The MFMAs of one B column (acc[tn][0..TM-1]) as one block that ends with 20
// wait states, so that whatever the compiler places after it (a copy or a
// spill of an accumulator, which it may schedule right behind an MFMA it
// does not see the latency of) reads finished results. Used by the K tail,
// which runs once per tile.
template <class S>
__device__ __forceinline__ void mfma16_column_fenced(const Frags16<S> &f, int tn, float4_t (&acc)[S::TN][S::TM]) {
    static_assert(S::TM == 8 || S::TM == 6, "a column of six or eight 16 x 16 tiles");
    const half8_t b =
        __builtin_bit_cast(half8_t, __builtin_shufflevector(f.blo[tn], f.bhi[tn], 0, 1, 2, 3, 4, 5, 6, 7));
    if constexpr (S::TM == 8) {
        asm volatile(
            "v_mfma_f32_16x16x32_f16 %0, %8, %9, %0\n\t"
            "v_mfma_f32_16x16x32_f16 %1, %8, %10, %1\n\t"
            "v_mfma_f32_16x16x32_f16 %2, %8, %11, %2\n\t"
            "v_mfma_f32_16x16x32_f16 %3, %8, %12, %3\n\t"
            "v_mfma_f32_16x16x32_f16 %4, %8, %13, %4\n\t"
            "v_mfma_f32_16x16x32_f16 %5, %8, %14, %5\n\t"
            "v_mfma_f32_16x16x32_f16 %6, %8, %15, %6\n\t"
            "v_mfma_f32_16x16x32_f16 %7, %8, %16, %7\n\t"
            "s_nop 7\n\ts_nop 7\n\ts_nop 3"
            : "+a"(acc[tn][0]), "+a"(acc[tn][1]), "+a"(acc[tn][2]), "+a"(acc[tn][3]), "+a"(acc[tn][4]),
              "+a"(acc[tn][5]), "+a"(acc[tn][6]), "+a"(acc[tn][7])
            : "v"(b), "v"(f.a[0]), "v"(f.a[1]), "v"(f.a[2]), "v"(f.a[3]), "v"(f.a[4]), "v"(f.a[5]), "v"(f.a[6]),
              "v"(f.a[7]));
    } else {
        asm volatile(
            "v_mfma_f32_16x16x32_f16 %0, %6, %7, %0\n\t"
            "v_mfma_f32_16x16x32_f16 %1, %6, %8, %1\n\t"
            "v_mfma_f32_16x16x32_f16 %2, %6, %9, %2\n\t"
            "v_mfma_f32_16x16x32_f16 %3, %6, %10, %3\n\t"
            "v_mfma_f32_16x16x32_f16 %4, %6, %11, %4\n\t"
            "v_mfma_f32_16x16x32_f16 %5, %6, %12, %5\n\t"
            "s_nop 7\n\ts_nop 7\n\ts_nop 3"
            : "+a"(acc[tn][0]), "+a"(acc[tn][1]), "+a"(acc[tn][2]), "+a"(acc[tn][3]), "+a"(acc[tn][4]),
              "+a"(acc[tn][5])
            : "v"(b), "v"(f.a[0]), "v"(f.a[1]), "v"(f.a[2]), "v"(f.a[3]), "v"(f.a[4]), "v"(f.a[5]));
    }
}

// The tile product of a 32-deep k-step s of the stage held in (sA, sB), for
// the K tail: the fragments, then the columns as fenced blocks.
template <class S, bool BT = false>
__device__ __forceinline__ void mma16_kstep_fenced(LDS_PTR(const char) sA, LDS_PTR(const char) sB,
                                                   const FragLanes16<S> &fo, int s,
                                                   float4_t (&acc)[S::TN][S::TM]) {
    Frags16<S> f;
#pragma unroll
    for (int r = 0; r < kFragReads16<S, BT>; ++r) frag_read16<S, BT>(f, sA, sB, fo, s, r);
#pragma unroll
    for (int tn = 0; tn < S::TN; ++tn) mfma16_column_fenced<S>(f, tn, acc);
}

// Rows of K past the loop's whole stages, after every wave is done with the
// stages. (1) Rows [64*(kmain/64), kmain) when kmain is not whole stages: one
// stage of direct-to-LDS loads into buffer 0 with every lane's chunk checked
// against kmain and against M or N, then both k-steps. (2) Rows [kmain, K) (1
// to 8 of them, when K or N is not a multiple of 8): one zero-padded 32-deep
// block staged element by element with bounds checks, then one k-step. BT:
// B's rows are those of the transposed B (n, K-contiguous), held like A's.
template <class S, int ASTAGES, bool BT = false>
__device__ __forceinline__ void pipe16_k_tail(const KArgs &a, int m0, int n0, int wave, int lane, int wm0, int wn0,
                                           const FragLanes16<S> &fo, float4_t (&acc)[S::TN][S::TM],
                                           LDS_PTR(char) lds) {
    constexpr int B_REGION = ASTAGES * S::A_BYTES;
    const int tid = threadIdx.x;
    const int kfull = (a.kmain / S::BK) * S::BK;
    if (kfull < a.kmain) {
        barrier_lds();  // no wave reads buffer 0 any more
        const int4_t ra = make_srd(a.A + (int64_t)m0 * a.lda + kfull);
        const int4_t rb = make_srd(BT ? a.B + (int64_t)n0 * a.ldb + kfull : a.B + (int64_t)kfull * a.ldb + n0);
#pragma unroll
        for (int i = 0; i < S::DMA_A; ++i) {
            const ChunkRef c = dma_a_chunk<S>(wave, i, lane);
            const bool in = m0 + c.row < a.M && kfull + 8 * c.chunk < a.kmain;
            p16_dma<BT>(ra, (uint32_t)(uintptr_t)(lds + (wave * S::DMA_A + i) * 1024),
                  in ? (uint32_t)(c.row * a.lda * 2 + c.chunk * 16) : kOOB);
        }
#pragma unroll
        for (int i = 0; i < S::DMA_B; ++i) {
            const ChunkRef c = BT ? dma_bt16_chunk<S>(wave, i, lane) : dma_b16_chunk<S>(wave, i, lane);
            const bool in = BT ? n0 + c.row < a.N && kfull + 8 * c.chunk < a.kmain
                               : kfull + c.row < a.kmain && n0 + 8 * c.chunk < a.N;
            p16_dma<BT>(rb, (uint32_t)(uintptr_t)(lds + B_REGION + (wave * S::DMA_B + i) * 1024),
                  in ? (uint32_t)(c.row * a.ldb * 2 + c.chunk * 16) : kOOB);
        }
        wait_vmcnt<0>();
        barrier_lds();
#pragma unroll
        for (int s = 0; s < S::KSTEPS; ++s) mma16_kstep_fenced<S, BT>(lds, lds + B_REGION, fo, s, acc);
    }
    if (a.kmain < a.K) {
        barrier_lds();
        // A: rows m of the tile, logical chunks 0..3 (k = kmain + 8c .. +7)
        for (int q = tid; q < S::BM * 4; q += S::NT) {
            const int row = q / 4, chunk = q % 4;
            const int m = m0 + row, k = a.kmain + 8 * chunk;
            half8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (m < a.M && k + e < a.K) ? a.A[(int64_t)m * a.lda + k + e] : (_Float16)0.0f;
            *(LDS_PTR(half8_t))(lds + lds_a_offset<S>(row, chunk)) = v;
        }
        if constexpr (BT) {
            // B: rows n of the tile, logical chunks 0..3 (k = kmain + 8c .. +7)
            for (int q = tid; q < S::BN * 4; q += S::NT) {
                const int row = q / 4, chunk = q % 4;
                const int n = n0 + row, k = a.kmain + 8 * chunk;
                half8_t v;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (n < a.N && k + e < a.K) ? a.B[(int64_t)n * a.ldb + k + e] : (_Float16)0.0f;
                *(LDS_PTR(half8_t))(lds + B_REGION + lds_a_offset<S>(row, chunk)) = v;
            }
        } else {
            // B: rows k = kmain .. kmain+31 of the block, all BN columns
            for (int q = tid; q < 32 * S::CB; q += S::NT) {
                const int row = q / S::CB, chunk = q % S::CB;
                const int k = a.kmain + row, n = n0 + 8 * chunk;
                half8_t v;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (k < a.K && n + e < a.N) ? a.B[(int64_t)k * a.ldb + n + e] : (_Float16)0.0f;
                *(LDS_PTR(half8_t))(lds + B_REGION + lds_b16_offset<S>(row, chunk)) = v;
            }
        }
        barrier_lds();
        mma16_kstep_fenced<S, BT>(lds, lds + B_REGION, fo, 0, acc);
    }
}

// One K step is a fixed sequence of KSTEPS*T MFMA slots, T = TM*TN (64), H = T/2:
//   slots 0..H-1      MFMAs H..T-1 of the previous stage's last k-step (f[1]);
//                     after them (not EARLY) the reads of this stage's
//                     k-step-0 fragments into f[0], one per slot;
//   next T per ks     k-steps 0..KSTEPS-2: T MFMAs on f[ks & 1], with the
//                     reads of k-step ks+1 into f[(ks+1) & 1], one per slot;
//   last H slots      MFMAs 0..H-1 of the last k-step (f[1]).
// The direct-to-LDS loads go after slots DOFF, DOFF+SPACING, ...: the tile of
// stage kt+STAGES-1 of B and of stage kt+ASTAGES-1 of A, the operand loaded
// fewer stages ahead first. Then this wave's loads of stage kt+1 are waited
// for and the barrier publishes it (and retires stage kt). EARLY: the wait and
// the barrier come before the last H slots (which read no LDS of stage kt),
// and the reads of stage kt+1's k-step-0 fragments move into those slots.
template <class S, int SPACING, int DOFF, int ASTAGES, bool EARLY, bool BT = false, bool BROWS = false>
__device__ __forceinline__ void pipe16_tile(const KArgs &a, int tm_idx, int tn_idx, LDS_PTR(char) lds) {
    constexpr int T = S::TM * S::TN;
    constexpr int H = T / 2;
    static_assert(T % 2 == 0 && S::KSTEPS % 2 == 0, "the last k-step of a stage must use f[1]");
    static_assert(!BT || S::BN * S::RA == S::B_BYTES, "a transposed B tile fills the B buffer like an A tile");
    constexpr int READS = kFragReads16<S, BT>;
    static_assert(READS <= H, "fragment reads must fit under half the MFMAs of a k-step");
    constexpr int LOADS = S::DMA_A + S::DMA_B;
    constexpr int AHEAD = S::STAGES - 1;
    constexpr int AHEAD_A = ASTAGES - 1;
    static_assert(ASTAGES >= S::STAGES - 1 && ASTAGES <= S::STAGES + 1, "A and B differ by at most one buffer");
    constexpr bool B_FIRST = ASTAGES > S::STAGES;
    constexpr int WAIT = (AHEAD_A - 1) * S::DMA_A + (AHEAD - 1) * S::DMA_B;
    constexpr int SLOTS = S::KSTEPS * T;
    static_assert(AHEAD >= 1 && AHEAD_A >= 1 && WAIT < 64, "vmcnt range");
    static_assert(DOFF + (LOADS - 1) * SPACING < (EARLY ? SLOTS - H : SLOTS), "loads must be issued before the stage's wait");
    constexpr int B_REGION = ASTAGES * S::A_BYTES;
    static_assert(pipe16_lds_bytes<S, ASTAGES>() <= 160 * 1024, "LDS of one work-group");
    static_assert(S::WAVES * S::WTM * S::WTN * 2 <= pipe16_lds_bytes<S, ASTAGES>(), "the C tile fits the LDS");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
    const int m0 = tm_idx * S::BM, n0 = tn_idx * S::BN;
    // The loop covers the whole 64-deep stages of K's rows [0, kmain); kmain
    // is K, or the largest multiple of 8 below K when K or N is not a
    // multiple of 8 (then no 16-byte chunk the loads fetch crosses the end of
    // an A row, and a chunk crossing column N of B reads into the next row,
    // whose values reach only columns >= N, which are never stored). The rows
    // past the last whole stage are added after the loop (pipe16_k_tail).
    const int nk = a.kmain / S::BK;

    // Loads. A: load i of this wave covers LDS slab (wave*DMA_A + i), rows
    // 8*slab .. +7 of the tile; its descriptor starts at the slab's first row
    // and ends after row M - 1 (rows past M read zeros), and the lane's offset
    // inside the slab depends only on the slab's parity (p16_a_lane_bytes). B:
    // load i covers slab (wave*DMA_B + i), rows 2*slab and 2*slab + 1 of the
    // stage; the slab's start is the instruction's scalar offset, and the
    // lane's offset (kOOB for a column chunk past N) takes one of four forms,
    // by the slab's swizzle pattern (p16_b_lane_bytes). BT: B's slabs are
    // laid out and read like A's, over the rows n of the transposed B; in a
    // tile whose rows all lie inside N one descriptor per stage serves them,
    // each slab's start the scalar offset, and only the tile that holds row
    // N (BROWS) gives each slab A's kind of descriptor, ending after row
    // N - 1 (a descriptor per slab everywhere spilled 61 scalar registers
    // instead of 20 at 256 x 256: 8192^3 907 vs 823 us).
    uint32_t voff_a[2], voff_b[BT ? 2 : 4];
#pragma unroll
    for (int q = 0; q < 2; ++q) voff_a[q] = (uint32_t)p16_a_lane_bytes<S>(lane, q, a.lda);
#pragma unroll
    for (int q = 0; q < (BT ? 2 : 4); ++q) {
        const int64_t o = BT ? p16_a_lane_bytes<S>(lane, q, a.ldb) : p16_b_lane_bytes<S>(lane, q, n0, a.N, a.ldb);
        voff_b[q] = o < 0 ? kOOB : (uint32_t)o;
    }
    uint32_t nrec_a[S::DMA_A];  // bytes of the slab's rows inside M
#pragma unroll
    for (int i = 0; i < S::DMA_A; ++i) {
        const int64_t rows = (int64_t)a.M - m0 - (int64_t)(wave * S::DMA_A + i) * 8;
        const int64_t bytes = rows <= 0 ? 0 : rows * a.lda * 2;
        nrec_a[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(bytes > (int64_t)kRange ? (int64_t)kRange : bytes));
    }
    uint32_t nrec_b[BROWS ? S::DMA_B : 1];  // BROWS: bytes of the slab's rows inside N
#pragma unroll
    for (int i = 0; i < (BROWS ? S::DMA_B : 0); ++i) {
        const int64_t rows = (int64_t)a.N - n0 - (int64_t)(wave * S::DMA_B + i) * 8;
        const int64_t bytes = rows <= 0 ? 0 : rows * a.ldb * 2;
        nrec_b[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(bytes > (int64_t)kRange ? (int64_t)kRange : bytes));
    }
    const _Float16 *a_tile = a.A + (int64_t)m0 * a.lda;
    const _Float16 *b_tile = BT ? a.B + (int64_t)n0 * a.ldb : a.B + n0;
    FragLanes16<S> fo;
    fo.a[0] = (uint32_t)frag_a16_lane<S>(wm0, 0, lane);
    fo.a[1] = (uint32_t)frag_a16_lane<S>(wm0, 1, lane);
    if constexpr (BT) {
        fo.b[0] = (uint32_t)frag_a16_lane<S>(wn0, 0, lane);
        fo.b[1] = (uint32_t)frag_a16_lane<S>(wn0, 1, lane);
    } else {
#pragma unroll
        for (int tn = 0; tn < S::TN; ++tn) fo.b[tn] = (uint32_t)frag_b16_lane<S>(wn0, tn, lane);
    }

    // Load j of stage kt into buffer buf of its operand; past the end of K
    // the descriptor's range is 0 bytes, so every lane writes zeros.
    auto dma = [&](int j, int kt, int buf) {
        const int k0 = kt * S::BK;
        if (j < S::DMA_A) {
            const int slab = wave * S::DMA_A + j;
            int4_t r = make_srd(a_tile + (int64_t)slab * 8 * a.lda + k0);
            r[2] = kt < nk ? (int)nrec_a[j] : 0;
            p16_dma<BROWS>(r, (uint32_t)(uintptr_t)(lds + buf * S::A_BYTES + slab * 1024), voff_a[slab % 2]);
        } else if constexpr (BROWS) {
            const int slab = wave * S::DMA_B + (j - S::DMA_A);
            int4_t r = make_srd(b_tile + (int64_t)slab * 8 * a.ldb + k0);
            r[2] = kt < nk ? (int)nrec_b[BROWS ? j - S::DMA_A : 0] : 0;
            p16_dma<BROWS>(r, (uint32_t)(uintptr_t)(lds + B_REGION + buf * S::B_BYTES + slab * 1024), voff_b[slab % 2]);
        } else if constexpr (BT) {
            const int slab = wave * S::DMA_B + (j - S::DMA_A);
            int4_t r = make_srd(b_tile + k0);
            if (kt >= nk) r[2] = 0;
            p16_dma_soff<BROWS>(r, (uint32_t)(uintptr_t)(lds + B_REGION + buf * S::B_BYTES + slab * 1024),
                                voff_b[slab % 2], (uint32_t)(slab * 8 * a.ldb * 2));
        } else {
            const int slab = wave * S::DMA_B + (j - S::DMA_A);
            int4_t r = make_srd(b_tile + (int64_t)k0 * a.ldb);
            if (kt >= nk) r[2] = 0;
            dma16_soff(r, (uint32_t)(uintptr_t)(lds + B_REGION + buf * S::B_BYTES + slab * 1024),
                       voff_b[p16_b_pattern(slab)], (uint32_t)p16_b_slab_bytes(slab, a.ldb));
        }
    };

    float4_t acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // f[1] starts at zero: the first step's first H slots add 0 * 0.
    Frags16<S> f[2];
#pragma unroll
    for (int t = 0; t < S::TN; ++t) {
        f[1].blo[t] = short4_t{0, 0, 0, 0};
        f[1].bhi[t] = short4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < S::TM; ++t) f[1].a[t] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};

#pragma unroll
    for (int s = 0; s < (AHEAD_A > AHEAD ? AHEAD_A : AHEAD); ++s) {
        if (B_FIRST && s < AHEAD)
#pragma unroll
            for (int j = S::DMA_A; j < LOADS; ++j) dma(j, s, s);
        if (s < AHEAD_A)
#pragma unroll
            for (int j = 0; j < S::DMA_A; ++j) dma(j, s, s);
        if (!B_FIRST && s < AHEAD)
#pragma unroll
            for (int j = S::DMA_A; j < LOADS; ++j) dma(j, s, s);
    }
    wait_vmcnt<WAIT>();
    barrier_lds();
    if (EARLY) {
#pragma unroll
        for (int r = 0; r < READS; ++r) frag_read16<S, BT>(f[0], lds, lds + B_REGION, fo, 0, r);
    }

    int bbuf = 0, abuf = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int nbbuf = bbuf == 0 ? S::STAGES - 1 : bbuf - 1;
        const int nabuf = abuf == 0 ? ASTAGES - 1 : abuf - 1;
        LDS_PTR(const char) sA = lds + abuf * S::A_BYTES;
        LDS_PTR(const char) sB = lds + B_REGION + bbuf * S::B_BYTES;
        LDS_PTR(const char) sA1 = lds + (abuf == ASTAGES - 1 ? 0 : abuf + 1) * S::A_BYTES;
        LDS_PTR(const char) sB1 = lds + B_REGION + (bbuf == S::STAGES - 1 ? 0 : bbuf + 1) * S::B_BYTES;
        TLG_SCHED_FENCE16();
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) {
            if (q < H) {
                mfma16_tile<S>(f[1], H + q, acc);
                if (!EARLY && q < READS) frag_read16<S, BT>(f[0], sA, sB, fo, 0, q);
            } else if (q < H + (S::KSTEPS - 1) * T) {
                const int ks = (q - H) / T, i = (q - H) % T;
                mfma16_tile<S>(f[ks & 1], i, acc);
                if (i < READS) frag_read16<S, BT>(f[(ks + 1) & 1], sA, sB, fo, ks + 1, i);
            } else {
                const int u = q - H - (S::KSTEPS - 1) * T;
                if (EARLY && u == 0) {
                    wait_vmcnt<WAIT>();  // this wave's loads of stage kt+1 are in LDS
                    barrier_lds();       // ... and every wave's; no wave reads stage kt any more
                }
                mfma16_tile<S>(f[1], u, acc);
                if (EARLY && u < READS) frag_read16<S, BT>(f[0], sA1, sB1, fo, 0, u);
            }
            if (q >= DOFF && (q - DOFF) % SPACING == 0 && (q - DOFF) / SPACING < LOADS) {
                const int n = (q - DOFF) / SPACING;
                const int j = !B_FIRST ? n : n < S::DMA_B ? S::DMA_A + n : n - S::DMA_B;
                if (j < S::DMA_A)
                    dma(j, kt + AHEAD_A, nabuf);
                else
                    dma(j, kt + AHEAD, nbbuf);
            }
            TLG_SCHED_FENCE16();
        }
        if (!EARLY) {
            wait_vmcnt<WAIT>();
            barrier_lds();
        }
        bbuf = bbuf == S::STAGES - 1 ? 0 : bbuf + 1;
        abuf = abuf == ASTAGES - 1 ? 0 : abuf + 1;
    }
#pragma unroll
    for (int i = H; i < T; ++i) mfma16_tile<S>(f[1], i, acc);
    wait_vmcnt<0>();  // no load may still be writing LDS
    if (nk * S::BK < a.K) pipe16_k_tail<S, ASTAGES, BT>(a, m0, n0, wave, lane, wm0, wn0, fo, acc, lds);
    mfma16_results_ready();
    barrier_lds();  // every wave is done with the stages
    store_c_tile16_lds<S>(a, m0, n0, wave, lane, acc, lds);
}

template <class S, int SPACING, int DOFF, int ASTAGES, bool EARLY, bool BT = false>
__global__ __launch_bounds__(S::NT) void k_tiled_pipe16(const KArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[pipe16_lds_bytes<S, ASTAGES>()];
    int tm_idx, tn_idx;
    grouped_tile(xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n), a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    if (BT && (tn_idx + 1) * S::BN > a.N)
        pipe16_tile<S, SPACING, DOFF, ASTAGES, EARLY, BT, BT>(a, tm_idx, tn_idx, (LDS_PTR(char))smem);
    else
        pipe16_tile<S, SPACING, DOFF, ASTAGES, EARLY, BT>(a, tm_idx, tn_idx, (LDS_PTR(char))smem);
}

// Several problems in one launch: work-group ids are dealt to the XCDs as in
// the single-problem kernel, then split by problem in order (tile_start holds
// the running tile counts), each problem's tiles in its own grouped order.
template <class S, int SPACING, int DOFF, int ASTAGES, bool EARLY, bool BT = false>
__global__ __launch_bounds__(S::NT) void k_tiled_pipe16_grouped(const GroupArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem[pipe16_lds_bytes<S, ASTAGES>()];
    const int v = xcd_remap(blockIdx.x, g.tile_start[g.count]);
    int p = 0;
    while (p + 1 < g.count && v >= g.tile_start[p + 1]) ++p;
    const KArgs &a = g.p[p];
    int tm_idx, tn_idx;
    grouped_tile(v - g.tile_start[p], a.tiles_m, a.tiles_n, a.group_m, &tm_idx, &tn_idx);
    if (BT && (tn_idx + 1) * S::BN > a.N)
        pipe16_tile<S, SPACING, DOFF, ASTAGES, EARLY, BT, BT>(a, tm_idx, tn_idx, (LDS_PTR(char))smem);
    else
        pipe16_tile<S, SPACING, DOFF, ASTAGES, EARLY, BT>(a, tm_idx, tn_idx, (LDS_PTR(char))smem);
}

using Pipe16w4 = TileShape16<256, 256, 64, 2, 2, 2>;    // four waves of 128 x 128, two B buffers
using Pipe16w4B3 = TileShape16<256, 256, 64, 2, 2, 3>;  // three B buffers
// 128 x 256 tiles, four waves of 128 x 64: twice the tiles of 256 x 256 for
// problems that would leave CUs idle at that size
using Pipe16h = TileShape16<128, 256, 64, 1, 4, 3>;
// eight waves of 128 x 64 (two per SIMD, 128 accumulators each)
using Pipe16w8 = TileShape16<256, 256, 64, 2, 4, 2>;
// 192 x 256 tiles, four waves of 96 x 128 (14 loads per wave and stage over
// a 96-slot step)
using Pipe16t = TileShape16<192, 256, 64, 2, 2, 2>;

template <class S, bool BT = false>
static KArgs pipe16_args(const Problem &p) {
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
    // BT: a chunk must not cross the end of a row of the transposed B (K
    // only); otherwise the end of an A row (K) or column N of B
    a.kmain = p.K % 8 == 0 && (BT || p.N % 8 == 0) ? (int)p.K : (int)(8 * ((p.K - 1) / 8));
    a.tiles_m = (a.M + S::BM - 1) / S::BM;
    a.tiles_n = (a.N + S::BN - 1) / S::BN;
    return a;
}

template <class S, int SPACING, int DOFF, int ASTAGES, bool EARLY, bool BT = false>
static hipError_t launch_pipe16_t(const Problem &p, hipStream_t stream) {
    if (p.trans_b != BT) return hipErrorInvalidValue;
    const KArgs a = pipe16_args<S, BT>(p);
    hipLaunchKernelGGL((k_tiled_pipe16<S, SPACING, DOFF, ASTAGES, EARLY, BT>), dim3((unsigned)(a.tiles_m * a.tiles_n)),
                       dim3(S::NT), 0, stream, a);
    return hipGetLastError();
}

// The default configuration (four waves, loads every eight MFMA slots) over
// up to kGroupMax problems, all with the same trans_b.
template <bool BT>
static hipError_t launch_pipe16_grouped_t(const Problem *ps, int count, hipStream_t stream) {
    using S = Pipe16w4;
    static_assert(sizeof(GroupArgs) <= 4096, "kernel arguments");
    GroupArgs g;
    g.count = count;
    g.tile_start[0] = 0;
    for (int i = 0; i < count; ++i) {
        g.p[i] = pipe16_args<S, BT>(ps[i]);
        g.tile_start[i + 1] = g.tile_start[i] + g.p[i].tiles_m * g.p[i].tiles_n;
    }
    if (g.tile_start[count] == 0) return hipSuccess;
    hipLaunchKernelGGL((k_tiled_pipe16_grouped<S, 8, 1, 3, false, BT>), dim3((unsigned)g.tile_start[count]),
                       dim3(S::NT), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_tiled_pipe16_grouped(const Problem *ps, int count, hipStream_t stream) {
    if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
    const bool bt = ps[0].trans_b;
    for (int i = 1; i < count; ++i)
        if (ps[i].trans_b != bt) return hipErrorInvalidValue;
    return bt ? launch_pipe16_grouped_t<true>(ps, count, stream) : launch_pipe16_grouped_t<false>(ps, count, stream);
}

hipError_t launch_tiled_pipe16(int config, const Problem &p, hipStream_t stream) {
    if (p.trans_b) {
        switch (config) {
            case PIPE16_256x256x64_A3_SP8: return launch_pipe16_t<Pipe16w4, 8, 1, 3, false, true>(p, stream);
            case PIPE16_128x256x64_A3: return launch_pipe16_t<Pipe16h, 4, 1, 3, false, true>(p, stream);
            case PIPE16_192x256x64_A3_SP6: return launch_pipe16_t<Pipe16t, 6, 1, 3, false, true>(p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (config) {
        // 16 loads per wave and stage, every four slots from slot 1 (the
        // 128-slot step leaves its last 64 slots free of loads)
        case PIPE16_256x256x64_A3: return launch_pipe16_t<Pipe16w4, 4, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_A3_EARLY: return launch_pipe16_t<Pipe16w4, 4, 1, 3, true>(p, stream);
        case PIPE16_256x256x64_B3: return launch_pipe16_t<Pipe16w4B3, 4, 1, 2, false>(p, stream);
        // the same loads every two or every six slots
        case PIPE16_256x256x64_A3_SP2: return launch_pipe16_t<Pipe16w4, 2, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_A3_SP6: return launch_pipe16_t<Pipe16w4, 6, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_A3_EARLY_SP2: return launch_pipe16_t<Pipe16w4, 2, 1, 3, true>(p, stream);
        case PIPE16_256x256x64_A3_SP7: return launch_pipe16_t<Pipe16w4, 7, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_A3_SP8: return launch_pipe16_t<Pipe16w4, 8, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_A3_SP6_D5: return launch_pipe16_t<Pipe16w4, 6, 5, 3, false>(p, stream);
        case PIPE16_256x256x64_B3_SP6: return launch_pipe16_t<Pipe16w4B3, 6, 1, 2, false>(p, stream);
        case PIPE16_256x256x64_A3_EARLY_SP6: return launch_pipe16_t<Pipe16w4, 6, 1, 3, true>(p, stream);
        // 12 loads per wave and stage over the 64-slot step
        case PIPE16_128x256x64_A3: return launch_pipe16_t<Pipe16h, 4, 1, 3, false>(p, stream);
        case PIPE16_128x256x64_A4: return launch_pipe16_t<Pipe16h, 4, 1, 4, false>(p, stream);
        // eight waves: 8 loads per wave and stage over the 64-slot step
        case PIPE16_256x256x64_W8_A3_SP8: return launch_pipe16_t<Pipe16w8, 8, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_W8_A3_SP4: return launch_pipe16_t<Pipe16w8, 4, 1, 3, false>(p, stream);
        case PIPE16_256x256x64_W8_A3_EARLY_SP6: return launch_pipe16_t<Pipe16w8, 6, 1, 3, true>(p, stream);
        case PIPE16_192x256x64_A3_SP6: return launch_pipe16_t<Pipe16t, 6, 1, 3, false>(p, stream);
        case PIPE16_192x256x64_A3_SP7: return launch_pipe16_t<Pipe16t, 7, 1, 3, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tlg
