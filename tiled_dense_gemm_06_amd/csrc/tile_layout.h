// Index arithmetic of the gfx950 GEMM+ReLU kernels: tile shapes, the LDS
// swizzles, which global chunk each lane of a direct-to-LDS load fetches,
// where each MFMA operand fragment is read from, and which C elements each
// lane owns. Everything here is plain integer arithmetic, usable from the
// kernels and from host-side emulation of the kernels' data movement.
//
// Tiling follows the quick-start kernel of the TileLang article
// (aiwiki.ai/wiki/tilelang, "Programming model"): one work-group per output
// tile, a K loop over shared-memory (LDS) tiles of A and B, an fp32
// accumulator fragment in registers, ReLU and the fp16 copy-out at the end.
// Shapes and layouts here are chosen for gfx950, not taken from that kernel.
//
// Facts about gfx950 this file relies on (measured on the device):
//  * v_mfma_f32_32x32x16_f16: lane l holds, for its first operand, row
//    (l % 32) and k = 8*(l/32) + e (e = 0..7); for the second operand,
//    column (l % 32) and the same k; result element r of lane l is row
//    8*(r/4) + 4*(l/32) + (r%4), column (l % 32).
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives
//    element (i % 4) of the 8-byte chunks addressed by lanes i/4 + 4*j,
//    j = 0..3. If lane s addresses row (k0 + s/4), columns n0 + 4*(s%4) .. +3
//    of a row-major (k, n) tile, lane i receives B[k0 + j][n0 + i], j = 0..3.
//  * buffer_load_dwordx4 ... lds writes lane t's 16 bytes at M0 + 16*t and
//    writes zeros for a lane whose offset is out of the buffer's range.
//  * LDS has 64 banks of 4 bytes: a ds_read_b128 is conflict-free when every
//    16 consecutive lanes touch 16 different 16-byte slots of a 256-byte
//    window; a ds_read_b64_tr_b16 when every 32 consecutive lanes do.
#ifndef TLG_TILE_LAYOUT_H
#define TLG_TILE_LAYOUT_H

#include <stdint.h>

#if defined(__HIPCC__)
#define TLG_HD __host__ __device__ __forceinline__
#else
#define TLG_HD inline
#endif

namespace tlg {

TLG_HD constexpr int imin(int a, int b) { return a < b ? a : b; }
TLG_HD constexpr int imax(int a, int b) { return a > b ? a : b; }

// Output tile BM x BN, K step BK, WM x WN waves (64 lanes each), STAGES LDS
// buffers. Each wave owns a (BM/WM) x (BN/WN) block of C made of 32 x 32
// MFMA tiles.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct TileShape {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
    static constexpr int WAVES = WM * WN, NT = WAVES * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;   // per-wave extents
    static constexpr int TM = WTM / 32, TN = WTN / 32;   // MFMA tiles per wave
    static constexpr int RA = BK * 2, RB = BN * 2;       // LDS row bytes of the A and B tiles
    static constexpr int CA = BK / 8, CB = BN / 8;       // 16-byte chunks per row
    static constexpr int A_BYTES = BM * RA, B_BYTES = BK * RB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGE_BYTES * STAGES;
    static constexpr int ROWS_A_SLAB = 1024 / RA, ROWS_B_SLAB = 1024 / RB; // rows per 1 KiB load
    static constexpr int SLABS_A = A_BYTES / 1024, SLABS_B = B_BYTES / 1024;
    static constexpr int DMA_A = SLABS_A / WAVES, DMA_B = SLABS_B / WAVES; // loads per wave per stage
    static constexpr int KSTEPS = BK / 16;                // MFMA k-steps per stage
    // register-staged loading: 16-byte chunks per thread per stage
    static constexpr int JA = BM * CA / NT, JB = BK * CB / NT;

    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be whole 32x32 MFMA tiles");
    static_assert(BK % 16 == 0 && BK >= 16, "BK must be a multiple of the MFMA k (16)");
    static_assert(RA <= 1024 && RB <= 1024 && 1024 % RA == 0 && 1024 % RB == 0, "rows must pack 1 KiB loads");
    static_assert(SLABS_A % WAVES == 0 && SLABS_B % WAVES == 0, "1 KiB loads must split evenly over waves");
    static_assert(CB >= 4, "BN must be at least 32");
    static_assert((BM * CA) % NT == 0 && (BK * CB) % NT == 0, "chunks must split evenly over threads");
};

// ---- LDS swizzles (16-byte granularity) ----
// A tile: rows of RA bytes, K-contiguous. Chunk c of row r is stored at chunk
// position c ^ swz_a(r). Sixteen consecutive rows read at one logical chunk
// land in 16 distinct 16-byte slots of a 256-byte bank window.
TLG_HD constexpr int swz_a(int r, int CA) {
    return (r / imax(1, 16 / CA)) % imin(CA, 16);
}
// B tile: rows of RB bytes (one k each), N-contiguous. Chunk c of row k is
// stored at chunk position c ^ swz_b(k). The four rows x four chunks read by
// 32 lanes of one transposing read land in 16 distinct slots.
TLG_HD constexpr int swz_b(int k, int CB) {
    return 4 * ((k / imax(1, 16 / CB)) & (imin(CB, 16) / 4 - 1));
}

// ---- direct-to-LDS loads ----
// Load i (0 <= i < DMA_A) of wave w fills LDS slab (w*DMA_A + i) of the A
// tile: 1 KiB holding rows [slab*ROWS_A_SLAB, +ROWS_A_SLAB). Lane t writes
// chunk position t % CA of row slab*ROWS_A_SLAB + t / CA, so it fetches the
// logical chunk (t % CA) ^ swz_a(row), i.e. columns k0 + 8*chunk .. +7.
struct ChunkRef {
    int row;    // row inside the tile (A: m, B: k)
    int chunk;  // logical 16-byte chunk inside the row
};
template <class S>
TLG_HD ChunkRef dma_a_chunk(int wave, int i, int lane) {
    int slab = wave * S::DMA_A + i;
    int row = slab * S::ROWS_A_SLAB + lane / S::CA;
    int pos = lane % S::CA;
    return ChunkRef{row, pos ^ swz_a(row, S::CA)};
}
template <class S>
TLG_HD ChunkRef dma_b_chunk(int wave, int i, int lane) {
    int slab = wave * S::DMA_B + i;
    int row = slab * S::ROWS_B_SLAB + lane / S::CB;
    int pos = lane % S::CB;
    return ChunkRef{row, pos ^ swz_b(row, S::CB)};
}
// LDS byte offset (inside a stage's A or B tile) of logical chunk c of row r.
template <class S>
TLG_HD int lds_a_offset(int r, int c) { return r * S::RA + 16 * (c ^ swz_a(r, S::CA)); }
template <class S>
TLG_HD int lds_b_offset(int k, int c) { return k * S::RB + 16 * (c ^ swz_b(k, S::CB)); }

// Register-staged loading: job j of thread t covers chunk q = t + j*NT.
template <class S>
TLG_HD ChunkRef reg_a_chunk(int tid, int j) {
    int q = tid + j * S::NT;
    return ChunkRef{q / S::CA, q % S::CA};
}
template <class S>
TLG_HD ChunkRef reg_b_chunk(int tid, int j) {
    int q = tid + j * S::NT;
    return ChunkRef{q / S::CB, q % S::CB};
}

// ---- MFMA operand fragments ----
// The kernels compute the transposed tile D = B^T A^T with
// v_mfma_f32_32x32x16_f16: the first operand comes from the B tile (its rows
// are output columns n), the second from the A tile (output rows m). Then
// each lane's four consecutive result registers are four consecutive n of
// one row m, which become one 8-byte store.
//
// Second operand (A tile), MFMA tile tm of a wave whose rows start at wm0,
// k-step s: lane l reads 16 bytes = A[wm0 + 32*tm + l%32][16*s + 8*(l/32) .. +7].
template <class S>
TLG_HD int frag_a_offset(int wm0, int tm, int s, int lane) {
    int r = wm0 + 32 * tm + lane % 32;
    int c = 2 * s + lane / 32;
    return lds_a_offset<S>(r, c);
}
// First operand (B tile), MFMA tile tn of a wave whose columns start at wn0,
// k-step s, half h (0: k 0..3 of the lane's 8, 1: k 4..7): the 8-byte
// address lane l supplies to ds_read_b64_tr_b16. After the read, lane l holds
// B[16*s + 8*(l/32) + 4*h + j][wn0 + 32*tn + l%32] for j = 0..3.
template <class S>
TLG_HD int frag_b_offset(int wn0, int tn, int s, int h, int lane) {
    int g = lane / 16, i = lane % 16;
    int k = 16 * s + 8 * (g / 2) + 4 * h + i / 4;
    int n = wn0 + 32 * tn + 16 * (g % 2) + 4 * (i % 4);
    return lds_b_offset<S>(k, n / 8) + 2 * (n % 8);
}

// ---- result ownership ----
// Result register r of MFMA tile (tn, tm) in lane l is C[m][n] with
// m = wm0 + 32*tm + l%32 and n = wn0 + 32*tn + 8*(r/4) + 4*(l/32) + r%4.
TLG_HD int acc_m(int wm0, int tm, int lane) { return wm0 + 32 * tm + lane % 32; }
TLG_HD int acc_n(int wn0, int tn, int r, int lane) {
    return wn0 + 32 * tn + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
}

// ---- epilogue through LDS ----
// A wave's block of C (WTM x WTN fp16) in LDS: rows of 2*WTN bytes (CH =
// WTN/8 pieces of 16 bytes), the piece c (columns 8c .. 8c+7) of row r at
// piece position c ^ ((r / (16/CH)) % CH). A 256-byte bank window holds
// 16/CH rows, so writes of 16 lanes (16 rows, one c) and reads of 16 lanes
// (16/CH consecutive rows, all their pieces) touch 16 distinct 16-byte slots
// of a window (CH = 4, 8 or 16).
template <class S>
TLG_HD int epi_lds_offset(int row, int c) {
    constexpr int CH = S::WTN / 8;
    return row * S::WTN * 2 + 16 * (c ^ ((row / (16 / CH)) % CH));
}
// After the lane-pair exchange, lane l holds piece pr (0 or 1) of MFMA tile
// (tn, tm): row 32*tm + l%32 of the wave block, piece 4*tn + 2*pr + l/32.
TLG_HD int epi_piece_row(int tm, int lane) { return 32 * tm + lane % 32; }
TLG_HD int epi_piece_index(int tn, int pr, int lane) { return 4 * tn + 2 * pr + lane / 32; }
// Read-back instruction k: lane l takes piece l % (WTN/8) of row
// k * (64 / (WTN/8)) + l / (WTN/8).
template <class S>
TLG_HD int epi_read_row(int k, int lane) { return k * (64 / (S::WTN / 8)) + lane / (S::WTN / 8); }
template <class S>
TLG_HD int epi_read_piece(int lane) { return lane % (S::WTN / 8); }

// ---- tiles of v_mfma_f32_16x16x32_f16 ----
// Facts relied on (same conventions as for the 32 x 32 instruction above):
// lane l holds, for its first operand, row (l % 16) and k = 8*(l/16) + e
// (e = 0..7); for its second operand, column (l % 16) and the same k; result
// element r of lane l is row 4*(l/16) + r, column (l % 16).
// The kernels again compute D = B^T A^T: the first operand comes from the B
// tile (output columns n), the second from the A tile (output rows m), so
// each lane's four result registers are four consecutive n of one row m.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct TileShape16 : TileShape<BM_, BN_, BK_, WM_, WN_, STAGES_> {
    using Base = TileShape<BM_, BN_, BK_, WM_, WN_, STAGES_>;
    static constexpr int TM = Base::WTM / 16, TN = Base::WTN / 16;  // MFMA tiles per wave
    static constexpr int KSTEPS = BK_ / 32;                          // 32-deep k-steps per stage
    static_assert(BK_ % 32 == 0, "BK must be a multiple of the MFMA k (32)");
    static_assert(Base::CB == 32, "the B swizzle below is written for 256-column B tiles");
};
// B tile swizzle for the 16 x 16 fragments: chunk c of row k at position
// c ^ swz_b16(k). A transposing read by 32 lanes covers rows 8g + 4h + q
// (g = 0, 1; q = 0..3) and two adjacent chunks; (q, g) select 8 distinct even
// offsets 4q ^ 2g, so the 32 lanes land in 16 distinct slots of a 256-byte
// window. Direct-to-LDS writes are linear, so any XOR swizzle suits them.
TLG_HD constexpr int swz_b16(int k) { return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)); }
template <class S>
TLG_HD int lds_b16_offset(int k, int c) { return k * S::RB + 16 * (c ^ swz_b16(k)); }
// A transposed B (N x K, rows of n with 64 k per stage) is held like the A
// tile: load i of wave w covers slab (w*DMA_B + i), rows 8*slab .. +7 (the
// same number of 1 KiB loads as a 256-column B tile).
template <class S>
TLG_HD ChunkRef dma_bt16_chunk(int wave, int i, int lane) {
    int slab = wave * S::DMA_B + i;
    int row = slab * S::ROWS_A_SLAB + lane / S::CA;
    int pos = lane % S::CA;
    return ChunkRef{row, pos ^ swz_a(row, S::CA)};
}
template <class S>
TLG_HD ChunkRef dma_b16_chunk(int wave, int i, int lane) {
    int slab = wave * S::DMA_B + i;
    int row = slab * S::ROWS_B_SLAB + lane / S::CB;
    int pos = lane % S::CB;
    return ChunkRef{row, pos ^ swz_b16(row)};
}
// The 16 x 16 x 32 pipelined kernel computes its load offsets once per lane
// (a stage changes only the buffer descriptor's base). A slab (8 rows of 64
// k, the rows of load dma_a_chunk(wave, i, lane)): the lane's byte offset from
// the slab's first row depends on the slab's parity q alone, since the
// swizzle of rows 16 apart repeats. B slab (2 rows of 256 n,
// dma_b16_chunk): the slab's start is the instruction's scalar offset
// (p16_b_slab_bytes), and the lane's offset inside the slab takes one of
// four forms, by the swizzle pattern of the slab's rows (p16_b_pattern); a
// chunk that starts at or past column N gets -1 (the kernel's out-of-range
// offset).
template <class S>
TLG_HD int64_t p16_a_lane_bytes(int lane, int q, int64_t lda) {
    static_assert(S::CA == 8 && S::ROWS_A_SLAB == 8, "64-deep A rows");
    return (int64_t)(lane / 8) * lda * 2 + 16 * ((lane % 8) ^ ((4 * q + lane / 16) % 8));
}
TLG_HD constexpr int p16_b_pattern(int slab) { return (slab % 2) + 2 * ((slab / 4) % 2); }
template <class S>
TLG_HD int64_t p16_b_lane_bytes(int lane, int pattern, int n0, int N, int64_t ldb) {
    static_assert(S::CB == 32 && S::ROWS_B_SLAB == 2, "256-column B rows");
    const int k = 2 * (pattern % 2) + 8 * (pattern / 2) + lane / 32;  // a row with the pattern's swizzle
    const int chunk = (lane % 32) ^ swz_b16(k);
    return n0 + 8 * chunk < N ? (int64_t)(lane / 32) * ldb * 2 + 16 * chunk : -1;
}
TLG_HD int64_t p16_b_slab_bytes(int slab, int64_t ldb) { return (int64_t)slab * 2 * ldb * 2; }
// Second operand (A tile), MFMA tile tm, 32-deep k-step s: lane l reads 16
// bytes = A[wm0 + 16*tm + l%16][32*s + 8*(l/16) .. +7].
template <class S>
TLG_HD int frag_a16_offset(int wm0, int tm, int s, int lane) {
    return lds_a_offset<S>(wm0 + 16 * tm + lane % 16, 4 * s + lane / 16);
}
// First operand (B tile), MFMA tile tn, k-step s, half h: the 8-byte address
// lane l supplies to ds_read_b64_tr_b16. After the read, lane l holds
// B[32*s + 8*(l/16) + 4*h + j][wn0 + 16*tn + l%16] for j = 0..3.
template <class S>
TLG_HD int frag_b16_offset(int wn0, int tn, int s, int h, int lane) {
    int g = lane / 16, i = lane % 16;
    int k = 32 * s + 8 * g + 4 * h + i / 4;
    int n = wn0 + 16 * tn + 4 * (i % 4);
    return lds_b16_offset<S>(k, n / 8) + 2 * (n % 8);
}
// The same offsets split into a per-lane part and a constant (for 64-deep
// A rows and 256-column B rows, wm0 and wn0 multiples of 128): the A swizzle
// of rows 16 apart is the same, so frag_a16_offset(wm0, tm, s, lane) =
// frag_a16_lane(wm0, s, lane) + tm * 16 * RA; the B swizzle depends on the
// lane alone, so frag_b16_offset(wn0, tn, s, h, lane) =
// frag_b16_lane(wn0, tn, lane) + (32*s + 4*h) * RB. A kernel keeps the lane
// parts in registers and the constants go into the LDS instructions' offset
// field.
template <class S>
TLG_HD int frag_a16_lane(int wm0, int s, int lane) {
    static_assert(S::CA == 8, "64-deep A rows");
    const int g = lane / 16, w = (lane % 16) / 2;
    return (wm0 + lane % 16) * S::RA + 16 * ((g ^ w) & 3) + 64 * (s ^ (w >> 2));
}
template <class S>
TLG_HD int frag_b16_lane(int wn0, int tn, int lane) {
    static_assert(S::CB == 32, "256-column B rows");
    return frag_b16_offset<S>(wn0, tn, 0, 0, lane);
}
// Result register r of MFMA tile (tn, tm) in lane l is C[m][n] with
// m = wm0 + 16*tm + l%16 and n = wn0 + 16*tn + 4*(l/16) + r.
TLG_HD int acc16_m(int wm0, int tm, int lane) { return wm0 + 16 * tm + lane % 16; }
TLG_HD int acc16_n(int wn0, int tn, int r, int lane) { return wn0 + 16 * tn + 4 * (lane / 16) + r; }
// Epilogue block of a wave (WTM x WTN fp16, rows of 2*WTN bytes; 16 pieces of
// 16 bytes per row for WTN = 128, 8 for WTN = 64): piece c of row r at
// position c ^ (r % 16), or c ^ ((r / 2) % 8) when two rows share a 256-byte
// window. The 8-byte result pieces of 16 rows written by one instruction and
// the 16-byte pieces of whole rows read back by one instruction are both
// spread over distinct banks.
template <class S>
TLG_HD int epi16_offset(int row, int piece) {
    static_assert(S::WTN == 128 || S::WTN == 64, "wave blocks 64 or 128 columns wide");
    return row * S::WTN * 2 + 16 * (piece ^ (S::WTN == 128 ? row % 16 : (row / 2) % 8));
}

// ---- tile order ----
// Work-groups are handed to the 8 XCDs of the device round-robin by id, so
// id p runs on XCD p % 8. Renumber so that each XCD receives a contiguous
// range of tiles, then walk tiles in groups of group_m tile-rows so that the
// work-groups resident at one time on one XCD share rows of A and columns of
// B in that XCD's L2. The map is a bijection on [0, nwg) for any nwg.
TLG_HD int xcd_remap(int pid, int nwg) {
    const int nx = 8;
    int per = nwg / nx, rem = nwg % nx;
    int x = pid % nx, idx = pid / nx;
    return x * per + imin(x, rem) + idx;
}
TLG_HD void grouped_tile(int q, int tiles_m, int tiles_n, int group_m, int *tm, int *tn) {
    int width = group_m * tiles_n;
    int first_m = (q / width) * group_m;
    int gsz = imin(tiles_m - first_m, group_m);
    int r = q % width;
    *tm = first_m + r % gsz;
    *tn = r / gsz;
}

// ---- stream-K ranges ----
// total iterations are split among G work-groups: work-group g takes
// [sk_begin(g), sk_begin(g + 1)); sk_owner(x) is the work-group whose range
// holds iteration x (the largest g with sk_begin(g) <= x).
TLG_HD int64_t sk_begin(int g, int64_t total, int G) { return (int64_t)g * total / G; }
TLG_HD int sk_owner(int64_t x, int64_t total, int G) { return (int)(((x + 1) * (int64_t)G - 1) / total); }

// ---- stream-K over strips ----
// The strips' K blocks (nkb per strip) in one strip-major sequence; a range
// [beg, end) of it that is at most nkb long touches at most two strips: its
// first strip s0 from beg up to min(end, bound), and, if two, strip s0 + 1
// from bound (the first block of s0 + 1) up to end. A part of a strip is
// whole when it covers all nkb blocks; the blocks a part adds to its strip's
// counter are part_blocks.
struct StripSegments {
    int s0;         // first strip of the range
    int64_t bound;  // first block of strip s0 + 1
    bool two;       // the range reaches strip s0 + 1
};
TLG_HD StripSegments strip_segments(int64_t beg, int64_t end, int nkb) {
    StripSegments r;
    r.s0 = (int)(beg / nkb);
    r.bound = (int64_t)(r.s0 + 1) * nkb;
    r.two = end > r.bound;
    return r;
}
// part q (0: strip s0, 1: strip s0 + 1) of the range
TLG_HD int64_t strip_part_blocks(const StripSegments &sg, int64_t beg, int64_t end, int q) {
    return q == 0 ? (end < sg.bound ? end : sg.bound) - beg : end - sg.bound;
}
TLG_HD bool strip_part_whole(const StripSegments &sg, int64_t beg, int64_t end, int nkb, int q) {
    return q == 0 ? beg == sg.bound - nkb && end >= sg.bound : end == sg.bound + nkb;
}

}  // namespace tlg

#endif
