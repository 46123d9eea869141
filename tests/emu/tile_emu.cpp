// CPU emulation of the data movement of the gfx950 GEMM+ReLU kernels (fp16
// and, at the end of the file, the block-scaled kernel)
// (test-only). It uses the kernels' own index arithmetic (tile_layout.h) and
// models, lane by lane:
//   * the direct-to-LDS loads (16 bytes per lane, zeros for out-of-range
//     lanes), checking that every real global access lies inside its matrix
//     and that each LDS stage is written exactly once;
//   * the operand fragment reads (ds_read_b128 and ds_read_b64_tr_b16 with
//     their measured lane semantics), checking LDS bounds and that each read
//     is free of bank conflicts on a 64-bank LDS;
//   * v_mfma_f32_32x32x16_f16 and v_mfma_f32_16x16x32_f16 with their
//     measured operand and result layouts (fp32 products, fp32 sums);
//   * the epilogue (ReLU and round-to-nearest-even fp16, or fp32 partials),
//     checking that every element of the M x N window is written exactly once
//     and nothing outside it.
// Its output is compared against the CPU oracle by the tests. It shares no
// code with the oracle.
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <cstdio>
#include <vector>

#include "tile_layout.h"

using namespace tlg;

namespace {

float h2f(uint16_t h) {
    // binary16 -> binary32 via the hardware-independent definition
    uint32_t s = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 31, f = h & 1023, u;
    if (e == 31) u = s | 0x7f800000u | (f << 13);
    else if (e == 0) {
        if (!f) u = s;
        else {
            int ex = -14;
            while (!(f & 1024)) { f <<= 1; ex--; }
            u = s | ((uint32_t)(ex + 127) << 23) | ((f & 1023) << 13);
        }
    } else u = s | ((e + 112) << 23) | (f << 13);
    float x;
    memcpy(&x, &u, 4);
    return x;
}

uint16_t f2h(float x) {  // round to nearest even via the C library's rounding of a scaled value
    if (std::isnan(x)) return 0x7e00;
    uint16_t sign = std::signbit(x) ? 0x8000 : 0;
    double a = std::fabs((double)x);
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < std::ldexp(1.0, -14)) {
        double q = std::nearbyint(a * std::ldexp(1.0, 24));  // FE_TONEAREST by default
        return sign | (uint16_t)q;
    }
    int e;
    std::frexp(a, &e);  // a = m * 2^e, m in [0.5, 1)
    double q = std::nearbyint(std::ldexp(a, 11 - e));  // 11 significant bits
    if (q >= 2048.0) { q /= 2; e += 1; }
    return sign | (uint16_t)(((e - 1 + 15) << 10) + ((int)q - 1024));
}

struct Errs {
    long oob_global = 0, lds_multi = 0, lds_oob = 0, bank_conflict = 0, c_multi = 0, c_missing = 0, c_outside = 0,
         tile_dup = 0;
};

struct Problem {
    int M, N, K;
    const uint16_t *A;
    long lda;
    const uint16_t *B;
    long ldb;
    uint16_t *C;
    long ldc;
    float *W;  // split mode: partials (splits x M x N)
    int k_split;
    int splits;
    bool bt = false;  // B given transposed: N x K row-major
};

// slot of a 16-byte access in a 256-byte bank window (64 banks x 4 bytes)
int slot16(int byte) { return (byte % 256) / 16; }

template <class S>
void run_dma(const Problem &p, bool split, Errs &er, std::vector<int> &cover) {
    const int tiles_m = (p.M + S::BM - 1) / S::BM, tiles_n = (p.N + S::BN - 1) / S::BN;
    const int nwg = tiles_m * tiles_n;
    std::vector<int> seen(nwg, 0);
    std::vector<uint8_t> lds(S::STAGE_BYTES);
    std::vector<int> lds_w(S::STAGE_BYTES);
    for (int y = 0; y < (split ? p.splits : 1); ++y)
        for (int pid = 0; pid < nwg; ++pid) {
            int tmi, tni;
            grouped_tile(xcd_remap(pid, nwg), tiles_m, tiles_n, 4, &tmi, &tni);
            if (tmi < 0 || tmi >= tiles_m || tni < 0 || tni >= tiles_n) { er.tile_dup++; continue; }
            if (y == 0) {
                if (seen[tmi * tiles_n + tni]++) er.tile_dup++;
            }
            const int m0 = tmi * S::BM, n0 = tni * S::BN;
            const int kbeg = split ? y * p.k_split : 0;
            // the tiled kernels' loads stop at kmain (K, or the largest multiple
            // of 8 below K when K or N is not a multiple of 8)
            const int kmain = (p.K % 8 == 0 && (p.bt || p.N % 8 == 0)) ? p.K : 8 * ((p.K - 1) / 8);
            const int kend = split ? std::min(p.K, kbeg + p.k_split) : kmain;
            const int nk = kend > kbeg ? (kend - kbeg + S::BK - 1) / S::BK : 0;
            // accumulators: [wave][tn][tm][lane][16]
            std::vector<float> acc((size_t)S::WAVES * S::TN * S::TM * 64 * 16, 0.0f);
            // fragments and MFMAs of the first nsteps k-steps of the stage in `lds`
            auto mfma_from_lds = [&](int nsteps) {
                for (int w = 0; w < S::WAVES; ++w) {
                    const int wm0 = (w / S::WN) * S::WTM, wn0 = (w % S::WN) * S::WTN;
                    for (int s = 0; s < nsteps; ++s) {
                        // bf[tn][lane][8], af[tm][lane][8]
                        std::vector<float> bf((size_t)S::TN * 64 * 8), af((size_t)S::TM * 64 * 8);
                        if (p.bt) {  // B tile held like A: A-style reads from the B region
                            for (int tn = 0; tn < S::TN; ++tn) {
                                int addr[64];
                                for (int l = 0; l < 64; ++l) {
                                    addr[l] = frag_a_offset<S>(wn0, tn, s, l);
                                    if (addr[l] < 0 || addr[l] + 16 > S::B_BYTES || addr[l] % 16) er.lds_oob++;
                                }
                                for (int q = 0; q < 4; ++q) {
                                    int used[16] = {0};
                                    for (int l = 16 * q; l < 16 * q + 16; ++l)
                                        if (used[slot16(addr[l])]++) er.bank_conflict++;
                                }
                                for (int l = 0; l < 64; ++l)
                                    for (int e = 0; e < 8; ++e) {
                                        uint16_t v = 0;
                                        if (addr[l] >= 0 && addr[l] + 16 <= S::B_BYTES)
                                            memcpy(&v, &lds[S::A_BYTES + addr[l] + 2 * e], 2);
                                        bf[((size_t)tn * 64 + l) * 8 + e] = h2f(v);
                                    }
                            }
                        }
                        for (int tn = 0; tn < (p.bt ? 0 : S::TN); ++tn)
                            for (int h = 0; h < 2; ++h) {
                                int addr[64];
                                for (int l = 0; l < 64; ++l) {
                                    addr[l] = frag_b_offset<S>(wn0, tn, s, h, l);
                                    if (addr[l] < 0 || addr[l] + 8 > S::B_BYTES || addr[l] % 8) er.lds_oob++;
                                }
                                // 32 lanes per LDS cycle: 32 x 8 bytes must hit 64 distinct banks
                                for (int half = 0; half < 2; ++half) {
                                    int used[64] = {0};
                                    for (int l = 32 * half; l < 32 * half + 32; ++l)
                                        for (int d = 0; d < 2; ++d) {
                                            int bank = ((addr[l] + 4 * d) / 4) % 64;
                                            if (used[bank]++) er.bank_conflict++;
                                        }
                                }
                                for (int l = 0; l < 64; ++l) {
                                    int g = l / 16, i = l % 16;
                                    for (int j = 0; j < 4; ++j) {
                                        int src = 16 * g + i / 4 + 4 * j;
                                        int a = addr[src];
                                        uint16_t v = 0;
                                        if (a >= 0 && a + 8 <= S::B_BYTES) memcpy(&v, &lds[S::A_BYTES + a + 2 * (i % 4)], 2);
                                        bf[((size_t)tn * 64 + l) * 8 + 4 * h + j] = h2f(v);
                                    }
                                }
                            }
                        for (int tm = 0; tm < S::TM; ++tm) {
                            int addr[64];
                            for (int l = 0; l < 64; ++l) {
                                addr[l] = frag_a_offset<S>(wm0, tm, s, l);
                                if (addr[l] < 0 || addr[l] + 16 > S::A_BYTES || addr[l] % 16) er.lds_oob++;
                            }
                            // 16 lanes per LDS cycle: 16 x 16 bytes must hit 16 distinct slots
                            for (int q = 0; q < 4; ++q) {
                                int used[16] = {0};
                                for (int l = 16 * q; l < 16 * q + 16; ++l)
                                    if (used[slot16(addr[l])]++) er.bank_conflict++;
                            }
                            for (int l = 0; l < 64; ++l)
                                for (int e = 0; e < 8; ++e) {
                                    uint16_t v = 0;
                                    if (addr[l] >= 0 && addr[l] + 16 <= S::A_BYTES) memcpy(&v, &lds[addr[l] + 2 * e], 2);
                                    af[((size_t)tm * 64 + l) * 8 + e] = h2f(v);
                                }
                        }
                        // D = X * Y: X from bf (rows i = lane%32, k = 8*(lane/32)+e), Y from af (cols j)
                        for (int tn = 0; tn < S::TN; ++tn)
                            for (int tm = 0; tm < S::TM; ++tm)
                                for (int l = 0; l < 64; ++l)
                                    for (int r = 0; r < 16; ++r) {
                                        int i = 8 * (r / 4) + 4 * (l / 32) + r % 4, j = l % 32;
                                        float sum = 0.0f;
                                        for (int kk = 0; kk < 16; ++kk) {
                                            int lx = i + 32 * (kk / 8), ly = j + 32 * (kk / 8), e = kk % 8;
                                            sum += bf[((size_t)tn * 64 + lx) * 8 + e] * af[((size_t)tm * 64 + ly) * 8 + e];
                                        }
                                        float &d = acc[((((size_t)w * S::TN + tn) * S::TM + tm) * 64 + l) * 16 + r];
                                        d = d + sum;
                                    }
                    }
                }
                        };
            for (int kt = 0; kt < nk; ++kt) {
                const int k0 = kbeg + kt * S::BK;
                std::fill(lds.begin(), lds.end(), 0xAB);
                std::fill(lds_w.begin(), lds_w.end(), 0);
                for (int w = 0; w < S::WAVES; ++w)
                    for (int lane = 0; lane < 64; ++lane) {
                        for (int i = 0; i < S::DMA_A; ++i) {
                            ChunkRef c = dma_a_chunk<S>(w, i, lane);
                            int dst = (w * S::DMA_A + i) * 1024 + lane * 16;
                            bool ok = m0 + c.row < p.M && k0 + 8 * c.chunk < kend;
                            for (int b = 0; b < 16; ++b) {
                                if (dst + b >= S::A_BYTES) { er.lds_oob++; continue; }
                                if (lds_w[dst + b]++) er.lds_multi++;
                            }
                            for (int e = 0; e < 8; ++e) {
                                uint16_t v = 0;
                                if (ok) {
                                    long row = m0 + c.row, col = k0 + 8 * c.chunk + e;
                                    if (row >= p.M || col >= p.K || col >= p.lda) er.oob_global++;
                                    else v = p.A[row * p.lda + col];
                                }
                                memcpy(&lds[dst + 2 * e], &v, 2);
                            }
                        }
                        for (int i = 0; i < S::DMA_B && p.bt; ++i) {  // rows n of the transposed B
                            ChunkRef c = dma_a_chunk<S>(w, i, lane);
                            int dst = S::A_BYTES + (w * S::DMA_B + i) * 1024 + lane * 16;
                            bool ok = n0 + c.row < p.N && k0 + 8 * c.chunk < kend;
                            for (int b = 0; b < 16; ++b) {
                                if (dst + b >= S::STAGE_BYTES) { er.lds_oob++; continue; }
                                if (lds_w[dst + b]++) er.lds_multi++;
                            }
                            for (int e = 0; e < 8; ++e) {
                                uint16_t v = 0;
                                if (ok) {
                                    long row = n0 + c.row, col = k0 + 8 * c.chunk + e;
                                    if (row >= p.N || col >= p.K || col >= p.ldb) er.oob_global++;
                                    else v = p.B[row * p.ldb + col];
                                }
                                memcpy(&lds[dst + 2 * e], &v, 2);
                            }
                        }
                        for (int i = 0; i < S::DMA_B && !p.bt; ++i) {
                            ChunkRef c = dma_b_chunk<S>(w, i, lane);
                            int dst = S::A_BYTES + (w * S::DMA_B + i) * 1024 + lane * 16;
                            bool ok = n0 + 8 * c.chunk < p.N && k0 + c.row < kend;
                            for (int b = 0; b < 16; ++b) {
                                if (dst + b >= S::STAGE_BYTES) { er.lds_oob++; continue; }
                                if (lds_w[dst + b]++) er.lds_multi++;
                            }
                            for (int e = 0; e < 8; ++e) {
                                uint16_t v = 0;
                                if (ok) {
                                    long row = k0 + c.row, col = n0 + 8 * c.chunk + e;
                                    // past column N only when N is not a multiple of 8, and then at
                                    // most into the next row, which must exist
                                    long idx = row * p.ldb + col;
                                    if (row >= p.K || (col >= p.N && p.N % 8 == 0) ||
                                        idx >= (long)(p.K - 1) * p.ldb + p.N)
                                        er.oob_global++;
                                    else v = p.B[idx];
                                }
                                memcpy(&lds[dst + 2 * e], &v, 2);
                            }
                        }
                    }
                for (int b = 0; b < S::STAGE_BYTES; ++b)
                    if (lds_w[b] != 1) er.lds_multi++;
                mfma_from_lds(S::KSTEPS);
            }
            // rows kmain .. K-1: one zero-padded 16-deep block staged element by
            // element (A chunks 0-1 of every row, B rows 0-15), one k-step
            if (!split && kmain < p.K) {
                std::fill(lds.begin(), lds.end(), 0xAB);
                for (int row = 0; row < S::BM; ++row)
                    for (int chunk = 0; chunk < 2; ++chunk)
                        for (int e = 0; e < 8; ++e) {
                            long m = m0 + row, k = kmain + 8 * chunk + e;
                            uint16_t v = (m < p.M && k < p.K) ? p.A[m * p.lda + k] : 0;
                            memcpy(&lds[lds_a_offset<S>(row, chunk) + 2 * e], &v, 2);
                        }
                for (int row = 0; row < S::BN && p.bt; ++row)  // transposed B: rows n, like A
                    for (int chunk = 0; chunk < 2; ++chunk)
                        for (int e = 0; e < 8; ++e) {
                            long n = n0 + row, k = kmain + 8 * chunk + e;
                            uint16_t v = (n < p.N && k < p.K) ? p.B[n * p.ldb + k] : 0;
                            memcpy(&lds[S::A_BYTES + lds_a_offset<S>(row, chunk) + 2 * e], &v, 2);
                        }
                for (int row = 0; row < (p.bt ? 0 : 16); ++row)
                    for (int chunk = 0; chunk < S::CB; ++chunk)
                        for (int e = 0; e < 8; ++e) {
                            long k = kmain + row, n = n0 + 8 * chunk + e;
                            uint16_t v = (k < p.K && n < p.N) ? p.B[k * p.ldb + n] : 0;
                            memcpy(&lds[S::A_BYTES + lds_b_offset<S>(row, chunk) + 2 * e], &v, 2);
                        }
                mfma_from_lds(1);
            }
            // epilogue
            for (int w = 0; w < S::WAVES; ++w) {
                const int wm0 = (w / S::WN) * S::WTM, wn0 = (w % S::WN) * S::WTN;
                for (int tn = 0; tn < S::TN; ++tn)
                    for (int tm = 0; tm < S::TM; ++tm)
                        for (int l = 0; l < 64; ++l)
                            for (int r = 0; r < 16; ++r) {
                                int m = m0 + acc_m(wm0, tm, l), n = n0 + acc_n(wn0, tn, r, l);
                                float v = acc[((((size_t)w * S::TN + tn) * S::TM + tm) * 64 + l) * 16 + r];
                                if (m >= p.M || n >= p.N) continue;  // the kernel masks these
                                if (split) {
                                    p.W[((size_t)y * p.M + m) * p.N + n] = v;
                                    cover[((size_t)y * p.M + m) * p.N + n]++;
                                } else {
                                    p.C[(size_t)m * p.ldc + n] = f2h(v > 0.0f ? v : 0.0f);
                                    cover[(size_t)m * p.N + n]++;
                                }
                            }
            }
        }
    for (int t = 0; t < nwg; ++t)
        if (seen[t] != 1) er.tile_dup++;
}

// The 16 x 16 x 32 pipelined kernel (gemm_relu_pipe16_gfx950.hip), with its
// own load offsets (p16_a_lane_bytes, p16_b_lane_bytes, p16_b_slab_bytes and
// the buffer ranges it sets), fragment address parts (frag_a16_lane,
// frag_b16_lane), v_mfma_f32_16x16x32_f16 with its measured layouts, the K
// tail (a masked stage, then a zero-padded 32-deep block) and the LDS-staged
// epilogue (epi16_offset).
// p.bt: B given transposed (N x K), its tile held like the A tile
// (dma_bt16_chunk, p16_a_lane_bytes, frag_a16_lane over the rows n).
template <class S>
void run_pipe16(const Problem &p, Errs &er, std::vector<int> &cover) {
    const bool bt = p.bt;
    const int tiles_m = (p.M + S::BM - 1) / S::BM, tiles_n = (p.N + S::BN - 1) / S::BN;
    const int nwg = tiles_m * tiles_n;
    std::vector<int> seen(nwg, 0);
    const int STAGE = S::A_BYTES + S::B_BYTES;
    std::vector<uint8_t> lds(STAGE);
    std::vector<int> lds_w(STAGE);
    const int kmain = (p.K % 8 == 0 && (bt || p.N % 8 == 0)) ? p.K : 8 * ((p.K - 1) / 8);
    const int nk = kmain / S::BK;
    const long b_end = (long)(p.K - 1) * p.ldb + p.N;  // elements of B the caller owns
    // a global element read by a direct-to-LDS load, given by its logical
    // position (row, col) and the element index the load's address gives:
    // the two must agree, the position must lie inside the matrix and inside
    // K's rows [0, kend)
    auto read_a = [&](long row, long col, long idx, int kend) -> uint16_t {
        if (idx != row * p.lda + col || row < 0 || row >= p.M || col < 0 || col >= kend) {
            er.oob_global++;
            return 0;
        }
        return p.A[idx];
    };
    // a transposed B: position (n, k), inside N and K's rows [0, kend)
    auto read_bt = [&](long row, long col, long idx, int kend) -> uint16_t {
        if (idx != row * p.ldb + col || row < 0 || row >= p.N || col < 0 || col >= kend) {
            er.oob_global++;
            return 0;
        }
        return p.B[idx];
    };
    auto read_b = [&](long row, long col, long idx, int kend) -> uint16_t {
        // past column N only when N is not a multiple of 8, then into the
        // row's padding or the next row, never past the caller's last element
        if (idx != row * p.ldb + col || row < 0 || row >= kend || (col >= p.N && p.N % 8 == 0) || idx >= b_end) {
            er.oob_global++;
            return 0;
        }
        return p.B[idx];
    };
    auto mark = [&](int dst, int n, int limit) {
        for (int b = 0; b < n; ++b) {
            if (dst + b < 0 || dst + b >= limit) { er.lds_oob++; continue; }
            if (lds_w[dst + b]++) er.lds_multi++;
        }
    };
    for (int pid = 0; pid < nwg; ++pid) {
        int tmi, tni;
        grouped_tile(xcd_remap(pid, nwg), tiles_m, tiles_n, 4, &tmi, &tni);
        if (tmi < 0 || tmi >= tiles_m || tni < 0 || tni >= tiles_n) { er.tile_dup++; continue; }
        if (seen[tmi * tiles_n + tni]++) er.tile_dup++;
        const int m0 = tmi * S::BM, n0 = tni * S::BN;
        std::vector<float> acc((size_t)S::WAVES * S::TN * S::TM * 64 * 4, 0.0f);
        // fragments of k-step s of the stage in `lds` and the MFMAs on them
        auto kstep = [&](int s) {
            for (int w = 0; w < S::WAVES; ++w) {
                const int wm0 = (w / S::WN) * S::WTM, wn0 = (w % S::WN) * S::WTN;
                std::vector<float> bf((size_t)S::TN * 64 * 8), af((size_t)S::TM * 64 * 8);
                for (int tn = 0; bt && tn < S::TN; ++tn) {  // one 16-byte read per lane, as for A
                    int addr[64];
                    for (int l = 0; l < 64; ++l) {
                        addr[l] = frag_a16_lane<S>(wn0, s & 1, l) + tn * 16 * S::RA;
                        if (addr[l] != frag_a16_offset<S>(wn0, tn, s, l)) er.lds_oob++;
                        if (addr[l] < 0 || addr[l] + 16 > S::B_BYTES || addr[l] % 16) er.lds_oob++;
                    }
                    for (int q = 0; q < 4; ++q) {  // 16 lanes x 16 bytes per LDS cycle
                        int used[16] = {0};
                        for (int l = 16 * q; l < 16 * q + 16; ++l)
                            if (used[slot16(addr[l])]++) er.bank_conflict++;
                    }
                    for (int l = 0; l < 64; ++l)
                        for (int e = 0; e < 8; ++e) {
                            uint16_t v = 0;
                            if (addr[l] >= 0 && addr[l] + 16 <= S::B_BYTES) memcpy(&v, &lds[S::A_BYTES + addr[l] + 2 * e], 2);
                            bf[((size_t)tn * 64 + l) * 8 + e] = h2f(v);
                        }
                }
                for (int tn = 0; !bt && tn < S::TN; ++tn)
                    for (int h = 0; h < 2; ++h) {
                        int addr[64];
                        for (int l = 0; l < 64; ++l) {
                            addr[l] = frag_b16_lane<S>(wn0, tn, l) + (32 * s + 4 * h) * S::RB;
                            if (addr[l] != frag_b16_offset<S>(wn0, tn, s, h, l)) er.lds_oob++;
                            if (addr[l] < 0 || addr[l] + 8 > S::B_BYTES || addr[l] % 8) er.lds_oob++;
                        }
                        for (int half = 0; half < 2; ++half) {  // 32 lanes x 8 bytes on 64 banks
                            int used[64] = {0};
                            for (int l = 32 * half; l < 32 * half + 32; ++l)
                                for (int d = 0; d < 2; ++d)
                                    if (used[((addr[l] + 4 * d) / 4) % 64]++) er.bank_conflict++;
                        }
                        for (int l = 0; l < 64; ++l) {  // the transposing read's lane semantics
                            int g = l / 16, i = l % 16;
                            for (int j = 0; j < 4; ++j) {
                                int a = addr[16 * g + i / 4 + 4 * j];
                                uint16_t v = 0;
                                if (a >= 0 && a + 8 <= S::B_BYTES) memcpy(&v, &lds[S::A_BYTES + a + 2 * (i % 4)], 2);
                                bf[((size_t)tn * 64 + l) * 8 + 4 * h + j] = h2f(v);
                            }
                        }
                    }
                for (int tm = 0; tm < S::TM; ++tm) {
                    int addr[64];
                    for (int l = 0; l < 64; ++l) {
                        addr[l] = frag_a16_lane<S>(wm0, s & 1, l) + tm * 16 * S::RA;
                        if (addr[l] != frag_a16_offset<S>(wm0, tm, s, l)) er.lds_oob++;
                        if (addr[l] < 0 || addr[l] + 16 > S::A_BYTES || addr[l] % 16) er.lds_oob++;
                    }
                    for (int q = 0; q < 4; ++q) {  // 16 lanes x 16 bytes per LDS cycle
                        int used[16] = {0};
                        for (int l = 16 * q; l < 16 * q + 16; ++l)
                            if (used[slot16(addr[l])]++) er.bank_conflict++;
                    }
                    for (int l = 0; l < 64; ++l)
                        for (int e = 0; e < 8; ++e) {
                            uint16_t v = 0;
                            if (addr[l] >= 0 && addr[l] + 16 <= S::A_BYTES) memcpy(&v, &lds[addr[l] + 2 * e], 2);
                            af[((size_t)tm * 64 + l) * 8 + e] = h2f(v);
                        }
                }
                // D = X * Y, X (16 x 32) the B fragment: lane l row l%16, k 8*(l/16)+e;
                // Y (32 x 16) the A fragment: lane l column l%16, k 8*(l/16)+e;
                // result register r of lane l: D[4*(l/16) + r][l%16]
                for (int tn = 0; tn < S::TN; ++tn)
                    for (int tm = 0; tm < S::TM; ++tm)
                        for (int l = 0; l < 64; ++l)
                            for (int r = 0; r < 4; ++r) {
                                int i = 4 * (l / 16) + r, j = l % 16;
                                float sum = 0.0f;
                                for (int kk = 0; kk < 32; ++kk) {
                                    int lx = i + 16 * (kk / 8), ly = j + 16 * (kk / 8), e = kk % 8;
                                    sum += bf[((size_t)tn * 64 + lx) * 8 + e] * af[((size_t)tm * 64 + ly) * 8 + e];
                                }
                                float &d = acc[((((size_t)w * S::TN + tn) * S::TM + tm) * 64 + l) * 4 + r];
                                d = d + sum;
                            }
            }
        };
        auto clear = [&]() {
            std::fill(lds.begin(), lds.end(), 0xAB);
            std::fill(lds_w.begin(), lds_w.end(), 0);
        };
        // the loop's whole stages: offsets computed once per lane, the stage
        // moving only the descriptor base; A's range ends after row M - 1
        for (int kt = 0; kt < nk; ++kt) {
            const int k0 = kt * S::BK;
            clear();
            for (int w = 0; w < S::WAVES; ++w)
                for (int lane = 0; lane < 64; ++lane) {
                    for (int i = 0; i < S::DMA_A; ++i) {
                        const int slab = w * S::DMA_A + i;
                        const long base = (long)(m0 + slab * 8) * p.lda + k0;  // the descriptor's base
                        const long rows = (long)p.M - m0 - slab * 8;
                        const long nrec = rows <= 0 ? 0 : rows * p.lda * 2;
                        const long off = (long)p16_a_lane_bytes<S>(lane, slab % 2, p.lda);
                        const int dst = slab * 1024 + lane * 16;
                        mark(dst, 16, S::A_BYTES);
                        const bool in = off + 16 <= nrec;
                        if (!in && off < nrec) er.oob_global++;  // a load only partly in range
                        const ChunkRef c = dma_a_chunk<S>(w, i, lane);  // what the layout expects here
                        if (in != (m0 + c.row < p.M)) er.oob_global++;
                        for (int e = 0; e < 8; ++e) {
                            uint16_t v = in ? read_a(m0 + c.row, k0 + 8 * c.chunk + e, base + off / 2 + e, kmain) : 0;
                            if (dst + 2 * e + 2 <= S::A_BYTES) memcpy(&lds[dst + 2 * e], &v, 2);
                        }
                    }
                    for (int i = 0; bt && i < S::DMA_B; ++i) {
                        const int slab = w * S::DMA_B + i;
                        const long base = (long)(n0 + slab * 8) * p.ldb + k0;  // the descriptor's base
                        const long rows = (long)p.N - n0 - slab * 8;
                        const long nrec = rows <= 0 ? 0 : rows * p.ldb * 2;
                        const long off = (long)p16_a_lane_bytes<S>(lane, slab % 2, p.ldb);
                        const int dst = S::A_BYTES + slab * 1024 + lane * 16;
                        mark(dst, 16, STAGE);
                        const bool in = off + 16 <= nrec;
                        if (!in && off < nrec) er.oob_global++;
                        const ChunkRef c = dma_bt16_chunk<S>(w, i, lane);
                        if (in != (n0 + c.row < p.N)) er.oob_global++;
                        for (int e = 0; e < 8; ++e) {
                            uint16_t v = in ? read_bt(n0 + c.row, k0 + 8 * c.chunk + e, base + off / 2 + e, kmain) : 0;
                            if (dst + 2 * e + 2 <= STAGE) memcpy(&lds[dst + 2 * e], &v, 2);
                        }
                    }
                    for (int i = 0; !bt && i < S::DMA_B; ++i) {
                        const int slab = w * S::DMA_B + i;
                        const long base = (long)k0 * p.ldb + n0;
                        const long soff = (long)p16_b_slab_bytes(slab, p.ldb);
                        const long off = (long)p16_b_lane_bytes<S>(lane, p16_b_pattern(slab), n0, p.N, p.ldb);
                        const int dst = S::A_BYTES + slab * 1024 + lane * 16;
                        mark(dst, 16, STAGE);
                        const ChunkRef c = dma_b16_chunk<S>(w, i, lane);
                        if ((off >= 0) != (n0 + 8 * c.chunk < p.N)) er.oob_global++;
                        for (int e = 0; e < 8; ++e) {
                            uint16_t v = off >= 0 ? read_b(k0 + c.row, n0 + 8 * c.chunk + e, base + (soff + off) / 2 + e,
                                                           kmain)
                                                  : 0;
                            if (dst + 2 * e + 2 <= STAGE) memcpy(&lds[dst + 2 * e], &v, 2);
                        }
                    }
                }
            for (int b = 0; b < STAGE; ++b)
                if (lds_w[b] != 1) er.lds_multi++;
            for (int s = 0; s < S::KSTEPS; ++s) kstep(s);
        }
        // rows [64*nk, kmain): one stage with every lane's chunk checked
        const int kfull = nk * S::BK;
        if (kfull < kmain) {
            clear();
            for (int w = 0; w < S::WAVES; ++w)
                for (int lane = 0; lane < 64; ++lane) {
                    for (int i = 0; i < S::DMA_A; ++i) {
                        const ChunkRef c = dma_a_chunk<S>(w, i, lane);
                        const int dst = (w * S::DMA_A + i) * 1024 + lane * 16;
                        mark(dst, 16, S::A_BYTES);
                        const bool in = m0 + c.row < p.M && kfull + 8 * c.chunk < kmain;
                        for (int e = 0; e < 8; ++e) {
                            const long row = m0 + c.row, col = kfull + 8 * c.chunk + e;
                            uint16_t v = in ? read_a(row, col, row * p.lda + col, kmain) : 0;
                            memcpy(&lds[dst + 2 * e], &v, 2);
                        }
                    }
                    for (int i = 0; bt && i < S::DMA_B; ++i) {
                        const ChunkRef c = dma_bt16_chunk<S>(w, i, lane);
                        const int dst = S::A_BYTES + (w * S::DMA_B + i) * 1024 + lane * 16;
                        mark(dst, 16, STAGE);
                        const bool in = n0 + c.row < p.N && kfull + 8 * c.chunk < kmain;
                        for (int e = 0; e < 8; ++e) {
                            const long row = n0 + c.row, col = kfull + 8 * c.chunk + e;
                            uint16_t v = in ? read_bt(row, col, row * p.ldb + col, kmain) : 0;
                            memcpy(&lds[dst + 2 * e], &v, 2);
                        }
                    }
                    for (int i = 0; !bt && i < S::DMA_B; ++i) {
                        const ChunkRef c = dma_b16_chunk<S>(w, i, lane);
                        const int dst = S::A_BYTES + (w * S::DMA_B + i) * 1024 + lane * 16;
                        mark(dst, 16, STAGE);
                        const bool in = kfull + c.row < kmain && n0 + 8 * c.chunk < p.N;
                        for (int e = 0; e < 8; ++e) {
                            const long row = kfull + c.row, col = n0 + 8 * c.chunk + e;
                            uint16_t v = in ? read_b(row, col, row * p.ldb + col, kmain) : 0;
                            memcpy(&lds[dst + 2 * e], &v, 2);
                        }
                    }
                }
            for (int b = 0; b < STAGE; ++b)
                if (lds_w[b] != 1) er.lds_multi++;
            for (int s = 0; s < S::KSTEPS; ++s) kstep(s);
        }
        // rows [kmain, K): a zero-padded 32-deep block, element by element
        if (kmain < p.K) {
            std::fill(lds.begin(), lds.end(), 0xAB);
            for (int row = 0; row < S::BM; ++row)
                for (int chunk = 0; chunk < 4; ++chunk)
                    for (int e = 0; e < 8; ++e) {
                        long m = m0 + row, k = kmain + 8 * chunk + e;
                        uint16_t v = (m < p.M && k < p.K) ? p.A[m * p.lda + k] : 0;
                        memcpy(&lds[lds_a_offset<S>(row, chunk) + 2 * e], &v, 2);
                    }
            for (int row = 0; bt && row < S::BN; ++row)
                for (int chunk = 0; chunk < 4; ++chunk)
                    for (int e = 0; e < 8; ++e) {
                        long n = n0 + row, k = kmain + 8 * chunk + e;
                        uint16_t v = (n < p.N && k < p.K) ? p.B[n * p.ldb + k] : 0;
                        memcpy(&lds[S::A_BYTES + lds_a_offset<S>(row, chunk) + 2 * e], &v, 2);
                    }
            for (int row = 0; !bt && row < 32; ++row)
                for (int chunk = 0; chunk < S::CB; ++chunk)
                    for (int e = 0; e < 8; ++e) {
                        long k = kmain + row, n = n0 + 8 * chunk + e;
                        uint16_t v = (k < p.K && n < p.N) ? p.B[k * p.ldb + n] : 0;
                        memcpy(&lds[S::A_BYTES + lds_b16_offset<S>(row, chunk) + 2 * e], &v, 2);
                    }
            kstep(0);
        }
        // epilogue: each wave's block through LDS, then whole row pieces
        constexpr int PIECES = S::WTN / 8;
        const int EPI = S::WAVES * S::WTM * S::WTN * 2;
        std::vector<uint8_t> elds(EPI, 0);
        std::vector<int> ew(EPI, 0);
        for (int w = 0; w < S::WAVES; ++w) {
            const int q = w * S::WTM * S::WTN * 2;
            const int wm0 = (w / S::WN) * S::WTM, wn0 = (w % S::WN) * S::WTN;
            for (int tn = 0; tn < S::TN; ++tn)
                for (int tm = 0; tm < S::TM; ++tm) {
                    int addr[64];
                    for (int l = 0; l < 64; ++l) {
                        const int row = 16 * tm + l % 16, col = 16 * tn + 4 * (l / 16);
                        addr[l] = q + epi16_offset<S>(row, col / 8) + 2 * (col % 8);
                        if (addr[l] < q || addr[l] + 8 > q + S::WTM * S::WTN * 2) { er.lds_oob++; continue; }
                        for (int r = 0; r < 4; ++r) {
                            float v = acc[((((size_t)w * S::TN + tn) * S::TM + tm) * 64 + l) * 4 + r];
                            uint16_t h = f2h(v > 0.0f ? v : 0.0f);
                            memcpy(&elds[addr[l] + 2 * r], &h, 2);
                        }
                        for (int b = 0; b < 8; ++b)
                            if (ew[addr[l] + b]++) er.lds_multi++;
                    }
                    for (int half = 0; half < 2; ++half) {  // 32 lanes x 8 bytes on 64 banks
                        int used[64] = {0};
                        for (int l = 32 * half; l < 32 * half + 32; ++l)
                            for (int d = 0; d < 2; ++d)
                                if (used[((addr[l] + 4 * d) / 4) % 64]++) er.bank_conflict++;
                    }
                }
            for (int k = 0; k < S::WTM / (64 / PIECES); ++k) {
                int addr[64];
                for (int l = 0; l < 64; ++l) addr[l] = q + epi16_offset<S>(k * (64 / PIECES) + l / PIECES, l % PIECES);
                for (int g = 0; g < 4; ++g) {
                    int used[16] = {0};
                    for (int l = 16 * g; l < 16 * g + 16; ++l)
                        if (used[slot16(addr[l])]++) er.bank_conflict++;
                }
                for (int l = 0; l < 64; ++l) {
                    const int row = k * (64 / PIECES) + l / PIECES, piece = l % PIECES;
                    const int m = m0 + wm0 + row;
                    if (m >= p.M) continue;  // dropped by the range check
                    for (int e = 0; e < 8; ++e) {
                        const int n = n0 + wn0 + 8 * piece + e;
                        if (n >= p.N) {
                            if (n0 + wn0 + 8 * piece + 8 <= p.N) er.c_outside++;
                            continue;  // stored element by element up to N
                        }
                        uint16_t v;
                        memcpy(&v, &elds[addr[l] + 2 * e], 2);
                        p.C[(size_t)m * p.ldc + n] = v;
                        cover[(size_t)m * p.N + n]++;
                    }
                }
            }
        }
        for (int b = 0; b < EPI; ++b)
            if (ew[b] != 1) er.lds_multi++;
    }
    for (int t = 0; t < nwg; ++t)
        if (seen[t] != 1) er.tile_dup++;
}

template <class S>
int emulate_pipe16(const Problem &p, long *errs) {
    Errs er;
    std::vector<int> cover((size_t)p.M * p.N, 0);
    run_pipe16<S>(p, er, cover);
    for (int c : cover) {
        if (c == 0) er.c_missing++;
        if (c > 1) er.c_multi++;
    }
    errs[0] = er.oob_global;
    errs[1] = er.lds_multi;
    errs[2] = er.lds_oob;
    errs[3] = er.bank_conflict;
    errs[4] = er.c_multi;
    errs[5] = er.c_missing;
    errs[6] = er.c_outside;
    errs[7] = er.tile_dup;
    return 0;
}

template <class S>
int emulate(const Problem &p, bool split, long *errs) {
    Errs er;
    std::vector<int> cover((size_t)(split ? p.splits : 1) * p.M * p.N, 0);
    run_dma<S>(p, split, er, cover);
    for (int c : cover) {
        if (c == 0) er.c_missing++;
        if (c > 1) er.c_multi++;
    }
    if (split) {  // stage 2: ordered sum over splits, ReLU, cast
        for (long mn = 0; mn < (long)p.M * p.N; ++mn) {
            float a = p.W[mn];
            for (int s = 1; s < p.splits; ++s) a = a + p.W[(size_t)s * p.M * p.N + mn];
            p.C[(mn / p.N) * p.ldc + mn % p.N] = f2h(a > 0.0f ? a : 0.0f);
        }
    }
    errs[0] = er.oob_global;
    errs[1] = er.lds_multi;
    errs[2] = er.lds_oob;
    errs[3] = er.bank_conflict;
    errs[4] = er.c_multi;
    errs[5] = er.c_missing;
    errs[6] = er.c_outside;
    errs[7] = er.tile_dup;
    return 0;
}

}  // namespace

// Shapes mirrored from the kernels' configuration table.
using E256 = TileShape<256, 256, 32, 2, 2, 4>;
using E128 = TileShape<128, 128, 32, 2, 2, 4>;
using E64 = TileShape<64, 64, 64, 2, 2, 3>;
using ES128 = TileShape<32, 128, 64, 1, 4, 4>;
using ES256 = TileShape<32, 256, 64, 1, 4, 3>;
using EP64 = TileShape<256, 256, 64, 2, 2, 2>;  // pipelined, 64-deep stages
using E256w8 = TileShape<256, 256, 64, 2, 4, 2>;
using E256w8x32 = TileShape<256, 256, 32, 2, 4, 4>;
using EP256x128 = TileShape<256, 128, 64, 2, 2, 3>;  // pipelined half tiles
using EP128x256 = TileShape<128, 256, 64, 1, 4, 3>;
using EStrip64 = TileShape<64, 64, 64, 1, 1, 3>;  // one wave per 64 x 64 strip ring
// the 16 x 16 x 32 pipelined kernel: four waves of 128 x 128, the 128 x 256
// half tiles, eight waves of 128 x 64
using E16w4 = TileShape16<256, 256, 64, 2, 2, 2>;
using E16h = TileShape16<128, 256, 64, 1, 4, 3>;
using E16w8 = TileShape16<256, 256, 64, 2, 4, 2>;
using E16t = TileShape16<192, 256, 64, 2, 2, 2>;

extern "C" int emu_gemm_relu(int config, int M, int N, int K, const uint16_t *A, long lda, const uint16_t *B,
                             long ldb, uint16_t *C, long ldc, int splits, int k_split, float *W, long *errs) {
    Problem p{M, N, K, A, lda, B, ldb, C, ldc, W, k_split, splits};
    switch (config) {
        case 0: return emulate<E256>(p, false, errs);
        case 1: return emulate<E128>(p, false, errs);
        case 2: return emulate<E64>(p, false, errs);
        case 3: return emulate<EP64>(p, false, errs);
        case 4: return emulate<E256w8>(p, false, errs);
        case 5: return emulate<E256w8x32>(p, false, errs);
        case 6: return emulate<EP256x128>(p, false, errs);
        case 7: return emulate<EP128x256>(p, false, errs);
        case 8: return emulate<EStrip64>(p, false, errs);
        case 10: return emulate<ES128>(p, true, errs);
        case 11: return emulate<ES256>(p, true, errs);
        case 20: return emulate_pipe16<E16w4>(p, errs);
        case 21: return emulate_pipe16<E16h>(p, errs);
        case 22: return emulate_pipe16<E16w8>(p, errs);
        case 23: return emulate_pipe16<E16t>(p, errs);
        default: return -1;
    }
}

// Transposed B (Bt is N x K row-major): direct-to-LDS configurations 0..2 and
// the stage layouts of the pipelined kernel (3, 4).
extern "C" int emu_gemm_relu_bt(int config, int M, int N, int K, const uint16_t *A, long lda, const uint16_t *Bt,
                                long ldbt, uint16_t *C, long ldc, long *errs) {
    Problem p{M, N, K, A, lda, Bt, ldbt, C, ldc, nullptr, 0, 1};
    p.bt = true;
    switch (config) {
        case 0: return emulate<E256>(p, false, errs);
        case 1: return emulate<E128>(p, false, errs);
        case 2: return emulate<E64>(p, false, errs);
        case 3: return emulate<EP64>(p, false, errs);    // pipelined, four waves
        case 4: return emulate<E256w8>(p, false, errs);  // pipelined, eight waves
        case 8: return emulate<EStrip64>(p, false, errs);  // the 64-row strip, B's blocks like A's rows
        case 20: return emulate_pipe16<E16w4>(p, errs);  // 16 x 16 x 32 pipelined tiles
        case 21: return emulate_pipe16<E16h>(p, errs);
        case 23: return emulate_pipe16<E16t>(p, errs);
        default: return -1;
    }
}

// Stream-K bookkeeping: the ranges partition [0, total); sk_owner finds the
// range of every iteration; every tile's parts, taken from its first owner to
// its last, are the consecutive pieces of the tile in ascending k, each
// assigned to slot 0 (the piece starts its work-group's range) or slot 1 (the
// piece ends a range that began in an earlier tile), never both slots taken
// by two split tiles of one work-group in the same slot. Returns the number
// of violations.
// Stream-K over strips (G >= strips): every range touches at most two
// strips, its parts cover each block exactly once, the blocks counted into a
// strip add up to nkb exactly when its last part arrives, a part is whole
// only when it is the strip's only part, and the slot a finisher reads for a
// contributor (slot 0 iff the contributor's range starts inside the strip)
// is the one that contributor wrote its part of this strip to.
extern "C" long emu_check_strip_sk(int strips, int nkb, int G) {
    long bad = 0;
    const int64_t T = (int64_t)strips * nkb;
    if (G > T) G = (int)T;
    std::vector<int> seen((size_t)T, 0);
    std::vector<int64_t> counted((size_t)strips, 0);
    std::vector<int> parts((size_t)strips, 0), whole((size_t)strips, 0);
    std::vector<int> slot_strip(2 * (size_t)G, -1);  // strip each written slot holds
    for (int g = 0; g < G; ++g) {
        const int64_t beg = sk_begin(g, T, G), end = sk_begin(g + 1, T, G);
        if (beg == end) continue;
        if (end - beg > nkb) bad++;
        const StripSegments sg = strip_segments(beg, end, nkb);
        if (sg.s0 < 0 || sg.s0 >= strips || (sg.two && sg.s0 + 1 >= strips)) { bad++; continue; }
        if (end > sg.bound + nkb) bad++;  // a third strip would be lost
        for (int q = 0; q < (sg.two ? 2 : 1); ++q) {
            const int s = sg.s0 + q;
            const int64_t lo = q == 0 ? beg : sg.bound, n = strip_part_blocks(sg, beg, end, q);
            if (n <= 0) bad++;
            for (int64_t u = lo; u < lo + n; ++u) {
                if (u / nkb != s) bad++;
                seen[(size_t)u]++;
            }
            counted[(size_t)s] += n;
            parts[(size_t)s]++;
            if (strip_part_whole(sg, beg, end, nkb, q)) whole[(size_t)s]++;
            else slot_strip[2 * (size_t)g + q] = s;
        }
    }
    for (int64_t u = 0; u < T; ++u)
        if (seen[(size_t)u] != 1) bad++;
    for (int s = 0; s < strips; ++s) {
        if (counted[(size_t)s] != nkb) bad++;
        if (whole[(size_t)s] != (parts[(size_t)s] == 1 ? 1 : 0)) bad++;
        if (parts[(size_t)s] == 1) continue;
        const int64_t first = (int64_t)s * nkb;
        const int g0 = sk_owner(first, T, G), g1 = sk_owner(first + nkb - 1, T, G);
        int found = 0;
        for (int gg = g0; gg <= g1; ++gg) {
            const int64_t gb = sk_begin(gg, T, G);
            if (sk_begin(gg + 1, T, G) == gb) continue;
            const int slot = gb >= first ? 0 : 1;
            if (slot_strip[2 * (size_t)gg + slot] != s) bad++;
            found++;
        }
        if (found != parts[(size_t)s]) bad++;
    }
    return bad;
}

extern "C" long emu_check_streamk(long total, int G, int ipt) {
    long bad = 0;
    if (sk_begin(0, total, G) != 0 || sk_begin(G, total, G) != total) bad++;
    for (int g = 0; g < G; ++g)
        if (sk_begin(g + 1, total, G) < sk_begin(g, total, G)) bad++;
    for (long x = 0; x < total; ++x) {
        int g = sk_owner(x, total, G);
        if (g < 0 || g >= G || !(sk_begin(g, total, G) <= x && x < sk_begin(g + 1, total, G))) bad++;
    }
    const long tiles = total / ipt;
    std::vector<int> used(2 * (size_t)G, 0);
    for (long t = 0; t < tiles; ++t) {
        const long first = t * ipt, last = first + ipt;  // [first, last)
        int g0 = sk_owner(first, total, G), g1 = sk_owner(last - 1, total, G);
        long covered = first;
        for (int g = g0; g <= g1; ++g) {
            long b = sk_begin(g, total, G), e = sk_begin(g + 1, total, G);
            if (b == e) continue;
            long lo = std::max(b, first), hi = std::min(e, last);
            if (lo != covered || hi <= lo) bad++;
            covered = hi;
            bool whole = lo == first && hi == last;
            if (whole) { if (g0 != g1) bad++; continue; }
            int slot = b >= first ? 0 : 1;
            // the kernel's own rule: slot 0 iff the piece starts the range
            if ((lo == b) != (slot == 0)) bad++;
            if (used[2 * g + slot]++) bad++;
        }
        if (covered != last) bad++;
    }
    return bad;
}

// xcd_remap must be a bijection on [0, nwg) for every nwg.
extern "C" long emu_check_remap(int max_nwg) {
    long bad = 0;
    for (int n = 1; n <= max_nwg; ++n) {
        std::vector<int> hit(n, 0);
        for (int p = 0; p < n; ++p) {
            int q = xcd_remap(p, n);
            if (q < 0 || q >= n || hit[q]++) bad++;
        }
    }
    return bad;
}

// The LDS epilogue (pipelined and direct-to-LDS kernels) for every wave block
// of tile shape S:
// every result register is followed through the conversion into 32-bit
// pairs, the lane-pair exchange (v_permlane32_swap: the upper 32 lanes of its
// first operand trade places with the lower 32 lanes of its second), the
// write to LDS and the read-back, and must reach the C position that
// acc_m/acc_n assign to it; every LDS piece is written once, and each group
// of 16 lanes touches 16 distinct 16-byte slots of a 256-byte window on both
// sides. Returns the number of violations.
template <class S>
long check_epilogue() {
    long bad = 0;
    const int CH = S::WTN / 8;
    for (int wave = 0; wave < S::WAVES; ++wave) {
        const int wm0 = (wave / S::WN) * S::WTM, wn0 = (wave % S::WN) * S::WTN;
        // LDS of the wave block: per half, the (m, n) it holds (-1: never written)
        std::vector<long> lds((size_t)S::WTM * S::WTN, -1);
        auto tag = [&](int m, int n) { return (long)m * 65536 + n; };
        for (int tn = 0; tn < S::TN; ++tn)
            for (int tm = 0; tm < S::TM; ++tm) {
                // d[lane][i]: the two halves (as tags) of 32-bit register i
                long d[64][8][2];
                for (int l = 0; l < 64; ++l)
                    for (int i = 0; i < 8; ++i)
                        for (int h = 0; h < 2; ++h)
                            d[l][i][h] = tag(acc_m(wm0, tm, l), acc_n(wn0, tn, 2 * i + h, l));
                for (int pr = 0; pr < 2; ++pr) {
                    long v[64][4][2];
                    for (int w = 0; w < 2; ++w) {  // the two exchanges: registers (4pr+w, 4pr+2+w)
                        const int xi = 4 * pr + w, yi = 4 * pr + 2 + w;
                        for (int l = 0; l < 64; ++l)
                            for (int h = 0; h < 2; ++h) {
                                const long x = l < 32 ? d[l][xi][h] : d[l - 32][yi][h];
                                const long y = l < 32 ? d[l + 32][xi][h] : d[l][yi][h];
                                v[l][w][h] = x;       // result 0 -> dword w of the piece
                                v[l][2 + w][h] = y;   // result 1 -> dword 2+w
                            }
                    }
                    std::vector<int> slot_seen(64, -1);
                    for (int l = 0; l < 64; ++l) {
                        const int row = epi_piece_row(tm, l), c = epi_piece_index(tn, pr, l);
                        const int off = epi_lds_offset<S>(row, c);
                        if (off < 0 || off + 16 > S::WTM * S::WTN * 2 || off % 16) { bad++; continue; }
                        const int slot = (off % 256) / 16;
                        if (slot_seen[16 * (l / 16) + slot]++ != -1) bad++;
                        for (int e = 0; e < 8; ++e) {
                            long &t = lds[off / 2 + e];
                            if (t != -1) bad++;
                            t = v[l][e / 2][e % 2];
                        }
                    }
                }
            }
        for (long t : lds)
            if (t == -1) bad++;
        // read-back
        for (int k = 0; k < S::WTM / (64 / CH); ++k) {
            std::vector<int> slot_seen(64, -1);
            for (int l = 0; l < 64; ++l) {
                const int row = epi_read_row<S>(k, l), c = epi_read_piece<S>(l);
                const int off = epi_lds_offset<S>(row, c);
                const int slot = (off % 256) / 16;
                if (slot_seen[16 * (l / 16) + slot]++ != -1) bad++;
                for (int e = 0; e < 8; ++e)
                    if (lds[off / 2 + e] != tag(wm0 + row, wn0 + 8 * c + e)) bad++;
            }
        }
    }
    return bad;
}

extern "C" long emu_check_epilogue(int config) {
    switch (config) {
        case 0: return check_epilogue<E256>();
        case 1: return check_epilogue<E128>();
        case 2: return check_epilogue<E64>();
        case 3: return check_epilogue<EP64>();
        case 4: return check_epilogue<E256w8>();
        case 5: return check_epilogue<E256w8x32>();
        case 6: return check_epilogue<EP256x128>();
        case 7: return check_epilogue<EP128x256>();
        default: return -1;
    }
}

// ---------------------------------------------------------------------------
// Block-scaled (MX) kernel k_mx: direct-to-LDS loads of 128 bytes of K per
// row and stage (16-byte chunks, A and B (given N x K) tiles alike), the
// stage's scale dwords (buffer_load_dword ... lds, one per lane, spread over
// the waves), the 16-byte fragment reads and scale reads of each 64-deep
// step, and v_mfma_scale_f32_32x32x64_f8f6f4 with its measured layouts: an
// 8-bit operand lane l holds k = 16*(l/32)+e and 32+16*(l/32)+e (e < 16),
// bytes 0..15 of lanes l%32 and l%32+32 are scaled by lane l%32's scale byte
// and bytes 16..31 by lane l%32+32's; a 4-bit lane holds 32 consecutive k,
// k = 32*(l/32)+e, scaled by its own scale byte.
// ---------------------------------------------------------------------------
namespace {

double emu_minifloat(unsigned code, int eb, int mb, int bias) {
    unsigned s = (code >> (eb + mb)) & 1, e = (code >> mb) & ((1u << eb) - 1), f = code & ((1u << mb) - 1);
    double v = e == 0 ? std::ldexp((double)f, 1 - bias - mb) : std::ldexp((double)((1u << mb) + f), (int)e - bias - mb);
    return s ? -v : v;
}

// hw format code: 0 E4M3, 1 E5M2, 4 E2M1 (finite codes only)
double emu_decode(int hw, unsigned c) {
    if (hw == 0) return emu_minifloat(c & 0xff, 4, 3, 7);
    if (hw == 1) return emu_minifloat(c & 0xff, 5, 2, 15);
    return emu_minifloat(c & 0xf, 2, 1, 1);
}

struct MxProb {
    int M, N, K, hw;
    const uint8_t *A, *B, *SA, *SB;  // codes (A: M rows, B: N rows), scales
    long lda, ldb, ldsa, ldsb;       // bytes per row
    uint16_t *C;
    long ldc;
};

template <class S>
void run_mx(const MxProb &p, Errs &er, std::vector<int> &cover) {
    const int EPB = p.hw == 4 ? 2 : 1;
    const int KPS = S::RA * EPB, SBR = KPS / 32, KSTEPS = KPS / 64;
    const int SC_A = S::BM * SBR, SC_B = S::BN * SBR;
    const int STAGE = S::STAGE_BYTES + SC_A + SC_B;
    const int NSA = SC_A / 256, NSB = SC_B / 256, SPW = (NSA + NSB) / S::WAVES;
    if ((NSA + NSB) % S::WAVES || SPW < 1 || NSA % SPW || S::RA != 128) { er.lds_oob++; return; }
    const int tiles_m = (p.M + S::BM - 1) / S::BM, tiles_n = (p.N + S::BN - 1) / S::BN, nwg = tiles_m * tiles_n;
    const int nk = (p.K + KPS - 1) / KPS, nkb = p.K / 32;
    std::vector<uint8_t> lds(STAGE);
    std::vector<int> lds_w(STAGE);
    std::vector<int> seen(nwg, 0);
    for (int pid = 0; pid < nwg; ++pid) {
        int tmi, tni;
        grouped_tile(xcd_remap(pid, nwg), tiles_m, tiles_n, 4, &tmi, &tni);
        if (tmi < 0 || tmi >= tiles_m || tni < 0 || tni >= tiles_n || seen[tmi * tiles_n + tni]++) {
            er.tile_dup++;
            continue;
        }
        const int m0 = tmi * S::BM, n0 = tni * S::BN;
        std::vector<double> acc((size_t)S::WAVES * S::TN * S::TM * 64 * 16, 0.0);
        for (int kt = 0; kt < nk; ++kt) {
            const int k0 = kt * KPS, kb0 = k0 / 32;
            const long k0b = k0 / EPB;
            std::fill(lds.begin(), lds.end(), 0xAB);
            std::fill(lds_w.begin(), lds_w.end(), 0);
            for (int w = 0; w < S::WAVES; ++w)
                for (int lane = 0; lane < 64; ++lane) {
                    for (int op = 0; op < 2; ++op)  // A then B, rows m or n
                        for (int i = 0; i < (op ? S::DMA_B : S::DMA_A); ++i) {
                            const ChunkRef c = dma_a_chunk<S>(w, i, lane);
                            const int dst = (op ? S::A_BYTES : 0) + (w * (op ? S::DMA_B : S::DMA_A) + i) * 1024 + 16 * lane;
                            const int r0 = op ? n0 : m0, lim = op ? p.N : p.M;
                            const bool ok = r0 + c.row < lim && k0 + 16 * EPB * c.chunk < p.K;
                            for (int b = 0; b < 16; ++b) {
                                if (dst + b >= S::STAGE_BYTES) { er.lds_oob++; continue; }
                                if (lds_w[dst + b]++) er.lds_multi++;
                                uint8_t v = 0;
                                if (ok) {
                                    const long row = r0 + c.row, byte = k0b + 16 * c.chunk + b;
                                    if (byte >= (long)p.K / EPB || byte >= (op ? p.ldb : p.lda)) er.oob_global++;
                                    else v = (op ? p.B : p.A)[row * (op ? p.ldb : p.lda) + byte];
                                }
                                lds[dst + b] = v;
                            }
                        }
                    for (int i = 0; i < SPW; ++i) {  // scale dwords
                        const int slab = w * SPW + i;
                        const bool sb = slab >= NSA;
                        const int q = (slab % NSA) * 64 + lane, row = q / (SBR / 4), d = q % (SBR / 4);
                        const int dst = S::STAGE_BYTES + (sb ? SC_A : 0) + (slab % NSA) * 256 + 4 * lane;
                        const int r0 = sb ? n0 : m0, lim = sb ? p.N : p.M;
                        const bool ok = r0 + row < lim && kb0 + 4 * d < nkb;
                        for (int b = 0; b < 4; ++b) {
                            if (dst + b >= STAGE) { er.lds_oob++; continue; }
                            if (lds_w[dst + b]++) er.lds_multi++;
                            uint8_t v = 0;
                            if (ok) {
                                const long col = kb0 + 4 * d + b;
                                if (col >= nkb || col >= (sb ? p.ldsb : p.ldsa)) er.oob_global++;
                                else v = (sb ? p.SB : p.SA)[(r0 + row) * (sb ? p.ldsb : p.ldsa) + col];
                            }
                            lds[dst + b] = v;
                        }
                    }
                }
            for (int b = 0; b < STAGE; ++b)
                if (lds_w[b] != 1) er.lds_multi++;
            // fragments, scales and MFMAs of every 64-deep step
            for (int w = 0; w < S::WAVES; ++w) {
                const int wm0 = (w / S::WN) * S::WTM, wn0 = (w % S::WN) * S::WTN;
                for (int J = 0; J < KSTEPS; ++J) {
                    // vals[op][t][lane][32] decoded codes, sc[op][t][lane] scale values
                    std::vector<double> vals((size_t)2 * 4 * 64 * 32, 0.0), sc((size_t)2 * 4 * 64, 0.0);
                    for (int op = 0; op < 2; ++op)  // 0: B operand (first, columns), 1: A operand (rows)
                        for (int t = 0; t < (op ? S::TM : S::TN); ++t) {
                            const int base = op ? 0 : S::A_BYTES, w0 = op ? wm0 : wn0;
                            for (int part = 0; part < (EPB == 1 ? 2 : 1); ++part) {
                                int addr[64];
                                for (int l = 0; l < 64; ++l) {
                                    const int row = w0 + 32 * t + l % 32, half = l / 32;
                                    const int chunk = EPB == 1 ? 4 * J + 2 * part + half : 2 * J + half;
                                    addr[l] = lds_a_offset<S>(row, chunk);
                                    if (addr[l] < 0 || addr[l] + 16 > S::A_BYTES || addr[l] % 16) er.lds_oob++;
                                }
                                for (int q = 0; q < 4; ++q) {
                                    int used[16] = {0};
                                    for (int l = 16 * q; l < 16 * q + 16; ++l)
                                        if (used[slot16(addr[l])]++) er.bank_conflict++;
                                }
                                for (int l = 0; l < 64; ++l)
                                    for (int b = 0; b < 16; ++b) {
                                        const uint8_t byte = lds[base + addr[l] + b];
                                        if (EPB == 1) {
                                            vals[(((size_t)op * 4 + t) * 64 + l) * 32 + 16 * part + b] = emu_decode(p.hw, byte);
                                        } else {
                                            vals[(((size_t)op * 4 + t) * 64 + l) * 32 + 2 * b] = emu_decode(p.hw, byte & 0xf);
                                            vals[(((size_t)op * 4 + t) * 64 + l) * 32 + 2 * b + 1] = emu_decode(p.hw, byte >> 4);
                                        }
                                    }
                            }
                            // the kernel's scale selection: the row's dword DW of the
                            // stage, shifted right by 8*(l/32), byte OPSEL of it
                            const int DW = EPB == 1 ? 0 : J / 2, OPSEL = EPB == 1 ? 2 * J : 2 * (J % 2);
                            for (int l = 0; l < 64; ++l) {
                                const int row = w0 + 32 * t + l % 32;
                                const int a = S::STAGE_BYTES + (op ? 0 : SC_A) + row * SBR + 4 * DW;
                                if (a + 4 > STAGE || a % 4) { er.lds_oob++; continue; }
                                uint32_t dword;
                                memcpy(&dword, &lds[a], 4);
                                const uint32_t byte = ((dword >> (8 * (l / 32))) >> (8 * OPSEL)) & 0xff;
                                sc[((size_t)op * 4 + t) * 64 + l] = std::ldexp(1.0, (int)byte - 127);
                            }
                        }
                    for (int tn = 0; tn < S::TN; ++tn)
                        for (int tm = 0; tm < S::TM; ++tm)
                            for (int l = 0; l < 64; ++l)
                                for (int r = 0; r < 16; ++r) {
                                    const int i = 8 * (r / 4) + 4 * (l / 32) + r % 4, j = l % 32;
                                    double d = 0;
                                    auto X = [&](int lane, int e) { return vals[(((size_t)0 * 4 + tn) * 64 + lane) * 32 + e]; };
                                    auto Y = [&](int lane, int e) { return vals[(((size_t)1 * 4 + tm) * 64 + lane) * 32 + e]; };
                                    auto sX = [&](int lane) { return sc[((size_t)0 * 4 + tn) * 64 + lane]; };
                                    auto sY = [&](int lane) { return sc[((size_t)1 * 4 + tm) * 64 + lane]; };
                                    if (EPB == 1) {
                                        for (int blk = 0; blk < 2; ++blk) {
                                            double s = 0;
                                            for (int h = 0; h < 2; ++h)
                                                for (int e = 0; e < 16; ++e) s += X(i + 32 * h, 16 * blk + e) * Y(j + 32 * h, 16 * blk + e);
                                            d += sX(i + 32 * blk) * sY(j + 32 * blk) * s;
                                        }
                                    } else {
                                        for (int h = 0; h < 2; ++h) {
                                            double s = 0;
                                            for (int e = 0; e < 32; ++e) s += X(i + 32 * h, e) * Y(j + 32 * h, e);
                                            d += sX(i + 32 * h) * sY(j + 32 * h) * s;
                                        }
                                    }
                                    acc[((((size_t)w * S::TN + tn) * S::TM + tm) * 64 + l) * 16 + r] += d;
                                }
                }
            }
        }
        for (int w = 0; w < S::WAVES; ++w) {
            const int wm0 = (w / S::WN) * S::WTM, wn0 = (w % S::WN) * S::WTN;
            for (int tn = 0; tn < S::TN; ++tn)
                for (int tm = 0; tm < S::TM; ++tm)
                    for (int l = 0; l < 64; ++l)
                        for (int r = 0; r < 16; ++r) {
                            const int m = m0 + acc_m(wm0, tm, l), n = n0 + acc_n(wn0, tn, r, l);
                            const double v = acc[((((size_t)w * S::TN + tn) * S::TM + tm) * 64 + l) * 16 + r];
                            if (m >= p.M || n >= p.N) continue;
                            p.C[(size_t)m * p.ldc + n] = f2h((float)(v > 0.0 ? v : 0.0));
                            cover[(size_t)m * p.N + n]++;
                        }
        }
    }
}

}  // namespace

// config 0: 256 x 256, eight waves, two stages; 1: 128 x 128, four waves.
// hw: 0 E4M3, 1 E5M2, 4 E2M1. Leading dimensions in bytes. Returns 0, and
// the error counts in errs[0..7] (global out of range, LDS written twice or
// never, LDS out of range, bank conflicts, C written twice, C missing, C
// outside, tile mapping).
extern "C" int emu_gemm_relu_mx(int config, int hw, int M, int N, int K, const uint8_t *A, long lda, const uint8_t *SA,
                                long ldsa, const uint8_t *B, long ldb, const uint8_t *SB, long ldsb, uint16_t *C,
                                long ldc, long *errs) {
    MxProb p{M, N, K, hw, A, B, SA, SB, lda, ldb, ldsa, ldsb, C, ldc};
    Errs er;
    std::vector<int> cover((size_t)M * N, 0);
    if (config == 0)
        run_mx<TileShape<256, 256, 64, 2, 4, 2>>(p, er, cover);
    else if (config == 1)
        run_mx<TileShape<128, 128, 64, 2, 2, 3>>(p, er, cover);
    else
        return -1;
    for (int c : cover) {
        if (c == 0) er.c_missing++;
        if (c > 1) er.c_multi++;
    }
    long v[8] = {er.oob_global, er.lds_multi, er.lds_oob, er.bank_conflict, er.c_multi, er.c_missing, er.c_outside,
                 er.tile_dup};
    memcpy(errs, v, sizeof v);
    return 0;
}
