// Wide-row streaming GEMM kernel for gfx950 (CDNA4): the default for large
// products.  Included by the instance translation units (one per operand
// width, compiled in parallel).
#pragma once

#include "gemm_common.h"

namespace tg {

// 256 x 256 tile, 4 waves of 128 x 128, stages of 128 bytes of K per operand
// row copied global -> LDS by LDS-DMA.  Each group of 8 lanes of a copy reads
// one whole 128-byte row segment (a full cache line), which halves the number
// of memory requests per byte against 64-byte rows; the L2 -> LDS request rate
// is what bounds the copy path of these kernels.  Per stage each wave runs four
// slabs of 16 MFMAs (32 bytes of K each).
//
// LDS holds NS slots of 32 KiB; a slot holds one operand's half of a stage
// (256 rows x 128 bytes).  Half-stage h (stage h/2, A if h is even, B if odd)
// lives in slot h % NS.  NS = 4 is plain double buffering; NS = 5 fills the
// 160 KiB of a CU and keeps one and a half stages of copies in flight.
//
// Schedule of stage s (barrier B_s sits between slabs 2 and 3):
//   slab 0: read slab 1 fragments; copy half-stage 2s + NS - 1
//   slab 1: read slab 2 fragments
//   slab 2: read slab 3 fragments
//   wait for this wave's reads and for its copies of stage s+1; B_s
//   (stage s+1 is published, and every wave is done reading stage s)
//   slab 3: read slab 0 of stage s+1; copy half-stage 2s + NS into the slot
//   stage s's A half just left
// A slot is refilled only after the barrier that ends the reads of the
// half-stage NS places earlier, which the two copy points respect.
//
// Knobs: GM tile-order group; RS = the MFMAs of a slab over which its 8
// fragment reads are spread; ADDR 0 = 64-bit per-lane addresses, 1 = buffer
// resources with 32-bit offsets; SCHED 0 = copies in bursts in slabs 0 and 3,
// 1 = one copy every 4 MFMAs over the whole stage (5 slots); EPI bit 0 =
// nontemporal D stores (D lines then do not displace operand panels in L2,
// measured ~2 % faster main loop when D columns start on 128-byte lines; when
// they do not, the partial lines at the tile edges make them about 20 %
// slower on the whole product, and the twins without the bit are used), bit 1 =
// fp32 D through an LDS transpose so each store writes a whole 1 KiB row run
// (no faster for line-aligned D, where the write burst at the end of a tile
// is bound by memory bandwidth either way; 2.5 % faster when D columns are
// only 4-byte aligned, so the plain-store twins carry it), bit 2 =
// the same for bf16/fp16 D, whose direct stores would write 64-byte halves of
// lines; bit 3 = the instance also carries the softmax epilogue (kept out of
// the plain instances, whose epilogue it would bloat); bit 4 = interior tiles
// transpose 4 x 4 register groups across lane quads and store 4 consecutive m
// per lane as one 8-byte vector for 16-bit D (measured: the bf16-D epilogue
// drops from about 31k to 21k cycles against the LDS transpose; the same for
// fp32 D as 16-byte vectors measured slower than direct stores, since fp32 D
// is bound by the write burst and the shuffles add VALU work), bit 6 =
// 8-bit operands with block scales (their loads sit in the main loop, and the
// waits the compiler puts before their use also wait for copies, so the
// instances without scales do not carry them).  LC = 16: copies by LDS-DMA,
// which needs 16-byte aligned row starts; LC = 4 or 2: rows only 4- or 2-byte
// aligned, copied through registers (see the register-staged schedule below).
template <int DT, int GM, int NS, int RS, int ADDR, int SCHED, int EPI, int LC>
__global__ __launch_bounds__(256, 1) void gemm_wide_kernel(GemmArgs p) {
    select_batch(p);
    constexpr int BM = 256, BN = 256, WM = 2;
    constexpr bool F8 = (DT == TG_E4M3 || DT == TG_E5M2);
    constexpr bool F4 = (DT == TG_E2M1);          // packed two per byte
    constexpr bool F6 = (DT == TG_E2M3 || DT == TG_E3M2);  // packed four per three bytes
    constexpr int ES = (DT == TG_F32) ? 4 : (F8 || F4 || F6) ? 1 : 2;  // bytes per element (packed: per byte)
    constexpr int EPC = F4 ? 32 : 16 / ES;       // K elements per 16-byte chunk (not for 6-bit)
    constexpr int BKE = F4 ? 2 * kRowBytes : F6 ? 128 : kRowBytes / ES;  // K elements per stage
    constexpr int STB = F6 ? 96 : kRowBytes;     // bytes of each row one stage covers
    constexpr int WTM = 128, WTN = 128;          // output owned by one wave
    constexpr int FM = WTM / 32, FN = WTN / 32;  // 32 x 32 MFMA blocks per wave
    constexpr int NC = BM / (8 * 4);             // 1 KiB copies per wave per half-stage
    constexpr int NR = FM + FN;                  // fragment reads per slab
    constexpr int MF = FM * FN;                  // MFMAs per slab
    constexpr int SLOT = BM * kRowBytes;         // 32 KiB
    static_assert(BM == BN && NC == 8 && MF == 16, "schedule assumes 8 copies per half-stage, 16 MFMAs a slab");
    static_assert(NS == 4 || NS == 5, "4 or 5 half-stage slots");
    static_assert(SCHED == 0 || NS == 5, "the spread copy schedule needs 5 slots");
    static_assert(RS >= 1 && RS <= MF, "reads spread over at most one slab");
    static_assert(LC == 16 || (ADDR == 1 && NS == 4 && !F8 && (ES == 2 ? LC >= 2 : ES == 4 ? LC == 4 : LC >= 1)),
                  "register-staged copies: buffer addressing, 4 slots, 16-bit, fp32 or 4-bit operands");
    static_assert(!F4 || (EPI & 8) == 0, "no softmax epilogue on 4-bit instances");
    static_assert(!F6 || (ADDR == 1 && LC == 16 && NS == 5 && SCHED == 1 && (EPI & 8) == 0),
                  "6-bit operands: buffer addressing (the copies of the two unused chunks of a row fall "
                  "outside the range), 16-byte aligned rows, the spread five-slot schedule");
    static_assert(!F4 || (EPI & 64) == 0 || (LC == 16 && NS == 4 && SCHED == 0 && ADDR == 1),
                  "4-bit block scales ride the four-slot schedule, the fifth slot holds them");
    // a chunk of the ragged last stage, exact zeros for k >= K
    auto tail_chunk = [](const char* row, int k0, int K) {
        if constexpr (F4)
            return load_chunk_bounded_e2m1(row, k0, K);
        else
            return load_chunk_bounded<ES>(row, k0, K);
    };

    // the whole 160 KiB of a CU (one workgroup per CU): the ring uses NS
    // slots, the transposing epilogues may use all of it
    constexpr int LDS_BYTES = 5 * SLOT;
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave % WM, wave_n = wave / WM;

    const TileCoord tile = grouped_tile(p.tile, p.tiles_m, p.tiles_n, GM);
    const int m0 = tile.tm * BM, n0 = tile.tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    const unsigned lds_base = __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(smem))));

    // copy sources.  ADDR 0: 64-bit addresses, rows past M or N clamp to
    // the last row.  ADDR 1: buffer resources over the tile's valid rows, 32-bit
    // row offsets (the plan keeps 256 * stride below 2^31); rows past M or N
    // fall outside the range and load zeros.  Either way those rows only feed
    // accumulators that are never stored.
    const char* src[2][NC];
    unsigned voff[2][NC];
    i32x4 rsrc[2];
    if constexpr (ADDR == 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int j = wave * NC + i;
            src[0][i] = p.A + static_cast<int64_t>(min(m0 + dma128_row(j, lane), M - 1)) * p.lda_b +
                        dma128_chunk(j, lane) * kChunkBytes;
            src[1][i] = p.B + static_cast<int64_t>(min(n0 + dma128_row(j, lane), N - 1)) * p.ldb_b +
                        dma128_chunk(j, lane) * kChunkBytes;
        }
    } else {
        rsrc[0] = buffer_rsrc(p.A + static_cast<int64_t>(m0) * p.lda_b,
                              static_cast<unsigned>(min(BM, M - m0) * p.lda_b));
        rsrc[1] = buffer_rsrc(p.B + static_cast<int64_t>(n0) * p.ldb_b,
                              static_cast<unsigned>(min(BN, N - n0) * p.ldb_b));
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int j = wave * NC + i;
            voff[0][i] = static_cast<unsigned>(dma128_row(j, lane) * p.lda_b) + dma128_chunk(j, lane) * kChunkBytes;
            voff[1][i] = static_cast<unsigned>(dma128_row(j, lane) * p.ldb_b) + dma128_chunk(j, lane) * kChunkBytes;
            if (F6 && dma128_chunk(j, lane) >= STB / kChunkBytes)  // past the 96 bytes of a 6-bit stage
                voff[0][i] = voff[1][i] = 0x80000000u;             // beyond every range: nothing is read
        }
    }
    // copy i of operand o (0: A, 1: B) of stage t into slot `slot`
    auto copy = [&](int o, int i, int t, int slot) {
        const unsigned dst = __builtin_amdgcn_readfirstlane(lds_base + slot * SLOT + (wave * NC + i) * 1024);
        if constexpr (ADDR == 0)
            dma16(src[o][i] + static_cast<int64_t>(t) * STB, dst);
        else
            dma16_buf(rsrc[o], voff[o][i], __builtin_amdgcn_readfirstlane(t * STB), dst);
    };
    auto wrap = [](int x) { return x >= NS ? x - NS : x; };

    // fragment read offsets within a slot (block steps are 32 rows, which
    // keep the swizzle)
    int mread[4], nread[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        mread[q] = wave_m * WTM * kRowBytes + lds_chunk_offset(frag_row(lane), frag_chunk(lane, q));
        nread[q] = wave_n * WTN * kRowBytes + lds_chunk_offset(frag_row(lane), frag_chunk(lane, q));
    }
    // read r of slab q from slots (sa, sb); m-side and n-side fragments alternate
    auto read = [&](int r, int q, int sa, int sb, u32x4 (&fa)[FM], u32x4 (&fb)[FN]) {
        const int blk = r >> 1;
        if ((r & 1) == 0)
            fa[blk] = *reinterpret_cast<const u32x4*>(smem + sa * SLOT + mread[q] + blk * 32 * kRowBytes);
        else
            fb[blk] = *reinterpret_cast<const u32x4*>(smem + sb * SLOT + nread[q] + blk * 32 * kRowBytes);
    };
    // the NR fragment reads of a slab go out after the first RS of its MFMAs
    auto reads_at = [&](int m, auto&& f) {
        if (m < RS) {
#pragma unroll
            for (int k = (m * NR + RS - 1) / RS; k < ((m + 1) * NR + RS - 1) / RS; ++k) f(k);
        }
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nfull = K / BKE;
    if constexpr (F8 || F6) {
        // 8-bit operands: a stage (128 k) is two 32x32x64 MFMAs per block.
        // The fragments of slabs 2p and 2p + 1 (chunks 4p + h and 4p + 2 + h
        // of half-wave h) together feed MFMA pair p; pair 0 runs while slabs
        // 2 and 3 are read and the copies of slabs 0-2 of the 16-bit schedule
        // go out (12), pair 1 after the barrier while slabs 0 and 1 of the
        // next stage are read and the last 4 copies go out, so the copy
        // order and the wait counts are those of the 16-bit schedule.  Block
        // scales (when given) come from the lane's rows, as in the
        // register-staged kernel.
        // 6-bit operands run the same schedule: a stage is 128 k as well (96
        // bytes, chunks 0-5 of each LDS row), and pair p takes the 24 bytes
        // [48p + 24h, 48p + 24h + 24) of half-wave h's row as three 8-byte
        // reads, each inside one chunk (24 reads a pair instead of 16).
        static_assert(SCHED == 1 && NS == 5, "the 8-bit schedule follows the spread copy schedule");
        constexpr bool SC = (EPI & 64) != 0;  // the instance applies block scales
        const int nk = nfull + ((K % BKE) != 0 ? 1 : 0);  // stages including a ragged one
        u32x4 g[4][FM], h[4][FN];
        u32x2 g6[2][FM][3], h6[2][FN][3];  // 6-bit fragments of pairs 0 and 1
        // 6-bit read offsets within a slot: piece i of pair pp
        int m6[2][3], n6[2][3];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int b = 48 * pp + 24 * (lane >> 5) + 8 * i;
                m6[pp][i] = wave_m * WTM * kRowBytes + lds_chunk_offset(frag_row(lane), b >> 4) + (b & 15);
                n6[pp][i] = wave_n * WTN * kRowBytes + lds_chunk_offset(frag_row(lane), b >> 4) + (b & 15);
            }
        // 6-bit read k (0..23) of pair pp: fragment r = k / 3 (even: m-side
        // block r / 2, odd: n-side), piece k % 3
        auto read6 = [&](int k, int pp, int sa, int sb, u32x2 (&fa)[FM][3], u32x2 (&fb)[FN][3]) {
            const int r = k / 3, i = k % 3, blk = r >> 1;
            if ((r & 1) == 0)
                fa[blk][i] = *reinterpret_cast<const u32x2*>(smem + sa * SLOT + m6[pp][i] + blk * 32 * kRowBytes);
            else
                fb[blk][i] = *reinterpret_cast<const u32x2*>(smem + sb * SLOT + n6[pp][i] + blk * 32 * kRowBytes);
        };
        // the reads of pair pp (from slots sa/sb) that go out after MFMA m of 16
        auto reads6_at = [&](int m, int pp, int sa, int sb, u32x2 (&fa)[FM][3], u32x2 (&fb)[FN][3]) {
#pragma unroll
            for (int k = (3 * m + 1) / 2; k < (3 * (m + 1) + 1) / 2; ++k) read6(k, pp, sa, sb, fa, fb);
        };
        // block scales of the lane's rows for the stage being consumed: one
        // dword per row (the stage's four 32-k blocks), loaded at the end of
        // the previous stage, after its copies, so that the waits the
        // compiler puts in front of their first use only also cover copies
        // issued a stage earlier
        unsigned scm[FM], scn[FN];
        const int nblk = (K + 31) / 32;
        // scale loads through buffer resources over the tile's scale rows:
        // 32-bit per-lane offsets and the rest in SGPRs, which keeps the loop
        // free of spills (a spill reload waits for every copy in flight).
        // Rows past M or N fall outside the range and read 0, i.e. a tiny
        // scale on rows whose data loads as zeros.
        // (an absent operand gets an empty range and is never loaded)
        const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
            p.scale_a ? const_cast<unsigned char*>(p.scale_a + static_cast<int64_t>(m0) * p.lds_a) : p.D,
            static_cast<short>(0), p.scale_a ? static_cast<int>(static_cast<unsigned>(min(BM, M - m0) * p.lds_a)) : 0,
            0x00020000);
        const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
            p.scale_b ? const_cast<unsigned char*>(p.scale_b + static_cast<int64_t>(n0) * p.lds_b) : p.D,
            static_cast<short>(0), p.scale_b ? static_cast<int>(static_cast<unsigned>(min(BN, N - n0) * p.lds_b)) : 0,
            0x00020000);
        // the whole row offset sits in the per-lane offset, which is what the
        // range check looks at (the scalar offset only carries the stage)
        unsigned vo_a[FM], vo_b[FN];
#pragma unroll
        for (int j = 0; j < FM; ++j) vo_a[j] = static_cast<unsigned>((wave_m * WTM + 32 * j + frag_row(lane)) * p.lds_a);
#pragma unroll
        for (int i = 0; i < FN; ++i) vo_b[i] = static_cast<unsigned>((wave_n * WTN + 32 * i + frag_row(lane)) * p.lds_b);
        auto load_scales = [&](int t) {
            if constexpr (!SC) return;
            if (p.scale_a) {
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    scm[j] = __builtin_amdgcn_raw_buffer_load_b32(rs_a, static_cast<int>(vo_a[j]), 4 * t, 0);
            } else {
#pragma unroll
                for (int j = 0; j < FM; ++j) scm[j] = 0x7F7F7F7Fu;
            }
            if (p.scale_b) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    scn[i] = __builtin_amdgcn_raw_buffer_load_b32(rs_b, static_cast<int>(vo_b[i]), 4 * t, 0);
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) scn[i] = 0x7F7F7F7Fu;
            }
        };
        // pair pp of stage t; scale blocks past the last one of K count as 1
        auto pair = [&](int pp, int t, auto&& side) {
            const int sub = 2 * pp + (lane >> 5);
            const bool live = 4 * t + sub < nblk;
            (void)live;
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                const int i = m / FM, j = m % FM;
                int sn = 127, sm = 127;
                if constexpr (SC) {
                    sn = live ? static_cast<int>((scn[i] >> (8 * sub)) & 0xFFu) : 127;
                    sm = live ? static_cast<int>((scm[j] >> (8 * sub)) & 0xFFu) : 127;
                }
                if constexpr (F6) {
                    acc[i][j] = mfma_f6<DT == TG_E2M3 ? 2 : 3>(h6[pp][i], g6[pp][j], acc[i][j], sn, sm);
                } else {
                    const u32x4 nn[2] = {h[2 * pp][i], h[2 * pp + 1][i]};
                    const u32x4 mm[2] = {g[2 * pp][j], g[2 * pp + 1][j]};
                    acc[i][j] = mfma_f8<DT>(nn, mm, acc[i][j], sn, sm);
                }
                side(m);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (nfull > 0) {
            constexpr int PRO = 3 * NC + NC / 2;  // prologue copies, as in the 16-bit schedule
#pragma unroll
            for (int c = 0; c < PRO; ++c) {
                const int hs = c / NC;
                copy(hs & 1, c % NC, min(hs >> 1, nfull - 1), hs);
            }
            wait_vm<PRO - 2 * NC>();
            barrier();
            if constexpr (F6) {
#pragma unroll
                for (int k = 0; k < 3 * NR; ++k) read6(k, 0, 0, 1, g6[0], h6[0]);
            } else {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    read(r, 0, 0, 1, g[0], h[0]);
                    read(r, 1, 0, 1, g[1], h[1]);
                }
            }
            load_scales(0);
            int slot0 = 0;
            for (int s = 0; s < nfull; ++s) {
                const int sa = slot0, sb = wrap(slot0 + 1);
                const int na = wrap(slot0 + 2), nb = wrap(slot0 + 3);
                const int slot_h0 = wrap(slot0 + NS - 1);
                const int t1 = min(s + 1, nfull - 1), t2 = min(s + 2, nfull - 1);
                pair(0, s, [&](int m) {
                    if constexpr (F6)
                        reads6_at(m, 1, sa, sb, g6[1], h6[1]);
                    else if (m < NR)
                        read(m, 2, sa, sb, g[2], h[2]);
                    else
                        read(m - NR, 3, sa, sb, g[3], h[3]);
                    if ((m & 3) != 3) {
                        const int c = m - (m >> 2);  // 0 .. 11
                        if (c < 4) copy(1, NC / 2 + c, t1, nb);
                        else if (c < 8) copy(0, c - 4, t2, slot_h0);
                        else copy(0, NC / 2 + c - 8, t2, slot_h0);
                    }
                });
                asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
                wait_vm<(NS - 4) * NC>();
                barrier();
                // on the last stage the reads below fetch values that go unused
                pair(1, s, [&](int m) {
                    if constexpr (F6)
                        reads6_at(m, 0, na, nb, g6[0], h6[0]);
                    else if (m < NR)
                        read(m, 0, na, nb, g[0], h[0]);
                    else
                        read(m - NR, 1, na, nb, g[1], h[1]);
                    if ((m & 3) == 1) copy(1, m >> 2, t2, sa);
                });
                if (s + 1 < nk) load_scales(s + 1);
                slot0 = na;
            }
            wait_vm<0>();  // no copy outlives the loop
        }
        if (K % BKE != 0) {
            // ragged last stage through registers into slots 0 (A) and 1 (B)
            __syncthreads();
            const int c = stage_chunk(tid);
            const int k0 = nfull * BKE + c * EPC;
            // 6-bit rows: the stage starts at byte 96 * nfull, and every bit
            // from bit 6K of the row on is zero
            const int64_t b0 = static_cast<int64_t>(nfull) * STB + c * kChunkBytes, kbits = 6 * static_cast<int64_t>(K);
#pragma unroll
            for (int i = 0; i < BM / 32; ++i) {
                const int r = stage_row(tid, i);
                const char* arow = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
                const char* brow = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
                *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) =
                    F6 ? load_chunk_bounded_bits(arow, b0, kbits) : tail_chunk(arow, k0, K);
                *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) =
                    F6 ? load_chunk_bounded_bits(brow, b0, kbits) : tail_chunk(brow, k0, K);
            }
            if (nfull == 0) load_scales(0);  // otherwise loaded at the end of the last full stage
            __syncthreads();
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                if (nfull * BKE + pp * (BKE / 2) >= K) break;  // the rest of the stage is zeros
                if constexpr (F6) {
#pragma unroll
                    for (int k = 0; k < 3 * NR; ++k) read6(k, pp, 0, 1, g6[pp], h6[pp]);
                } else {
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        read(r, 2 * pp, 0, 1, g[2 * pp], h[2 * pp]);
                        read(r, 2 * pp + 1, 0, 1, g[2 * pp + 1], h[2 * pp + 1]);
                    }
                }
                pair(pp, nfull, [](int) {});
            }
        }
    } else if constexpr (F4 && (EPI & 64) != 0) {
        // 4-bit operands with block scales.  A stage is 256 k, i.e. eight
        // 32-k scale blocks per row, and slab q of a stage is one 32x32x64
        // MFMA per block whose half-wave h takes k-block 2q + h (mfma_f4).
        // The scales reach the lanes through LDS: a 16-byte piece of each
        // operand row holds the blocks of two stages (a "pair"), and LDS-DMA
        // copies the pieces of pair p -- two copies per wave, 64 rows each --
        // into the fifth slot (which the four-slot ring leaves free) during
        // slab 0 of stage 2p - 2.  Every barrier of this schedule waits for all
        // of the wave's copies, so pair p is complete at the barrier of stage
        // 2p - 2; its buffer (p & 1) was last read in slab 3 of stage 2p - 4.
        // After each barrier (slab 3 of stage t - 1) a lane reads the 8
        // bytes of stage t for each of its rows and permutes them into one
        // dword whose byte q is block 2q + h, which the MFMA of slab q selects.
        // The scale loads thus go through the same explicit waits as the
        // operand copies instead of the compiler's own (which cannot see the
        // copies and would wait for all of them).
        u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
        constexpr int SC_BUF = 2 * BM * 16;  // one pair of stages: A rows, then B rows, 16 bytes each
        static_assert(4 * SLOT + 2 * SC_BUF <= LDS_BYTES, "scale buffers fit the fifth slot");
        const bool has_a = p.scale_a != nullptr, has_b = p.scale_b != nullptr;  // uniform
        const i32x4 srs[2] = {
            buffer_rsrc(has_a ? p.scale_a + static_cast<int64_t>(m0) * p.lds_a : nullptr,
                        has_a ? static_cast<unsigned>(min(BM, M - m0) * p.lds_a) : 0u),
            buffer_rsrc(has_b ? p.scale_b + static_cast<int64_t>(n0) * p.lds_b : nullptr,
                        has_b ? static_cast<unsigned>(min(BN, N - n0) * p.lds_b) : 0u)};
        const unsigned svoff[2] = {static_cast<unsigned>((64 * wave + lane) * p.lds_a),
                                   static_cast<unsigned>((64 * wave + lane) * p.lds_b)};
        // scale pieces of pair pr (stages 2pr, 2pr + 1) into buffer pr & 1;
        // rows past M or N fall outside the range and read zeros (they only
        // scale accumulators that are never stored)
        auto scale_copy = [&](int pr) {
#pragma unroll
            for (int o = 0; o < 2; ++o) {
                const unsigned dst = __builtin_amdgcn_readfirstlane(lds_base + 4 * SLOT + (pr & 1) * SC_BUF +
                                                                     o * (BM * 16) + wave * 64 * 16);
                dma16_buf(srs[o], svoff[o], __builtin_amdgcn_readfirstlane(16 * pr), dst);
            }
        };
        const unsigned sel = (lane >> 5) ? 0x07050301u : 0x06040200u;  // bytes h, 2 + h, 4 + h, 6 + h
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        unsigned scm[FM], scn[FN], nscm[FM], nscn[FN];
        // the lane's scales of stage t from its pair buffer
        auto read_scales = [&](int t, unsigned (&sm)[FM], unsigned (&sn)[FN]) {
            const char* buf = smem + 4 * SLOT + ((t >> 1) & 1) * SC_BUF + (t & 1) * 8;
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(buf + (wave_m * WTM + 32 * j + frag_row(lane)) * 16);
                sm[j] = has_a ? __builtin_amdgcn_perm(v.y, v.x, sel) : 0x7F7F7F7Fu;
            }
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const u32x2 v =
                    *reinterpret_cast<const u32x2*>(buf + BM * 16 + (wave_n * WTN + 32 * i + frag_row(lane)) * 16);
                sn[i] = has_b ? __builtin_amdgcn_perm(v.y, v.x, sel) : 0x7F7F7F7Fu;
            }
        };
        // slab Q of the stage: 16 MFMAs, side(m) after MFMA m
        auto slab_sc = [&](auto qc, const u32x4 (&fa)[FM], const u32x4 (&fb)[FN], auto&& side) {
            constexpr int Q = decltype(qc)::value;
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                const int i = m / FM, j = m % FM;
                acc[i][j] = mfma_f4<Q>(fb[i], fa[j], acc[i][j], static_cast<int>(scn[i]), static_cast<int>(scm[j]));
                side(m);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        using Q0 = std::integral_constant<int, 0>;
        using Q1 = std::integral_constant<int, 1>;
        using Q2 = std::integral_constant<int, 2>;
        using Q3 = std::integral_constant<int, 3>;

        if (nfull > 0) {
            // prologue: the scales of pair 0 first, then half-stages 0 .. 2;
            // the wait leaves only half-stage 2 in flight
            scale_copy(0);
            constexpr int PRO = 3 * NC;
#pragma unroll
            for (int c = 0; c < PRO; ++c) {
                const int h = c / NC;
                copy(h & 1, c % NC, min(h >> 1, nfull - 1), h);
            }
            wait_vm<PRO - 2 * NC>();
            barrier();
#pragma unroll
            for (int r = 0; r < NR; ++r) read(r, 0, 0, 1, fa0, fb0);
            read_scales(0, scm, scn);

            int slot0 = 0;  // slot of stage s's A half, (2s) % 4
            for (int s = 0; s < nfull; ++s) {
                const int sa = slot0, sb = slot0 + 1;
                const int na = (slot0 + 2) & 3, nb = (slot0 + 3) & 3;
                const int t1 = min(s + 1, nfull - 1), t2 = min(s + 2, nfull - 1);
                const bool pair_copy = (s & 1) == 0 && s + 2 < nfull;
                // slab 0: the copies of B(s+1) (into nb), and on even stages
                // the scales of the pair of stages s+2 and s+3
                slab_sc(Q0{}, fa0, fb0, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 1, sa, sb, fa1, fb1); });
                    if (m & 1) copy(1, m >> 1, t1, nb);
                    if (m == 2 && pair_copy) scale_copy((s >> 1) + 1);
                });
                slab_sc(Q1{}, fa1, fb1, [&](int m) { reads_at(m, [&](int k) { read(k, 2, sa, sb, fa0, fb0); }); });
                slab_sc(Q2{}, fa0, fb0, [&](int m) { reads_at(m, [&](int k) { read(k, 3, sa, sb, fa1, fb1); }); });
                asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
                wait_vm<0>();
                barrier();
                // slab 3: read slab 0 and the scales of stage s+1; copy A(s+2)
                // into the slot A(s) just left (on the last stage the reads
                // fetch values that go unused)
                slab_sc(Q3{}, fa1, fb1, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 0, na, nb, fa0, fb0); });
                    if (m & 1) copy(0, m >> 1, t2, sa);
                    if (m == 4) read_scales(s + 1, nscm, nscn);
                });
#pragma unroll
                for (int j = 0; j < FM; ++j) scm[j] = nscm[j];
#pragma unroll
                for (int i = 0; i < FN; ++i) scn[i] = nscn[i];
                slot0 = na;
            }
            wait_vm<0>();  // no copy outlives the loop
        }

        if (K % BKE != 0) {
            // ragged last stage through registers into slots 0 (A) and 1 (B);
            // k >= K become exact zeros, and its scales come straight from
            // memory: blocks past the last one of K count as 1 (their elements
            // are zeros, and a NaN scale byte there must not reach the sums),
            // rows past M or N are not read
            __syncthreads();
            const int c = stage_chunk(tid);
            const int k0 = nfull * BKE + c * EPC;
#pragma unroll
            for (int i = 0; i < BM / 32; ++i) {
                const int r = stage_row(tid, i);
                const char* arow = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
                const char* brow = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
                *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) = tail_chunk(arow, k0, K);
                *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) = tail_chunk(brow, k0, K);
            }
            const int nblk = (K + 31) / 32;
            const int h = lane >> 5;
            unsigned live = 0;  // byte q: 0xFF when block 8 * nfull + 2q + h holds elements below K
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (8 * nfull + 2 * q + h < nblk) live |= 0xFFu << (8 * q);
            auto tail_scale = [&](const unsigned char* sc, int64_t lds, int row, int rows) {
                if (!sc || row >= rows) return 0x7F7F7F7Fu;
                const u32x2 v = *reinterpret_cast<const u32x2*>(sc + static_cast<int64_t>(row) * lds + 8 * nfull);
                return (__builtin_amdgcn_perm(v.y, v.x, sel) & live) | (0x7F7F7F7Fu & ~live);
            };
#pragma unroll
            for (int j = 0; j < FM; ++j) scm[j] = tail_scale(p.scale_a, p.lds_a, m0 + wave_m * WTM + 32 * j + frag_row(lane), M);
#pragma unroll
            for (int i = 0; i < FN; ++i) scn[i] = tail_scale(p.scale_b, p.lds_b, n0 + wave_n * WTN + 32 * i + frag_row(lane), N);
            __syncthreads();
            // slabs wholly past K hold zeros and are skipped
            const int live_slabs = (K - nfull * BKE + BKE / 4 - 1) / (BKE / 4);
#pragma unroll
            for (int r = 0; r < NR; ++r) read(r, 0, 0, 1, fa0, fb0);
            slab_sc(Q0{}, fa0, fb0, [](int) {});
            if (live_slabs > 1) {
#pragma unroll
                for (int r = 0; r < NR; ++r) read(r, 1, 0, 1, fa0, fb0);
                slab_sc(Q1{}, fa0, fb0, [](int) {});
            }
            if (live_slabs > 2) {
#pragma unroll
                for (int r = 0; r < NR; ++r) read(r, 2, 0, 1, fa0, fb0);
                slab_sc(Q2{}, fa0, fb0, [](int) {});
            }
            if (live_slabs > 3) {
#pragma unroll
                for (int r = 0; r < NR; ++r) read(r, 3, 0, 1, fa0, fb0);
                slab_sc(Q3{}, fa0, fb0, [](int) {});
            }
        }
    } else if constexpr (LC < 16) {
        // Operand rows only 4- or 2-byte aligned: LDS-DMA needs 16-byte
        // aligned sources, so each lane gathers the same 16-byte chunks the
        // DMA copies would move (row dma128_row, logical chunk dma128_chunk
        // of copy j) into registers with buffer loads, and scatters them with
        // ds_write_b128 into the same swizzled slots.  A chunk that starts
        // mid-dword is loaded as the dword-aligned 16 bytes at or below it plus
        // the next dword and shifted into place (v_alignbyte).  Per stage the 16 chunk
        // groups of a lane (8 of A, 8 of B) are scattered in slabs 0-2, each
        // one stage after its gather, and the same registers then gather the
        // chunk group of the stage after next: one stage of loads in flight,
        // 64 KiB per workgroup in registers.  Stage s lives in slots
        // 2(s % 2) and 2(s % 2) + 1; the scatters of stage s+1 in slabs 0-2 of
        // stage s go to slots freed by barrier B_{s-1}, and B_s (after slab 2,
        // with every scatter complete) publishes them.
        // Rows past M or N get an offset beyond the buffer range and load
        // zeros; the extra dword is only loaded for rows that need the shift,
        // so every dword read holds at least one byte of a valid row.  The
        // buffer base is the tile's first row rounded down to 4 bytes and
        // every offset is a multiple of 4: dword loads at offsets that are
        // not measured wrong on gfx950 when the base itself was not aligned.
        u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
        constexpr int NG = 2 * NC;  // chunk groups per lane and stage: 8 of A, then 8 of B
        constexpr unsigned kOut = 0x80000000u;  // beyond every buffer range (256 rows x stride <= 2^31)
        const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
        const char* first[2] = {p.A + static_cast<int64_t>(m0) * p.lda_b, p.B + static_cast<int64_t>(n0) * p.ldb_b};
        const unsigned lead[2] = {static_cast<unsigned>(reinterpret_cast<uintptr_t>(first[0]) & 3u),
                                  static_cast<unsigned>(reinterpret_cast<uintptr_t>(first[1]) & 3u)};
        const __amdgpu_buffer_rsrc_t br[2] = {
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(first[0] - lead[0]), static_cast<short>(0),
                                              static_cast<int>(lead[0] + rows_a * p.lda_b), 0x00020000),
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(first[1] - lead[1]), static_cast<short>(0),
                                              static_cast<int>(lead[1] + rows_b * p.ldb_b), 0x00020000)};
        unsigned off_lo[NG], off_hi[NG], shift[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int o = g / NC, j = wave * NC + g % NC;
            const int r = dma128_row(j, lane);
            const unsigned ldb = static_cast<unsigned>(o == 0 ? p.lda_b : p.ldb_b);
            const unsigned at = lead[o] + static_cast<unsigned>(r) * ldb + dma128_chunk(j, lane) * kChunkBytes;
            const unsigned sub = at & 3u;  // 0 for LC 4; 0 or 2 for LC 2; any for LC 1
            const bool valid = r < (o == 0 ? rows_a : rows_b);
            off_lo[g] = valid ? at - sub : kOut;
            off_hi[g] = (valid && sub) ? at - sub + kChunkBytes : kOut;
            shift[g] = sub;
        }
        u32x4 glo[NG];
        unsigned ghi[NG];
        // gather chunk group g of stage t into registers
        auto gather = [&](int g, int t) {
            const int o = g / NC;
            const int soff = __builtin_amdgcn_readfirstlane(t * kRowBytes);
            glo[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(br[o], static_cast<int>(off_lo[g]),
                                                                                     soff, 0));
            if constexpr (LC < 4)
                ghi[g] = __builtin_amdgcn_raw_buffer_load_b32(br[o], static_cast<int>(off_hi[g]), soff, 0);
        };
        // scatter chunk group g into slot `slot`
        auto scatter = [&](int g, int slot) {
            u32x4 v = glo[g];
            if constexpr (LC < 4) {
                const unsigned sh = shift[g];
                v.x = __builtin_amdgcn_alignbyte(glo[g].y, glo[g].x, sh);
                v.y = __builtin_amdgcn_alignbyte(glo[g].z, glo[g].y, sh);
                v.z = __builtin_amdgcn_alignbyte(glo[g].w, glo[g].z, sh);
                v.w = __builtin_amdgcn_alignbyte(ghi[g], glo[g].w, sh);
            }
            *reinterpret_cast<u32x4*>(smem + slot * SLOT + (wave * NC + g % NC) * 1024 + lane * kChunkBytes) = v;
        };
        // chunk group p of a stage goes out after MFMA 3p + 1 of slabs 0-2
        auto pairs_at = [&](int k, int m, auto&& f) {
#pragma unroll
            for (int q = 0; q < NG; ++q)
                if (3 * q + 1 == 16 * k + m) f(q);
        };

        if (nfull > 0) {
            // prologue: stage 0 through registers into slots 0/1, then stage 1 in flight
#pragma unroll
            for (int g = 0; g < NG; ++g) gather(g, 0);
#pragma unroll
            for (int g = 0; g < NG; ++g) scatter(g, g / NC);
#pragma unroll
            for (int g = 0; g < NG; ++g) gather(g, min(1, nfull - 1));
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
            barrier();
    #pragma unroll
            for (int r = 0; r < NR; ++r) read(r, 0, 0, 1, fa0, fb0);

            int slot0 = 0;  // slot of stage s's A half: 2 * (s % 2)
            for (int s = 0; s < nfull; ++s) {
                const int sa = slot0, sb = slot0 + 1;
                const int na = slot0 ^ 2, nb = na + 1;
                // a stage index past the last full stage reloads it (values unused)
                const int t2 = min(s + 2, nfull - 1);
                auto step = [&](int q) {
                    scatter(q, q < NC ? na : nb);  // stage s+1, gathered one stage ago
                    gather(q, t2);
                };
                slab_with_side<DT, FM, FN, MF>(acc, fa0, fb0, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 1, sa, sb, fa1, fb1); });
                    pairs_at(0, m, step);
                });
                slab_with_side<DT, FM, FN, MF>(acc, fa1, fb1, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 2, sa, sb, fa0, fb0); });
                    pairs_at(1, m, step);
                });
                slab_with_side<DT, FM, FN, MF>(acc, fa0, fb0, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 3, sa, sb, fa1, fb1); });
                    pairs_at(2, m, step);
                });
                asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
                barrier();
                // on the last stage the reads below fetch values that go unused
                slab_with_side<DT, FM, FN, MF>(acc, fa1, fb1, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 0, na, nb, fa0, fb0); });
                });
                slot0 = na;
            }
            wait_vm<0>();  // no load outlives the loop
        }

        if (K % BKE != 0) {
            // ragged last stage through registers into slots 0 (A) and 1 (B);
            // k >= K become exact zeros
            __syncthreads();
            const int c = stage_chunk(tid);
            const int k0 = nfull * BKE + c * EPC;
    #pragma unroll
            for (int i = 0; i < BM / 32; ++i) {
                const int r = stage_row(tid, i);
                const char* arow = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
                const char* brow = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
                *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) = tail_chunk(arow, k0, K);
                *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) = tail_chunk(brow, k0, K);
            }
            __syncthreads();
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (nfull * BKE + q * (BKE / 4) >= K) break;  // the rest of the stage is zeros
    #pragma unroll
                for (int r = 0; r < NR; ++r) read(r, q, 0, 1, fa0, fb0);
    #pragma unroll
                for (int i = 0; i < FN; ++i)
    #pragma unroll
                    for (int j = 0; j < FM; ++j) acc[i][j] = mfma_slab<DT>(fb0[i], fa0[j], acc[i][j]);
            }
        }
    } else {
        u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];

        if (nfull > 0) {
            // prologue: half-stages 0 .. NS-2 (a stage index past the last full
            // stage reloads that stage, so the copy counts stay uniform)
            constexpr int PRO = (SCHED == 0) ? (NS - 1) * NC : 3 * NC + NC / 2;  // prologue copies
    #pragma unroll
            for (int c = 0; c < PRO; ++c) {
                const int h = c / NC;
                copy(h & 1, c % NC, min(h >> 1, nfull - 1), h);
            }
            wait_vm<PRO - 2 * NC>();
            barrier();
    #pragma unroll
            for (int r = 0; r < NR; ++r) read(r, 0, 0, 1, fa0, fb0);

            constexpr int H0 = NS - 1;                 // half-stage copied in slab 0, minus 2s
            int slot0 = 0;                             // slot of stage s's A half, (2s) % NS
            for (int s = 0; s < nfull; ++s) {
                const int sa = slot0, sb = wrap(slot0 + 1);
                const int na = wrap(slot0 + 2), nb = wrap(slot0 + 3);
                const int t0 = min(s + (H0 >> 1), nfull - 1);       // stage of half-stage 2s + H0
                const int t3 = min(s + ((H0 + 1) >> 1), nfull - 1); // stage of half-stage 2s + H0 + 1
                const int slot_h0 = wrap(slot0 + NS - 1);
                // SCHED 1 (5 slots): one copy every 4 MFMAs through the whole stage --
                // the second half of B(s+1) in slab 0, A(s+2) in slabs 1-2 and the
                // first half of B(s+2) in slab 3 -- instead of bursts in slabs 0 and 3
                const int t1 = min(s + 1, nfull - 1), t2 = min(s + 2, nfull - 1);
                slab_with_side<DT, FM, FN, MF>(acc, fa0, fb0, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 1, sa, sb, fa1, fb1); });
                    if constexpr (SCHED == 0) {
                        if (m & 1) copy(H0 & 1, m >> 1, t0, slot_h0);
                    } else {
                        if ((m & 3) == 1) copy(1, NC / 2 + (m >> 2), t1, nb);
                    }
                });
                slab_with_side<DT, FM, FN, MF>(acc, fa1, fb1, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 2, sa, sb, fa0, fb0); });
                    if constexpr (SCHED == 1) {
                        if ((m & 3) == 1) copy(0, m >> 2, t2, slot_h0);
                    }
                });
                slab_with_side<DT, FM, FN, MF>(acc, fa0, fb0, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 3, sa, sb, fa1, fb1); });
                    if constexpr (SCHED == 1) {
                        if ((m & 3) == 1) copy(0, NC / 2 + (m >> 2), t2, slot_h0);
                    }
                });
                asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
                wait_vm<(NS - 4) * NC>();
                barrier();
                // on the last stage the reads below fetch values that go unused
                slab_with_side<DT, FM, FN, MF>(acc, fa1, fb1, [&](int m) {
                    reads_at(m, [&](int k) { read(k, 0, na, nb, fa0, fb0); });
                    if constexpr (SCHED == 0) {
                        if (m & 1) copy((H0 + 1) & 1, m >> 1, t3, sa);
                    } else {
                        if ((m & 3) == 1) copy(1, m >> 2, t2, sa);
                    }
                });
                slot0 = na;
            }
            wait_vm<0>();  // no copy outlives the loop
        }

        if (K % BKE != 0) {
            // ragged last stage through registers into slots 0 (A) and 1 (B);
            // k >= K become exact zeros
            __syncthreads();
            const int c = stage_chunk(tid);
            const int k0 = nfull * BKE + c * EPC;
    #pragma unroll
            for (int i = 0; i < BM / 32; ++i) {
                const int r = stage_row(tid, i);
                const char* arow = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
                const char* brow = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
                *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) = tail_chunk(arow, k0, K);
                *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) = tail_chunk(brow, k0, K);
            }
            __syncthreads();
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (nfull * BKE + q * (BKE / 4) >= K) break;  // the rest of the stage is zeros
    #pragma unroll
                for (int r = 0; r < NR; ++r) read(r, q, 0, 1, fa0, fb0);
    #pragma unroll
                for (int i = 0; i < FN; ++i)
    #pragma unroll
                    for (int j = 0; j < FM; ++j) acc[i][j] = mfma_slab<DT>(fb0[i], fa0[j], acc[i][j]);
            }
        }
    }

    if constexpr ((EPI & 8) != 0) {
        if (p.epi == TG_EPI_SOFTMAX) {  // the plan makes one tile span all of N
            softmax_epilogue<BM, WTM, WTN, FM, FN>(acc, p, m0, wave_m, wave_n, lane, smem);
            return;
        }
    }

    // epilogue: alpha, then ReLU, in registers
    const float alpha = p.alpha;
    const bool relu = p.relu != 0;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float v = acc[i][j][r] * alpha;
                acc[i][j][r] = relu ? fmaxf(v, 0.0f) : v;
            }
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    const bool aligned16 = (reinterpret_cast<uintptr_t>(p.D) & 15) == 0;
    const bool trans32 = (EPI & 2) && p.out_dtype == TG_F32 && interior;
    const bool trans16 = (EPI & 4) && p.out_dtype != TG_F32 && interior && aligned16 && (p.ldd & 7) == 0;
    const bool quad = (EPI & 16) && p.out_dtype != TG_F32 && interior && (p.ldd & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.D) & 7u) == 0;
    if (quad) {
        // Interior tile, 16-bit D: transpose each 4 x 4 group (4 lanes of a
        // quad = 4 consecutive m, 4 registers = 4 consecutive n) in registers
        // with two DPP butterfly steps, so each lane holds 4 consecutive m of
        // one n and stores them as one 8-byte vector: a quarter of the store
        // instructions, each writing whole 64-byte row pieces.
        const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
        auto dpp = [](float v, int ctrl_is_pair) {
            const int x = __builtin_bit_cast(int, v);
            return __builtin_bit_cast(float, ctrl_is_pair ? __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true)
                                                          : __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
        };
        const int64_t ldd = p.ldd;
        const int64_t lane_off = static_cast<int64_t>(n0 + wave_n * WTN + 4 * (lane >> 5) + (lane & 3)) * ldd +
                                 (m0 + wave_m * WTM + 4 * ((lane & 31) >> 2));
        with_out_type(p.out_dtype, [&](auto out) {
            constexpr int OUT = decltype(out)::value;
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float x[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
#pragma unroll
                        for (int q = 0; q < 4; q += 2) {  // swap within lane pairs
                            const float r = dpp(b0 ? x[q] : x[q + 1], 1);
                            x[q] = b0 ? r : x[q];
                            x[q + 1] = b0 ? x[q + 1] : r;
                        }
#pragma unroll
                        for (int q = 0; q < 2; ++q) {  // swap between lane pairs
                            const float r = dpp(b1 ? x[q] : x[q + 2], 0);
                            x[q] = b1 ? r : x[q];
                            x[q + 2] = b1 ? x[q + 2] : r;
                        }
                        const int64_t idx = lane_off + (32 * i + 8 * g) * ldd + 32 * j;
                        if constexpr (OUT != TG_F32) {
                            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                            u32x2 v;
                            if constexpr (OUT == TG_BF16) {
                                v.x = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2));
                                v.y = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2));
                            } else {
                                v.x = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[0], x[1]}, f16x2));
                                v.y = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[2], x[3]}, f16x2));
                            }
                            u32x2* d = reinterpret_cast<u32x2*>(static_cast<unsigned short*>(p.D) + idx);
                            if constexpr (EPI & 1) __builtin_nontemporal_store(v, d); else *d = v;
                        }
                    }
        });
    } else if (!trans32 && !trans16) {
        // store by ownership: each instruction writes 2 x 32 consecutive m.
        // Interior tiles store without per-element checks; the row offsets
        // of a block's 16 registers are wave-uniform multiples of ldd.
        with_out_type(p.out_dtype, [&](auto out) {
            constexpr int OUT = decltype(out)::value;
            const int64_t ldd = p.ldd;
            const int64_t lane_off = static_cast<int64_t>(n0 + wave_n * WTN + acc_row(lane, 0)) * ldd +
                                     (m0 + wave_m * WTM + acc_col(lane));
            if (interior) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            store_out<OUT, (EPI & 1) != 0>(
                                p.D, lane_off + (32 * i + 8 * (r >> 2) + (r & 3)) * ldd + 32 * j, acc[i][j][r]);
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        const int m = m0 + wave_m * WTM + 32 * j + acc_col(lane);
                        const int nbase = n0 + wave_n * WTN + 32 * i;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int n = nbase + acc_row(lane, r);
                            if (m < M && n < N)
                                store_out<OUT, (EPI & 1) != 0>(p.D, static_cast<int64_t>(n) * ldd + m, acc[i][j][r]);
                        }
                    }
                }
            }
        });
    } else if (trans16) {
        // 16-bit D, interior tile, 16-byte aligned rows: the whole rounded
        // tile (256 x 256 x 2 bytes) goes through LDS in one pass and each
        // store instruction writes two whole 512-byte row runs, instead of
        // 64-byte pieces of lines that other instructions complete later.
        constexpr int PITCH16 = 528;
        static_assert((EPI & 4) == 0 || 256 * PITCH16 <= LDS_BYTES, "16-bit tile fits the LDS");
        __syncthreads();  // every wave is done with the ring
        with_out_type(p.out_dtype, [&](auto out) {
            constexpr int OUT = decltype(out)::value;
            if constexpr (OUT != TG_F32) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int nl = wave_n * WTN + 32 * i + acc_row(lane, r);
                            const int ml = wave_m * WTM + 32 * j + acc_col(lane);
                            const float v = acc[i][j][r];
                            unsigned short h;
                            if constexpr (OUT == TG_BF16)
                                h = bf16_rne(v);
                            else
                                h = __builtin_bit_cast(unsigned short, static_cast<_Float16>(v));
                            *reinterpret_cast<unsigned short*>(smem + nl * PITCH16 + ml * 2) = h;
                        }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < 32; ++q) {
                    const int nl = 64 * wave + 2 * q + (lane >> 5);
                    const int c = lane & 31;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + nl * PITCH16 + c * 16);
                    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<unsigned short*>(p.D) +
                                                          static_cast<int64_t>(n0 + nl) * p.ldd + m0) + c;
                    if constexpr (EPI & 1)
                        __builtin_nontemporal_store(v, dst);
                    else
                        *dst = v;
                }
            }
        });
    } else {
        // interior tile: transpose through LDS so that each store instruction
        // writes one whole 1 KiB row run of the tile (256 consecutive m).
        // With line-aligned D columns this is no faster than the direct
        // stores; with columns only 4-byte aligned (odd ldd) it touches 9
        // lines per run instead of two lines per 128-byte piece and measured
        // 2.5 % faster on the whole product.  The 16-byte stores only assume
        // 4-byte alignment.  Two passes of 128 rows (n); the row pitch of
        // 1056 bytes keeps the two half-waves of each LDS write on disjoint
        // banks.
        constexpr int PITCH = 1056;
        static_assert(EPI < 2 || 128 * PITCH <= LDS_BYTES, "transpose buffer fits the LDS");
        __syncthreads();  // every wave is done with the ring
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wave_n == pass) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int nl = 32 * i + acc_row(lane, r);
                            const int ml = wave_m * WTM + 32 * j + acc_col(lane);
                            *reinterpret_cast<float*>(smem + nl * PITCH + ml * 4) = acc[i][j][r];
                        }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                const int nl = 32 * wave + q;
                typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
                const f32x4_a4 v = *reinterpret_cast<const f32x4*>(smem + nl * PITCH + lane * 16);
                f32x4_a4* dst = reinterpret_cast<f32x4_a4*>(static_cast<float*>(p.D) +
                                                            static_cast<int64_t>(n0 + 128 * pass + nl) * p.ldd +
                                                            m0) + lane;
                if constexpr (EPI & 1)
                    __builtin_nontemporal_store(v, dst);
                else
                    *dst = v;
            }
            __syncthreads();
        }
    }
}

template <int DT, int GM, int NS, int RS, int ADDR, int SCHED, int EPI, int LC>
static hipError_t launch_wide(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_wide_kernel<DT, GM, NS, RS, ADDR, SCHED, EPI, LC>),
                       dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg

// Instance rows of the wide kernel: (id, dtype, group_m, slots NS, read spread
// RS, ADDR, SCHED, EPI, row alignment class LC, eff%).  eff% weighs the
// instance's tiles in the host plan chooser.  ADDR 1 instances address a tile
// through 32-bit byte offsets, so they take operand row strides up to 8 MiB
// (256 rows x stride < 2^31); the ADDR 0 twins cover longer rows.
#define TG_INSTANTIATE_WIDE(id, DT, GM, NS, RS, ADDR, SCHED, EPI, LC, EFF) \
    template __global__ void tg::gemm_wide_kernel<DT, GM, NS, RS, ADDR, SCHED, EPI, LC>(GemmArgs);

#define TG_ENTRY_WIDE(id, DT, GM, NS, RS, ADDR, SCHED, EPI, LC, EFF)                                         \
    {id, DT, 256, 256, TG_WIDE_STAGE_K(DT), 2, 2, 128, 128, 256, NS, 5 * 256 * 128, 256, LC, GM, EFF,         \
     &tg::launch_wide<DT, GM, NS, RS, ADDR, SCHED, EPI, LC>, (ADDR) ? (int64_t(1) << 23) : 0,                  \
     ((EPI) & 8) ? 1 : 0, (EPI) & 1, ((EPI) & 64) ? 1 : 0},
