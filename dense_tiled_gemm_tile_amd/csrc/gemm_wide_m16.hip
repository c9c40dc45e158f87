// Wide streaming GEMM kernel for bf16 and fp16 operands on 16x16x32 MFMAs.
//
// The tile, the copies and the stage schedule are those of the wide kernel
// (256 x 256 tile, 4 waves of 128 x 128, 128-byte K stages moved by LDS-DMA
// through a ring of five 32 KiB half-stage slots; Tylo.jl manual, "Walk
// through GEMM", sections 3 and 4), but each wave's 128 x 128 is 8 x 8
// blocks of 16 x 16 and every MFMA takes 32 k.  Under the power limit this
// is what pays: the same MFMA stream with random operands and no memory
// traffic ran 2237 TFLOP/s on 16x16x32 against 1953 on 32x32x16 (2.21
// against 1.96 GHz at the same MFMA busy), since a 16x16x32 MFMA moves half
// the accumulator data per multiply-add.
//
// Per stage: two slabs of 32 k, 64 MFMAs each, in rows of 8 (one n-block,
// the eight m-blocks).  During slab 0 the wave reads all of slab 1's
// fragments, so that stage s is in registers when the barrier comes: the
// barrier (after every wave has waited for its copies of stage s+1 and for
// its fragment reads) publishes stage s+1 and frees both slots of stage s,
// and during slab 1 the wave copies B of stage s+2 and A of stage s+3 into
// them.  So each copy of B is issued a stage, each copy of A two stages,
// before the barrier that publishes it.
// The m-side fragments are double buffered; each n-side fragment is read
// into the register of the row that has just used it, except those of rows
// 6 and 7, which alternate with two spare registers so that every read of a
// slab is issued 16 MFMAs before its end (no read is waited for at the
// barrier).
#include "gemm_common.h"

namespace tg {

// c += the 16x16x32 product of the n-side fragment nb and the m-side
// fragment ma, accumulating in place in four AGPRs.  Written as tied inline
// assembly: with 64 accumulators per lane the builtin's untied form makes the
// register allocator copy accumulators between MFMAs (over 300 moves per
// stage).  Volatile, so the MFMAs keep their order against the other
// volatile statements below.
template <int DT>
__device__ __forceinline__ void mfma16(f32x4& c, const u32x4& nb, const u32x4& ma) {
    if constexpr (DT == TG_BF16)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(nb), "v"(ma));
    else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(nb), "v"(ma));
}
// Per-lane copy offset of a row past the operand's end: beyond every buffer
// range the plan allows (256 rows of at most 8 MiB), also less the largest
// immediate offset, and far enough below 2^32 that no offset sum wraps.
constexpr unsigned kFarOffset = 0xF0000000u;

// The compiler does not see the assembly above as MFMAs, so it cannot count
// the wait states between them and other instructions that write or read the
// accumulators (the zeroing before the K loop, the epilogue after it; at most
// passes + 2 = 18 for these): the kernel waits them out with these nops, and
// pins the accumulators on the right side of them with an empty statement
// that claims to rewrite each one.
__device__ __forceinline__ void mfma16_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
template <int FN, int FM>
__device__ __forceinline__ void acc_fence(f32x4 (&acc)[FN][FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// EPI: bit 0 = nontemporal D stores, bit 1 = fp32 D of interior tiles through
// an LDS transpose (whole 1 KiB row runs per store instruction).
template <int DT, int GM, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_wide_m16_kernel(GemmArgs p) {
    select_batch(p);
    static_assert(DT == TG_BF16 || DT == TG_F16, "16-bit operands");
    constexpr int BM = 256, BN = 256, WM = 2, NS = 5;
    constexpr int ES = 2;
    constexpr int EPC = 16 / ES;                 // K elements per 16-byte chunk
    constexpr int BKE = kRowBytes / ES;          // K elements per stage (64)
    constexpr int WTM = 128, WTN = 128;          // output owned by one wave
    constexpr int FM = WTM / 16, FN = WTN / 16;  // 16 x 16 MFMA blocks per wave
    constexpr int NC = BM / (8 * 4);             // 1 KiB copies per wave per half-stage
    constexpr int SLOT = BM * kRowBytes;         // 32 KiB
    constexpr int LDS_BYTES = 5 * SLOT;
    static_assert(NS == 5, "the K loop is unrolled over the five slots");
    static_assert(FM == 8 && FN == 8 && NC == 8, "schedule assumes 8 x 8 blocks and 8 copies per half-stage");
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

    // copy sources: buffer resources over the tile's valid rows, 32-bit row
    // offsets (the plan keeps 256 * stride below 2^31); rows past M or N fall
    // outside the range and load zeros (they only feed accumulators that are
    // never stored)
    const i32x4 rsrc[2] = {
        buffer_rsrc(p.A + static_cast<int64_t>(m0) * p.lda_b, static_cast<unsigned>(min(BM, M - m0) * p.lda_b)),
        buffer_rsrc(p.B + static_cast<int64_t>(n0) * p.ldb_b, static_cast<unsigned>(min(BN, N - n0) * p.ldb_b))};
    // Copies 4g .. 4g + 3 of a wave share one LDS base in M0 and take the
    // immediate offsets 0, 1024, 2048 and 3072, which move the global address
    // by the same amount, so their per-lane offsets are lowered by it (copy j
    // starts 8 j rows into the operand, and rows hold at least the 128 bytes
    // of a full stage whenever copies run, so the offsets stay non-negative).
    // Rows past the operand's end get an offset far beyond any range: with or
    // without the immediate they load zeros.
    unsigned voff[2][NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int j = wave * NC + i;
        const int r = dma128_row(j, lane);
        const unsigned low = 1024u * (i & 3), chunk = dma128_chunk(j, lane) * kChunkBytes;
        voff[0][i] = r < min(BM, M - m0) ? static_cast<unsigned>(r * p.lda_b) + chunk - low : kFarOffset;
        voff[1][i] = r < min(BN, N - n0) ? static_cast<unsigned>(r * p.ldb_b) + chunk - low : kFarOffset;
    }
    // LDS base of copies 4g .. 4g + 3 of this wave into slot `slot`
    auto copy_base = [&](int g, int slot) {
        return __builtin_amdgcn_readfirstlane(lds_base + slot * SLOT + (wave * NC + 4 * g) * 1024);
    };
    // M0 for the group of copies 4g .. 4g + 3 into `slot`, then the wait
    // state an LDS-DMA load needs after an M0 write.  The copies read M0
    // without naming it, so that the compiler neither reloads it in front of
    // each one nor drops the wait; the kernel has no other M0 user (its
    // assembly is checked on the host: every M0 write is this one, and every
    // copy follows one).  Both are volatile, so they stay in program order.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved: nothing is kept in it across this
    auto set_m0 = [&](int g, int slot) {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(copy_base(g, slot)) : "m0");
    };
#pragma clang diagnostic pop
    // copy i of operand o (0: A, 1: B) of stage t (byte offset so = t * 128)
    // into the slot whose group base set_m0 put in M0
    auto copy = [&](int o, int i, unsigned so) {
        switch (i & 3) {
            case 0:
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff[o][i]), "s"(rsrc[o]), "s"(so) : "memory");
                break;
            case 1:
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:1024 lds"
                             : : "v"(voff[o][i]), "s"(rsrc[o]), "s"(so) : "memory");
                break;
            case 2:
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:2048 lds"
                             : : "v"(voff[o][i]), "s"(rsrc[o]), "s"(so) : "memory");
                break;
            default:
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:3072 lds"
                             : : "v"(voff[o][i]), "s"(rsrc[o]), "s"(so) : "memory");
                break;
        }
    };

    // fragment read offsets within a slot: lane l reads row l % 16 of a
    // 16-row block and, for its k-group g = l / 16, chunk 4q + (0, 2, 1, 3)[g]
    // of slab q (the MFMA takes its four k-groups in any order, the same on
    // both sides).  The LDS serves a 16-byte read to lanes 4i..4i+3 and
    // 4i+32..4i+35 together; with this order those lanes read two chunks that
    // differ in bit 0, which the row swizzle keeps on distinct banks, where
    // the plain order (chunks differing in bit 1, as the swizzle of rows r and
    // r + 2 does) measured 4 conflict cycles a read.  Block steps are 16 rows,
    // which keep the swizzle.
    const int g = frag16_chunk(lane);
    const int gchunk = ((g & 1) << 1) | (g >> 1);
    int mread[2], nread[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        mread[q] = wave_m * WTM * kRowBytes + lds_chunk_offset(frag16_row(lane), 4 * q + gchunk);
        nread[q] = wave_n * WTN * kRowBytes + lds_chunk_offset(frag16_row(lane), 4 * q + gchunk);
    }
    // A read's immediate offset reaches 64 KiB, two slots: each read position
    // keeps one base per slot pair (slots 0-1, 2-3, 4), set up here once, so
    // that with the slot known at compile time no read needs an address add.
    int mbase[2][3], nbase[2][3];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            mbase[q][k] = mread[q] + 2 * k * SLOT;
            nbase[q][k] = nread[q] + 2 * k * SLOT;
            asm volatile("" : "+v"(mbase[q][k]), "+v"(nbase[q][k]));  // kept as registers
        }
    auto rd_m = [&](int j, int q, int slot) {
        return *reinterpret_cast<const u32x4*>(smem + mbase[q][slot >> 1] + (slot & 1) * SLOT + j * 16 * kRowBytes);
    };
    auto rd_n = [&](int i, int q, int slot) {
        return *reinterpret_cast<const u32x4*>(smem + nbase[q][slot >> 1] + (slot & 1) * SLOT + i * 16 * kRowBytes);
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    acc_fence(acc);  // the zeros are written here, and waited out before the first MFMA
    mfma16_drain();

    // fragments: m-side double buffered (set 0 for slab 0, set 1 for slab 1);
    // n-side rows 0-5 in fb[0..5], rows 6-7 in fb[6..7] on slab 0 and in
    // fs[0..1] on slab 1
    u32x4 fa[2][FM], fb[FN], fs[2];
    // the MFMAs of one slab, row by row; side(m) after MFMA m
    auto slab = [&](auto set, auto&& side) {
        constexpr int X = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const u32x4& bn = (X == 1 && i >= 6) ? fs[i - 6] : fb[i];
                mfma16<DT>(acc[i][j], bn, fa[X][j]);
                side(FM * i + j);
                __builtin_amdgcn_sched_barrier(0);
            }
    };

    const int nfull = K / BKE;
    if (nfull > 0) {
        // prologue: half-stages 0 .. 4 (A0, B0, A1, B1, A2) into slots 0 .. 4,
        // stage 0 waited for, slab 0 read
        constexpr int PRO = 5 * NC;
#pragma unroll
        for (int c = 0; c < PRO; ++c) {
            const int h = c / NC;
            if (c % 4 == 0) set_m0((c % NC) >> 2, h);
            copy(h & 1, c % NC, __builtin_amdgcn_readfirstlane(min(h >> 1, nfull - 1) * kRowBytes));
        }
        wait_vm<PRO - 2 * NC>();
        barrier();
#pragma unroll
        for (int j = 0; j < FM; ++j) fa[0][j] = rd_m(j, 0, 0);
#pragma unroll
        for (int i = 0; i < FN; ++i) fb[i] = rd_n(i, 0, 1);

        // The ring turns by two slots a stage and repeats after five, so the
        // loop body is five stages with their slots known at compile time:
        // stage 5k + U keeps A in slot 2U mod 5 and B in the next one.
        const int last_so = (nfull - 1) * kRowBytes;
        auto stage = [&](auto u, int s) {
            constexpr int U = decltype(u)::value;
            constexpr int SA = (2 * U) % NS, SB = (2 * U + 1) % NS, NA = (2 * U + 2) % NS, NB = (2 * U + 3) % NS;
            // byte offsets of stages s+2 (B) and s+3 (A) along K; past the last
            // full stage they reload it (values unused)
            unsigned so2 = 0, so3 = 0;
            // slab 0: read slab 1 (m-side set 1 first, rows 6/7 into the spares,
            // rows 0-5 after their last MFMA); the scalar work of slab 1's
            // copies goes into its quiet second half
            slab(std::integral_constant<int, 0>(), [&](int m) {
                if (m < FM) fa[1][m] = rd_m(m, 1, SA);
                if (m == 8 || m == 9) fs[m - 8] = rd_n(m - 2, 1, SB);
                if ((m & 7) == 7 && m < 48) fb[m >> 3] = rd_n(m >> 3, 1, SB);
                if (m == 50) {
                    so2 = __builtin_amdgcn_readfirstlane(min((s + 2) * kRowBytes, last_so));
                    asm volatile("" : "+s"(so2));  // computed here
                }
                if (m == 52) {
                    so3 = __builtin_amdgcn_readfirstlane(min((s + 3) * kRowBytes, last_so));
                    asm volatile("" : "+s"(so3));
                }
                if (m == 56) set_m0(0, SA);
            });
            // this wave's fragment reads are done and its copies of stage s+1
            // have landed (A(s+2) may be in flight): vmcnt(8) lgkmcnt(0), in
            // the builtin that the compiler's wait-count pass sees
            static_assert(NC == 8, "vmcnt field below");
            __builtin_amdgcn_s_waitcnt(0x0078);
            barrier();  // ... and everyone's; both slots of stage s are free
            // slab 1: read slab 0 of stage s+1 (on the last stage the values go
            // unused); copies: B(s+2) into slot SA, then A(s+3) into slot SB,
            // one every four MFMAs, M0 set one MFMA ahead of each group of four
            slab(std::integral_constant<int, 1>(), [&](int m) {
                if (m < FM) fa[0][m] = rd_m(m, 0, NA);
                if (m == 8 || m == 9) fb[m - 2] = rd_n(m - 2, 0, NB);
                if ((m & 7) == 7 && m < 48) fb[m >> 3] = rd_n(m >> 3, 0, NB);
                if ((m & 3) == 1) {
                    const int c = m >> 2;  // 0 .. 15
                    if (c < NC) copy(1, c, so2);
                    else copy(0, c - NC, so3);
                }
                if (m == 14) set_m0(1, SA);
                if (m == 30) set_m0(0, SB);
                if (m == 46) set_m0(1, SB);
            });
        };
        for (int s = 0;;) {
            stage(std::integral_constant<int, 0>(), s);
            if (++s == nfull) break;
            stage(std::integral_constant<int, 1>(), s);
            if (++s == nfull) break;
            stage(std::integral_constant<int, 2>(), s);
            if (++s == nfull) break;
            stage(std::integral_constant<int, 3>(), s);
            if (++s == nfull) break;
            stage(std::integral_constant<int, 4>(), s);
            if (++s == nfull) break;
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
            *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) = load_chunk_bounded<ES>(arow, k0, K);
            *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) = load_chunk_bounded<ES>(brow, k0, K);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (nfull * BKE + q * (BKE / 2) >= K) break;  // the rest of the stage is zeros
#pragma unroll
            for (int j = 0; j < FM; ++j) fa[0][j] = rd_m(j, q, 0);
#pragma unroll
            for (int i = 0; i < FN; ++i) fb[i] = rd_n(i, q, 1);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) mfma16<DT>(acc[i][j], fb[i], fa[0][j]);
        }
    }
    mfma16_drain();
    acc_fence(acc);  // the epilogue reads the accumulators only after the wait

    // epilogue: alpha, then ReLU, in registers; register r of block (i, j)
    // is (n, m) = (16 i + acc16_row(lane, r), 16 j + acc16_col(lane)) of the
    // wave's 128 x 128
    const float alpha = p.alpha;
    const bool relu = p.relu != 0;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = acc[i][j][r] * alpha;
                acc[i][j][r] = relu ? fmaxf(v, 0.0f) : v;
            }
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    const bool trans32 = (EPI & 2) && p.out_dtype == TG_F32 && interior;
    const bool quad = p.out_dtype != TG_F32 && interior && (p.ldd & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.D) & 7u) == 0;
    // Interior tiles pair the blocks j and j + 1 of each register with one
    // lane swap (v_permlane16_swap: lanes 16-31 of the first with lanes 0-15
    // of the second, and the same for 48-63 and 32-47), after which lanes
    // 0-31 hold 32 consecutive m of one n and lanes 32-63 of the n eight
    // rows below: whole 128-byte lines of fp32 D per half-wave.
    auto pair_swap = [](float x, float y, float& lo, float& hi) {
        const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                        __builtin_bit_cast(unsigned, y), false, false);
        lo = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));  // n = r (+8 for lanes 32-63)
        hi = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));  // n = 4 + r (+8)
    };
    if (quad) {
        // 16-bit D: after the swap, the four registers of a block pair are four
        // consecutive n and the four lanes of a quad four consecutive m, so two
        // DPP butterfly steps transpose each 4 x 4 group and every lane stores
        // four consecutive m of one n as one 8-byte vector (64-byte runs)
        const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
        auto dpp = [](float v, int ctrl_is_pair) {
            const int x = __builtin_bit_cast(int, v);
            return __builtin_bit_cast(float, ctrl_is_pair ? __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true)
                                                          : __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
        };
        auto transpose4 = [&](float (&x)[4]) {
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
        };
        const int64_t ldd = p.ldd;
        const int64_t lane_off = static_cast<int64_t>(n0 + wave_n * WTN + 8 * (lane >> 5) + (lane & 3)) * ldd +
                                 (m0 + wave_m * WTM + 4 * ((lane & 31) >> 2));
        with_out_type(p.out_dtype, [&](auto out) {
            constexpr int OUT = decltype(out)::value;
            if constexpr (OUT != TG_F32) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; j += 2) {
                        float lo[4], hi[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) pair_swap(acc[i][j][r], acc[i][j + 1][r], lo[r], hi[r]);
                        transpose4(lo);
                        transpose4(hi);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const float* x = h ? hi : lo;
                            u32x2 v;
                            if constexpr (OUT == TG_BF16) {
                                v.x = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2));
                                v.y = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2));
                            } else {
                                v.x = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[0], x[1]}, f16x2));
                                v.y = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[2], x[3]}, f16x2));
                            }
                            u32x2* d = reinterpret_cast<u32x2*>(static_cast<unsigned short*>(p.D) + lane_off +
                                                                (16 * i + 4 * h) * ldd + 16 * j);
                            if constexpr (EPI & 1) __builtin_nontemporal_store(v, d); else *d = v;
                        }
                    }
            }
        });
    } else if (!trans32) {
        // store by ownership (interior tiles: each instruction writes two runs
        // of 32 consecutive m, edge tiles: four runs of 16, with checks)
        with_out_type(p.out_dtype, [&](auto out) {
            constexpr int OUT = decltype(out)::value;
            const int64_t ldd = p.ldd;
            if (interior) {
                const int64_t pair_off = static_cast<int64_t>(n0 + wave_n * WTN + 8 * (lane >> 5)) * ldd +
                                         (m0 + wave_m * WTM + (lane & 31));
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; j += 2)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float lo, hi;
                            pair_swap(acc[i][j][r], acc[i][j + 1][r], lo, hi);
                            store_out<OUT, (EPI & 1) != 0>(p.D, pair_off + (16 * i + r) * ldd + 16 * j, lo);
                            store_out<OUT, (EPI & 1) != 0>(p.D, pair_off + (16 * i + 4 + r) * ldd + 16 * j, hi);
                        }
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
#pragma unroll
                    for (int j = 0; j < FM; ++j) {
                        const int m = m0 + wave_m * WTM + 16 * j + acc16_col(lane);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int n = n0 + wave_n * WTN + 16 * i + acc16_row(lane, r);
                            if (m < M && n < N)
                                store_out<OUT, (EPI & 1) != 0>(p.D, static_cast<int64_t>(n) * ldd + m, acc[i][j][r]);
                        }
                    }
                }
            }
        });
    } else {
        // interior tile, fp32 D: through LDS in two passes of 128 rows (n), so
        // that each store instruction writes one whole 1 KiB row run (256
        // consecutive m); only 4-byte alignment of D is assumed.  The row pitch
        // of 1056 bytes keeps the writes of a quarter-wave on distinct banks.
        constexpr int PITCH = 1056;
        static_assert(128 * PITCH <= LDS_BYTES, "transpose buffer fits the LDS");
        __syncthreads();  // every wave is done with the ring
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wave_n == pass) {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int nl = 16 * i + acc16_row(lane, r);
                            const int ml = wave_m * WTM + 16 * j + acc16_col(lane);
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

template <int DT, int GM, int EPI>
static hipError_t launch_wide_m16(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_wide_m16_kernel<DT, GM, EPI>), dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg

// Instances: (id, dtype, group_m, EPI, eff%): 67/68 nontemporal D stores,
// 69/70 plain stores and the fp32 LDS transpose (for D columns not on
// 128-byte lines), as the 32x32x16 instances 0-3 of the wide kernel; they
// weigh a little more than those, and the plan chooser considers them for K
// loops of at least 16 stages (see `choose`).
#define TG_WIDE_M16_LIST(X)                \
    X(67, TG_BF16, 4, 1, 109)              \
    X(68, TG_F16, 4, 1, 109)               \
    X(69, TG_BF16, 4, 2, 109)              \
    X(70, TG_F16, 4, 2, 109)

#define TG_INSTANTIATE_WIDE_M16(id, DT, GM, EPI, EFF) \
    template __global__ void tg::gemm_wide_m16_kernel<DT, GM, EPI>(GemmArgs);
TG_WIDE_M16_LIST(TG_INSTANTIATE_WIDE_M16)

#ifndef __HIP_DEVICE_COMPILE__
// 256 x 256 tile, 2 x 2 waves of 128 x 128, 64 k per stage, 5 slots of 32 KiB,
// 64 accumulators per lane; buffer addressing limits the row stride to 8 MiB
#define TG_ENTRY_WIDE_M16(id, DT, GM, EPI, EFF)                                                           \
    {id, DT, 256, 256, 64, 2, 2, 128, 128, 256, 5, 5 * 256 * 128, 256, 16, GM, EFF,                       \
     &tg::launch_wide_m16<DT, GM, EPI>, int64_t(1) << 23, 0, (EPI) & 1, 0, 0, 1},
extern const TgKernelDesc tg_entries_wide_m16[] = {TG_WIDE_M16_LIST(TG_ENTRY_WIDE_M16)};
extern const int tg_entries_wide_m16_count = sizeof(tg_entries_wide_m16) / sizeof(tg_entries_wide_m16[0]);
#endif  // __HIP_DEVICE_COMPILE__
