// Register-staged tiled GEMM kernel for gfx950 (CDNA4): the instances for
// operand rows that are only 4-, 2- or (8-, 6- and 4-bit operands) 1-byte
// aligned, for small problems and for the fused row-softmax epilogue.
//
// One workgroup owns one BM x BN output tile (cuTile.jl tutorial "Matrix
// Multiplication", Step 2: each output tile depends on no other, so each gets
// its own block) and walks K in stages of 128 bytes per operand row
// (Step 3: the K loop carries an fp32 accumulator).  Each stage is staged
// global -> registers -> LDS with 16-byte vectors along logical K for both
// operands (Tylo.jl manual, "Walk through GEMM", section 3 "Copy one K stage"),
// double-buffered, and consumed by MFMA instructions reading 16-byte fragments
// from LDS (section 4).  The epilogue scales by alpha, clamps at zero when
// ReLU is on, and stores every accumulator at the output coordinate its
// lane/register ownership gives (section 5).
//
// LDS layout of one stage: [A: BM rows x 128 B][B: BN rows x 128 B].  Row r
// keeps its eight 16-byte chunks in swizzled slots, chunk c at slot
// c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1).  Any 8 consecutive rows at one
// logical chunk then hit 8 distinct 16-byte slots modulo 128 bytes, and any 16
// consecutive rows hit 16 distinct slots modulo 256 bytes, for both the
// fragment reads (ds_read_b128) and the stage writes (ds_write_b128).
//
// Edges: rows beyond M (or N) are clamped to the last valid row; they only feed
// accumulators that are never stored.  Elements with k >= K are never read and
// are replaced by exact zeros (the final, partial K stage).  Stores are masked
// to m < M, n < N.
#include "gemm_common.h"

namespace tg {

// SM = 1: the instance also carries the softmax epilogue.
template <int DT, int BM, int BN, int LOADCLASS, int MINWAVES, int SM>
__global__ __launch_bounds__(kThreads, MINWAVES) void gemm_kernel(GemmArgs p) {
    select_batch(p);
    constexpr bool F8 = (DT == TG_E4M3 || DT == TG_E5M2);
    constexpr bool F4 = (DT == TG_E2M1);                   // packed two per byte
    constexpr bool F6 = (DT == TG_E2M3 || DT == TG_E3M2);  // packed four per three bytes
    constexpr bool SCL = F8 || F4 || F6;                   // block scales apply
    constexpr int ES = (DT == TG_F32) ? 4 : (F8 || F4 || F6) ? 1 : 2;  // element bytes (packed: per byte)
    constexpr int EPC = F4 ? 32 : 16 / ES;          // elements per 16-byte chunk (not for 6-bit)
    constexpr int BKE = F4 ? 256 : F6 ? 128 : kRowBytes / ES;  // K elements per stage
    constexpr int STB = F6 ? 96 : kRowBytes;        // bytes of a row per stage (6-bit: chunks 0-5)
    constexpr int SCW = F4 ? 2 : 1;                 // scale dwords per row and stage
    constexpr int WTM = BM / 2, WTN = BN / 2;       // 2 x 2 waves
    constexpr int FM = WTM / 32, FN = WTN / 32;     // 32 x 32 MFMA blocks per wave
    constexpr int RA = BM / 32, RB = BN / 32;       // staged rows per thread
    constexpr int STAGE = (BM + BN) * kRowBytes;

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave & 1, wave_n = wave >> 1;

    const TileCoord tile = grouped_tile(p.tile, p.tiles_m, p.tiles_n, p.group_m);
    const int m0 = tile.tm * BM, n0 = tile.tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    // ---- staging assignment: thread covers chunk column c of rows srow + 32*i
    const int c = stage_chunk(tid);
    const int srow = stage_row(tid, 0);
    // rows srow + 32*i share srow's swizzle, so one offset serves every i
    const int wslot = lds_chunk_offset(srow, c);
    const char* arow[RA];
    const char* brow[RB];
#pragma unroll
    for (int i = 0; i < RA; ++i)
        arow[i] = p.A + static_cast<int64_t>(min(m0 + srow + 32 * i, M - 1)) * p.lda_b;
#pragma unroll
    for (int i = 0; i < RB; ++i)
        brow[i] = p.B + static_cast<int64_t>(min(n0 + srow + 32 * i, N - 1)) * p.ldb_b;

    // ---- fragment read offsets (bytes within a stage)
    // (wave tile origins and block steps are multiples of 32 rows, which
    // leave the swizzle unchanged)
    int mread[4], nread[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        mread[q] = wave_m * WTM * kRowBytes + lds_chunk_offset(frag_row(lane), frag_chunk(lane, q));
        nread[q] = (BM + wave_n * WTN) * kRowBytes + lds_chunk_offset(frag_row(lane), frag_chunk(lane, q));
    }

    // 8-bit operands: pair p of a stage covers k [64p, 64p + 64); half-wave h
    // supplies chunks 4p + h (bytes 0-15) and 4p + 2 + h (bytes 16-31) of its
    // row, which the MFMA takes as k [16h, 16h + 16) and [32 + 16h, 48 + 16h)
    // of the 64: so k-block 2p (the first 32) sits in bytes 0-15 of both
    // halves and takes its scale from half 0, block 2p + 1 from half 1
    // (measured with one-hot operands and distinct scales per block)
    int mread8[2][2], nread8[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int ch = 4 * q + 2 * e + (lane >> 5);
            mread8[q][e] = wave_m * WTM * kRowBytes + lds_chunk_offset(frag_row(lane), ch);
            nread8[q][e] = (BM + wave_n * WTN) * kRowBytes + lds_chunk_offset(frag_row(lane), ch);
        }
    // 6-bit operands: pair p of a stage is the 48 bytes [48p, 48p + 48) of a
    // row; half-wave h takes bytes [48p + 24h, 48p + 24h + 24) as three 8-byte
    // reads, each inside one 16-byte chunk (mfma_f6)
    int mread6[2][3], nread6[2][3];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            const int b = 48 * q + 24 * (lane >> 5) + 8 * e;
            mread6[q][e] = wave_m * WTM * kRowBytes + lds_chunk_offset(frag_row(lane), b >> 4) + (b & 15);
            nread6[q][e] = (BM + wave_n * WTN) * kRowBytes + lds_chunk_offset(frag_row(lane), b >> 4) + (b & 15);
        }
    // block scales of the lane's rows: SCW dwords per row and stage (the
    // stage's 32-k blocks, four per dword), for the stage being consumed
    // (cur) and the one being loaded (nxt)
    unsigned scm_cur[FM][SCW], scn_cur[FN][SCW], scm_nxt[FM][SCW], scn_nxt[FN][SCW];
    const int nblk = (K + 31) / 32;
    auto load_scales = [&](int s) {
        if constexpr (SCL) {
            if (p.scale_a) {
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int m = min(m0 + wave_m * WTM + 32 * j + frag_row(lane), M - 1);
#pragma unroll
                    for (int w = 0; w < SCW; ++w)
                        scm_nxt[j][w] = *reinterpret_cast<const unsigned*>(
                            p.scale_a + m * p.lds_a + 4 * (SCW * static_cast<int64_t>(s) + w));
                }
            } else {
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int w = 0; w < SCW; ++w) scm_nxt[j][w] = 0x7F7F7F7Fu;
            }
            if (p.scale_b) {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    const int n = min(n0 + wave_n * WTN + 32 * i + frag_row(lane), N - 1);
#pragma unroll
                    for (int w = 0; w < SCW; ++w)
                        scn_nxt[i][w] = *reinterpret_cast<const unsigned*>(
                            p.scale_b + n * p.lds_b + 4 * (SCW * static_cast<int64_t>(s) + w));
                }
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int w = 0; w < SCW; ++w) scn_nxt[i][w] = 0x7F7F7F7Fu;
            }
        }
    };
    auto next_scales = [&]() {
        if constexpr (SCL) {
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int w = 0; w < SCW; ++w) scm_cur[j][w] = scm_nxt[j][w];
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int w = 0; w < SCW; ++w) scn_cur[i][w] = scn_nxt[i][w];
        }
    };
    // exponent of 32-k block b (0 .. 4*SCW-1) of stage s from a row's dwords;
    // blocks past the last one of K (their data is zero) count as 1
    // (a select, not an index, picks the dword: b varies by lane)
    auto scale_byte = [&](const unsigned (&w)[SCW], int b, int s) {
        const unsigned d = (SCW == 2 && b >= 4) ? w[SCW - 1] : w[0];
        return 4 * SCW * s + b < nblk ? static_cast<int>((d >> (8 * (b & 3))) & 0xFFu) : 127;
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Full stages 0 .. nfull-1, then (when K is not a multiple of BKE) one
    // ragged stage whose elements past K load as exact zeros.
    const int nfull = K / BKE;
    const int nk = nfull + ((K % BKE) != 0 ? 1 : 0);

    u32x4 sa[RA], sb[RB];
    // 6-bit stages cover chunks 0-5 of each LDS row; chunks 6 and 7 are never
    // read, and their threads load nothing
    const bool chunk_used = !F6 || c < STB / 16;
    auto load_full = [&](int s) {
        load_scales(s);
        const int64_t kb = static_cast<int64_t>(s) * STB + c * 16;
        if (!chunk_used) return;
#pragma unroll
        for (int i = 0; i < RA; ++i) sa[i] = load_chunk<LOADCLASS>(arow[i] + kb);
#pragma unroll
        for (int i = 0; i < RB; ++i) sb[i] = load_chunk<LOADCLASS>(brow[i] + kb);
    };
    auto load_ragged = [&](int s) {
        load_scales(s);
        if (!chunk_used) return;
        const int k0 = s * BKE + c * EPC;
        const int64_t b0 = static_cast<int64_t>(s) * STB + c * 16, kbits = 6 * static_cast<int64_t>(K);
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            if constexpr (F6)
                sa[i] = load_chunk_bounded_bits(arow[i], b0, kbits);
            else if constexpr (F4)
                sa[i] = load_chunk_bounded_e2m1(arow[i], k0, K);
            else
                sa[i] = load_chunk_bounded<ES>(arow[i], k0, K);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if constexpr (F6)
                sb[i] = load_chunk_bounded_bits(brow[i], b0, kbits);
            else if constexpr (F4)
                sb[i] = load_chunk_bounded_e2m1(brow[i], k0, K);
            else
                sb[i] = load_chunk_bounded<ES>(brow[i], k0, K);
        }
    };
    auto store_stage = [&](int buf) {
        char* base = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < RA; ++i)
            *reinterpret_cast<u32x4*>(base + 32 * i * kRowBytes + wslot) = sa[i];
#pragma unroll
        for (int i = 0; i < RB; ++i)
            *reinterpret_cast<u32x4*>(base + (BM + 32 * i) * kRowBytes + wslot) = sb[i];
    };
    // Fragments of slab q come from LDS while the MFMAs of slab q-1 run.
    auto read_frags = [&](const char* base, int q, u32x4* mf, u32x4* nf) {
#pragma unroll
        for (int j = 0; j < FM; ++j)
            mf[j] = *reinterpret_cast<const u32x4*>(base + mread[q] + j * 32 * kRowBytes);
#pragma unroll
        for (int i = 0; i < FN; ++i)
            nf[i] = *reinterpret_cast<const u32x4*>(base + nread[q] + i * 32 * kRowBytes);
    };
    // 8-bit operands, stage s in buffer buf: two MFMAs of 64 k per block;
    // scale blocks past the last one of K (their data is zero) count as 1
    auto compute8 = [&](int buf, int s) {
        const char* base = smem + buf * STAGE;
        u32x4 mf[2][FM][2], nf[2][FN][2];
        auto read_pair = [&](int q, u32x4 (&m8)[FM][2], u32x4 (&n8)[FN][2]) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    m8[j][e] = *reinterpret_cast<const u32x4*>(base + mread8[q][e] + j * 32 * kRowBytes);
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    n8[i][e] = *reinterpret_cast<const u32x4*>(base + nread8[q][e] + i * 32 * kRowBytes);
            }
        };
        read_pair(0, mf[0], nf[0]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (q == 0) read_pair(1, mf[1], nf[1]);
            const int sub = 2 * q + (lane >> 5);      // block within the stage
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int sn = scale_byte(scn_cur[i], sub, s), sm = scale_byte(scm_cur[j], sub, s);
                    acc[i][j] = mfma_f8<DT>(nf[q][i], mf[q][j], acc[i][j], sn, sm);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // 6-bit operands, stage s in buffer buf: two MFMAs of 64 k per block
    auto compute6 = [&](int buf, int s) {
        const char* base = smem + buf * STAGE;
        u32x2 mf[2][FM][3], nf[2][FN][3];
        auto read_pair = [&](int q, u32x2 (&m6)[FM][3], u32x2 (&n6)[FN][3]) {
#pragma unroll
            for (int e = 0; e < 3; ++e) {
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    m6[j][e] = *reinterpret_cast<const u32x2*>(base + mread6[q][e] + j * 32 * kRowBytes);
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    n6[i][e] = *reinterpret_cast<const u32x2*>(base + nread6[q][e] + i * 32 * kRowBytes);
            }
        };
        read_pair(0, mf[0], nf[0]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (q == 0) read_pair(1, mf[1], nf[1]);
            const int sub = 2 * q + (lane >> 5);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[i][j] = mfma_f6<DT == TG_E2M3 ? 2 : 3>(nf[q][i], mf[q][j], acc[i][j],
                                                                scale_byte(scn_cur[i], sub, s),
                                                                scale_byte(scm_cur[j], sub, s));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto compute = [&](int buf, int s) {
        if constexpr (F8) {
            compute8(buf, s);
            return;
        } else if constexpr (F6) {
            compute6(buf, s);
            return;
        }
        const char* base = smem + buf * STAGE;
        u32x4 mf[2][FM], nf[2][FN];
        read_frags(base, 0, mf[0], nf[0]);
        // The scheduling barriers pin the order "reads of slab q+1, then MFMAs
        // of slab q"; left alone, the scheduler sinks the reads next to their
        // first use and the MFMA pipe waits on LDS latency.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < 3) read_frags(base, q + 1, mf[(q + 1) & 1], nf[(q + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    if constexpr (F4) {
                        // slab q: half-wave h takes 32-k block 2q + h of the stage
                        const int sub = 2 * q + (lane >> 5);
                        acc[i][j] = mfma_f4(nf[q & 1][i], mf[q & 1][j], acc[i][j], scale_byte(scn_cur[i], sub, s),
                                            scale_byte(scm_cur[j], sub, s));
                    } else {
                        acc[i][j] = mfma_slab<DT>(nf[q & 1][i], mf[q & 1][j], acc[i][j]);
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Double-buffered pipeline with one barrier per stage: while stage s is
    // consumed from LDS buffer s&1, stage s+1 travels global -> registers; it
    // is written to the other buffer only after this wave's MFMAs of stage s
    // were issued, and the barrier publishes it (and frees buffer s&1).
    int s = 0;
    if (nk > 0) {
        if (nfull > 0) load_full(0); else load_ragged(0);
        store_stage(0);
        __syncthreads();
        for (; s + 1 < nfull; ++s) {
            next_scales();
            load_full(s + 1);
            __builtin_amdgcn_sched_barrier(0);  // keep the global loads ahead of the MFMAs
            compute(s & 1, s);
            store_stage((s + 1) & 1);
            __syncthreads();
        }
        if (s + 1 < nk) {  // the ragged stage is still to come
            next_scales();
            load_ragged(s + 1);
            compute(s & 1, s);
            store_stage((s + 1) & 1);
            __syncthreads();
            ++s;
        }
        next_scales();
        compute(s & 1, s);
    }

    // ---- epilogue: alpha, optional ReLU, store by ownership.
    // Accumulator register r of lane l in block (i, j) holds
    //   m = m0 + wave_m*WTM + 32*j + (l & 31)
    //   n = n0 + wave_n*WTN + 32*i + 8*(r/4) + 4*(l/32) + (r%4).
    const float alpha = p.alpha;
    const bool relu = p.relu != 0;
    if constexpr (SM != 0) {
        if (p.epi == TG_EPI_SOFTMAX) {  // the plan makes one tile span all of N
            softmax_epilogue<BM, WTM, WTN, FM, FN>(acc, p, m0, wave_m, wave_n, lane, smem);
            return;
        }
    }
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    with_out_type(p.out_dtype, [&](auto out) {
        constexpr int OUT = decltype(out)::value;
        const int64_t ldd = p.ldd;
        if (interior) {
            // no per-element checks; row offsets are wave-uniform multiples of ldd
            const int64_t lane_off = static_cast<int64_t>(n0 + wave_n * WTN + acc_row(lane, 0)) * ldd +
                                     (m0 + wave_m * WTM + acc_col(lane));
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float v = acc[i][j][r] * alpha;
                        if (relu) v = fmaxf(v, 0.0f);
                        store_out<OUT>(p.D, lane_off + (32 * i + 8 * (r >> 2) + (r & 3)) * ldd + 32 * j, v);
                    }
            return;
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = m0 + wave_m * WTM + 32 * j + acc_col(lane);
                const int nb = n0 + wave_n * WTN + 32 * i;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = nb + acc_row(lane, r);
                    float v = acc[i][j][r] * alpha;
                    if (relu) v = fmaxf(v, 0.0f);
                    if (m < M && n < N) store_out<OUT>(p.D, static_cast<int64_t>(n) * ldd + m, v);
                }
            }
        }
    });
}

template <int DT, int BM, int BN, int LC, int MW, int SM>
static hipError_t launch_rs(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, LC, MW, SM>),
                       dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg

// Instances: (id, dtype, BM, BN, min row alignment class, min waves per SIMD,
// group_m, softmax epilogue, eff%).  eff% is the expected MFMA efficiency the
// host plan chooser weighs tiles by (instances with the 2-byte shifting loader
// measure about 0.8x their 4-byte twins).
#define TG_RS_LIST(X)                              \
    X(19, TG_BF16, 128, 128, 4, 2, 4, 1, 45)       \
    X(20, TG_BF16, 128, 128, 2, 2, 4, 1, 36)       \
    X(21, TG_F16, 128, 128, 4, 2, 4, 1, 45)        \
    X(22, TG_F16, 128, 128, 2, 2, 4, 1, 36)        \
    X(23, TG_F32, 128, 128, 4, 2, 4, 1, 45)        \
    X(24, TG_BF16, 64, 64, 4, 2, 4, 1, 25)         \
    X(25, TG_F16, 64, 64, 4, 2, 4, 1, 25)          \
    X(26, TG_F32, 64, 64, 4, 2, 4, 1, 25)          \
    X(27, TG_BF16, 64, 64, 2, 2, 4, 1, 20)         \
    X(28, TG_F16, 64, 64, 2, 2, 4, 1, 20)          \
    X(29, TG_BF16, 256, 256, 4, 1, 4, 1, 69)       \
    X(30, TG_BF16, 256, 256, 2, 1, 4, 1, 55)       \
    X(31, TG_F16, 256, 256, 4, 1, 4, 1, 69)        \
    X(32, TG_F16, 256, 256, 2, 1, 4, 1, 55)        \
    X(33, TG_E4M3, 256, 256, 4, 1, 4, 0, 70)       \
    X(34, TG_E4M3, 256, 256, 1, 1, 4, 0, 56)       \
    X(35, TG_E4M3, 128, 128, 4, 2, 4, 0, 45)       \
    X(36, TG_E4M3, 64, 64, 4, 2, 4, 0, 25)         \
    X(37, TG_E4M3, 64, 64, 1, 2, 4, 0, 20)         \
    X(38, TG_E5M2, 256, 256, 4, 1, 4, 0, 70)       \
    X(39, TG_E5M2, 256, 256, 1, 1, 4, 0, 56)       \
    X(40, TG_E5M2, 128, 128, 4, 2, 4, 0, 45)       \
    X(41, TG_E5M2, 64, 64, 4, 2, 4, 0, 25)         \
    X(42, TG_E5M2, 64, 64, 1, 2, 4, 0, 20)        \
    X(61, TG_E2M1, 256, 256, 1, 1, 4, 0, 56)       \
    X(62, TG_E2M1, 64, 64, 1, 2, 4, 0, 20)         \
    X(63, TG_E2M3, 256, 256, 1, 1, 4, 0, 56)       \
    X(64, TG_E2M3, 64, 64, 1, 2, 4, 0, 20)         \
    X(65, TG_E3M2, 256, 256, 1, 1, 4, 0, 56)       \
    X(66, TG_E3M2, 64, 64, 1, 2, 4, 0, 20)

// Explicit instantiation, seen by both the device and the host pass.
#define TG_INSTANTIATE_RS(id, DT, BM, BN, LC, MW, GM, SM, EFF) \
    template __global__ void tg::gemm_kernel<DT, BM, BN, LC, MW, SM>(GemmArgs);
TG_RS_LIST(TG_INSTANTIATE_RS)

// The descriptors hold host launch functions, so they exist only in the host pass.
#ifndef __HIP_DEVICE_COMPILE__
#define TG_ENTRY_RS(id, DT, BM, BN, LC, MW, GM, SM, EFF)                                                  \
    {id, DT, BM, BN, TG_WIDE_STAGE_K(DT), 2, 2, (BM) / 2, (BN) / 2, 256, 2, 2 * ((BM) + (BN)) * 128,      \
     ((BM) / 2) * ((BN) / 2) / 64, LC, GM, EFF, &tg::launch_rs<DT, BM, BN, LC, MW, SM>, 0, SM, 0,          \
     TG_ELEM_BITS(DT) <= 8 ? 1 : 0},
extern const TgKernelDesc tg_entries_rs[] = {TG_RS_LIST(TG_ENTRY_RS)};
extern const int tg_entries_rs_count = sizeof(tg_entries_rs) / sizeof(tg_entries_rs[0]);
#endif  // __HIP_DEVICE_COMPILE__
