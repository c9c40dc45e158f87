// Small-tile streaming GEMM kernel for gfx950 (CDNA4): 64 x 64 and 128 x 128
// tiles for problems with few output tiles and a long K, on operand rows that
// start 16-byte aligned.
//
// Stages of SW = 64 or 128 bytes of K per row go global -> LDS directly
// (gfx950 LDS-DMA, one 16-byte vector per lane per instruction, no register
// staging; Tylo.jl manual, "Walk through GEMM", section 3 "Copy one K stage"),
// S stages deep, so each copy is issued about S-2 stages before its data is
// consumed.  The WM x WN waves that own the tile may be doubled into KG = 2
// groups, group 1 taking the second half of every stage's slabs: two waves
// per SIMD, so each SIMD keeps twice the LDS reads in flight, and the second
// group's partial tile is added into the first's through LDS at the end.
// Per stage, each wave runs SW/32/KG slabs of MFMAs; the LDS reads of
// the next slab and the copies of a future stage are issued one per MFMA so
// that the MFMA pipe never waits for them.  One barrier per stage, before its
// last slab, both publishes stage s+1 (every wave waited for its own copies
// first) and frees the buffer of stage s-1 for the copies issued right after
// it (section 4 "Consume, then release, the shared stage").  128-byte stages
// fetch whole 128-byte lines per row and need half the barriers per MFMA.
#include "gemm_common.h"

namespace tg {

template <int DT, int BM, int BN, int WM, int WN, int S, int GM, int SW, int KG>
__global__ __launch_bounds__(64 * WM * WN * KG, (WM * WN * KG) / 4) void gemm_stream_kernel(GemmArgs p) {
    select_batch(p);
    constexpr int NW = WM * WN * KG;            // waves per workgroup
    constexpr int NT = 64 * NW;
    constexpr int ES = (DT == TG_F32) ? 4 : 2;
    constexpr int EPC = 16 / ES;
    static_assert(SW == 64 || SW == 128, "stages of 64 or 128 bytes per row");
    constexpr int Q = SW / 32;                  // slabs (32 bytes of K per row) per stage
    constexpr int QL = Q / KG;                  // slabs per stage of one wave
    constexpr int CPR = SW / kChunkBytes;       // 16-byte chunks per row
    constexpr int RPC = 1024 / SW;              // rows per 1 KiB copy
    constexpr int BKE = SW / ES;                // K elements per stage
    constexpr int WTM = BM / WM, WTN = BN / WN; // output owned by one wave
    constexpr int FM = WTM / 32, FN = WTN / 32; // 32 x 32 MFMA blocks per wave
    constexpr int NA = BM / (RPC * NW);         // 1 KiB copies of A per wave per stage
    constexpr int NB = BN / (RPC * NW);
    constexpr int PER = NA + NB;
    constexpr int NR = FM + FN;                 // fragment reads per slab
    constexpr int STAGE = (BM + BN) * SW;
    static_assert(NA * RPC * NW == BM && NB * RPC * NW == BN, "copies must tile the stage");
    static_assert(S >= 3, "at least one stage in flight beyond the next");
    static_assert(KG == 1 || KG == 2, "one or two groups of waves over K");
    static_assert(QL % 2 == 0, "the last slab of a stage uses the second fragment set");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wave_mn = wave % (WM * WN);
    const int kg = wave / (WM * WN);                              // K group: slabs kg*QL .. kg*QL+QL-1 of each stage
    const int wave_m = wave_mn % WM, wave_n = wave_mn / WM;

    const TileCoord tile = grouped_tile(p.tile, p.tiles_m, p.tiles_n, GM);
    const int m0 = tile.tm * BM, n0 = tile.tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    const unsigned lds_base = __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) char*)(smem))));

    // ---- copy sources (rows past M or N clamp to the last row: their
    // products only reach accumulators that are never stored)
    const char* asrc[NA];
    const char* bsrc[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int j = wave * NA + i;
        const int row = SW == 64 ? dma_row(j, lane) : dma128_row(j, lane);
        const int chunk = SW == 64 ? dma_chunk(j, lane) : dma128_chunk(j, lane);
        asrc[i] = p.A + static_cast<int64_t>(min(m0 + row, M - 1)) * p.lda_b + chunk * kChunkBytes;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int j = wave * NB + i;
        const int row = SW == 64 ? dma_row(j, lane) : dma128_row(j, lane);
        const int chunk = SW == 64 ? dma_chunk(j, lane) : dma128_chunk(j, lane);
        bsrc[i] = p.B + static_cast<int64_t>(min(n0 + row, N - 1)) * p.ldb_b + chunk * kChunkBytes;
    }
    // copy d of stage t into buffer b
    auto copy = [&](int d, int t, int b) {
        const unsigned dst = __builtin_amdgcn_readfirstlane(lds_base + b * STAGE);
        const int64_t kb = static_cast<int64_t>(t) * SW;
        if (d < NA)
            dma16(asrc[d] + kb, dst + (wave * NA + d) * 1024);
        else
            dma16(bsrc[d - NA] + kb, dst + BM * SW + (wave * NB + d - NA) * 1024);
    };

    // ---- fragment read offsets within a stage; block steps are 32 rows
    auto chunk_offset = [](int row, int chunk) {
        return SW == 64 ? lds64_chunk_offset(row, chunk) : lds_chunk_offset(row, chunk);
    };
    int mread[QL], nread[QL];
#pragma unroll
    for (int q = 0; q < QL; ++q) {
        mread[q] = wave_m * WTM * SW + chunk_offset(frag_row(lane), frag_chunk(lane, kg * QL + q));
        nread[q] = (BM + wave_n * WTN) * SW + chunk_offset(frag_row(lane), frag_chunk(lane, kg * QL + q));
    }
    // read r of slab q from buffer b: m-side and n-side fragments alternate
    // while both last, so the first MFMAs of the slab get their operands first
    auto read = [&](int r, int q, int b, u32x4 (&fa)[FM], u32x4 (&fb)[FN]) {
        constexpr int P = FM < FN ? FM : FN;
        const char* base = smem + b * STAGE;
        bool is_m;
        int blk;
        if (r < 2 * P) {
            is_m = (r & 1) == 0;
            blk = r >> 1;
        } else {
            is_m = FM > FN;
            blk = r - P;
        }
        if (is_m)
            fa[blk] = *reinterpret_cast<const u32x4*>(base + mread[q] + blk * 32 * SW);
        else
            fb[blk] = *reinterpret_cast<const u32x4*>(base + nread[q] + blk * 32 * SW);
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nfull = K / BKE;
    u32x4 fa[2][FM], fb[2][FN];  // fragments of two consecutive slabs

    if (nfull > 0) {
        // prologue: stages 0 .. S-2 (indices past the last full stage reload
        // it, so every iteration sees the same number of copies in flight)
#pragma unroll
        for (int t = 0; t < S - 1; ++t)
#pragma unroll
            for (int d = 0; d < PER; ++d) copy(d, min(t, nfull - 1), t);
        wait_vm<(S - 2) * PER>();
        barrier();
#pragma unroll
        for (int r = 0; r < NR; ++r) read(r, 0, 0, fa[0], fb[0]);

        int buf = 0;           // buffer of stage s
        int fill = S - 1;      // buffer that receives stage s + S - 1
        for (int s = 0; s < nfull; ++s) {
            // this wave's slabs 0 .. QL-2 of stage s, each while reading the next
#pragma unroll
            for (int q = 0; q + 1 < QL; ++q)
                slab_with_side<DT, FM, FN, NR>(acc, fa[q & 1], fb[q & 1],
                                               [&](int k) { read(k, q + 1, buf, fa[(q + 1) & 1], fb[(q + 1) & 1]); });
            wait_vm<(S - 3) * PER>();  // this wave's copies of stage s+1 have landed
            barrier();                 // ... and everyone's; stage s-1's buffer is free
            const int nbuf = (buf + 1 == S) ? 0 : buf + 1;
            const int tload = min(s + S - 1, nfull - 1);
            // its last slab of stage s; meanwhile read its slab 0 of stage s+1 (on
            // the last stage this reads a buffer whose values go unused), then
            // copy stage s+S-1
            slab_with_side<DT, FM, FN, NR + PER>(acc, fa[1], fb[1], [&](int k) {
                if (k < NR)
                    read(k, 0, nbuf, fa[0], fb[0]);
                else
                    copy(k - NR, tload, fill);
            });
            buf = nbuf;
            fill = (fill + 1 == S) ? 0 : fill + 1;
        }
        wait_vm<0>();  // no copy outlives the loop
    }

    if (K % BKE != 0) {
        // ragged last stage: loaded through registers, elements with k >= K
        // become exact zeros; buffer 0 is free once every wave is past the loop
        __syncthreads();
        const int c = tid % CPR;
        const int k0 = nfull * BKE + c * EPC;
        char* base = smem;
#pragma unroll
        for (int i = 0; i < BM * CPR / NT; ++i) {
            const int r = tid / CPR + (NT / CPR) * i;
            const char* row = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
            *reinterpret_cast<u32x4*>(base + chunk_offset(r, c)) = load_chunk_bounded<ES>(row, k0, K);
        }
#pragma unroll
        for (int i = 0; i < BN * CPR / NT; ++i) {
            const int r = tid / CPR + (NT / CPR) * i;
            const char* row = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
            *reinterpret_cast<u32x4*>(base + BM * SW + chunk_offset(r, c)) = load_chunk_bounded<ES>(row, k0, K);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < QL; ++q) {
            // slabs wholly past K hold zeros only
            if (nfull * BKE + (kg * QL + q) * (BKE / Q) >= K) break;
#pragma unroll
            for (int r = 0; r < NR; ++r) read(r, q, 0, fa[0], fb[0]);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = mfma_slab<DT>(fb[0][i], fa[0][j], acc[i][j]);
        }
    }

    if constexpr (KG == 2) {
        // the second group's partial tile through LDS into the first group's
        // accumulators (one fixed order: the same bits on every launch)
        __syncthreads();  // every wave is done with the ring
        float* part = reinterpret_cast<float*>(smem) + wave_mn * (FN * FM * 16 * 64) + lane;
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) part[((i * FM + j) * 16 + r) * 64] = acc[i][j][r];
        }
        __syncthreads();
        if (kg == 1) return;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] += part[((i * FM + j) * 16 + r) * 64];
    }

    // ---- epilogue: alpha, optional ReLU, store by ownership (as above)
    const float alpha = p.alpha;
    const bool relu = p.relu != 0;
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    with_out_type(p.out_dtype, [&](auto out) {
        constexpr int OUT = decltype(out)::value;
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
                    if (interior || (m < M && n < N)) store_out<OUT>(p.D, static_cast<int64_t>(n) * p.ldd + m, v);
                }
            }
        }
    });
}

template <int DT, int BM, int BN, int WM, int WN, int S, int GM, int SW, int KG>
static hipError_t launch_stream(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_stream_kernel<DT, BM, BN, WM, WN, S, GM, SW, KG>),
                       dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)),
                       dim3(64 * WM * WN * KG), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg

// Instances: (id, dtype, BM, BN, waves along m, waves along n, LDS stages,
// group_m, stage bytes per row, K groups, eff%).  Each copy is issued S-2 stages
// ahead of its use; they win where few tiles each run a long K (kernel trace, bf16:
// 512x512x16384 64 us against 109 us for the register-staged 64 x 64; 2048^3
// 26.5 us against 30.0 us for the register-staged 128 x 128); the fp32
// 128 x 128 instance takes 2048^3 in 143.5 us against 162 us for the
// register-staged 128 x 128.  128-byte stages against 64-byte ones (bf16,
// same box): 64 x 64 at 1024 x 1024 x 4096 17.6 against 19.2 us, a tie at
// 1024^3; 128 x 128 at 2048^3 22.7 against 24.7 us and at 2048 x 2048 x 4096
// 36.9 against 40.5 us; fp32 (16 k per 64 bytes) gained nothing and keeps
// 64-byte stages.  KG = 2 groups of waves (two waves per SIMD) on the 64 x 64
// tile: 1024^3 7.0 against 7.8 us, 1024 x 1024 x 4096 16.4 against 18.8 us,
// 512 x 512 x 16384 42.7 against 54.8 us; on 128 x 128, whose waves already
// run four MFMAs per fragment pair, no gain.
#define TG_STREAM_LIST(X)                          \
    X(14, TG_BF16, 64, 64, 2, 2, 8, 4, 128, 2, 25)    \
    X(15, TG_F16, 64, 64, 2, 2, 8, 4, 128, 2, 25)     \
    X(16, TG_BF16, 128, 128, 2, 2, 5, 4, 128, 1, 46)  \
    X(17, TG_F16, 128, 128, 2, 2, 5, 4, 128, 1, 46)   \
    X(18, TG_F32, 128, 128, 2, 2, 8, 4, 64, 1, 50)

#define TG_INSTANTIATE_STREAM(id, DT, BM, BN, WM, WN, S, GM, SW, KG, EFF) \
    template __global__ void tg::gemm_stream_kernel<DT, BM, BN, WM, WN, S, GM, SW, KG>(GemmArgs);
TG_STREAM_LIST(TG_INSTANTIATE_STREAM)

#ifndef __HIP_DEVICE_COMPILE__
#define TG_ENTRY_STREAM(id, DT, BM, BN, WM, WN, S, GM, SW, KG, EFF)                                       \
    {id, DT, BM, BN, (SW) / TG_ELEM_BYTES(DT), WM, WN, (BM) / (WM), (BN) / (WN), 64 * (WM) * (WN) * (KG), S,  \
     (S) * ((BM) + (BN)) * (SW), ((BM) / (WM)) * ((BN) / (WN)) / 64, 16, GM, EFF,                            \
     &tg::launch_stream<DT, BM, BN, WM, WN, S, GM, SW, KG>, 0, 0, 0, 0, KG},
extern const TgKernelDesc tg_entries_stream[] = {TG_STREAM_LIST(TG_ENTRY_STREAM)};
extern const int tg_entries_stream_count = sizeof(tg_entries_stream) / sizeof(tg_entries_stream[0]);
#endif  // __HIP_DEVICE_COMPILE__
