// K-sliced GEMM kernel for gfx950 (CDNA4): problems with few output tiles,
// on operand rows that start 16-byte aligned.
//
// With a 64 x 64 tile split 2 x 2 over four waves, each wave runs only two
// 32 x 32 MFMAs per 64-byte K stage between workgroup barriers.  Here every
// wave owns the whole 64 x 64 tile (2 x 2 blocks of 32 x 32, sixteen MFMAs per
// 128-byte K stage) and every fourth K stage: wave w takes stages w,
// w + 4, w + 8, ..., streamed global -> LDS by LDS-DMA (Tylo.jl manual, "Walk
// through GEMM", section 3 "Copy one K stage") into a ring of R stages that no
// other wave touches, so the only waits in the K loop are the wave's own
// vmcnt counts and no barrier is needed (section 4: the stage is released as
// soon as its consumer is done with it).  At the end the four partial tiles
// are written to LDS and summed in the fixed order w = 0, 1, 2, 3 (the same
// bits on every launch), then the epilogue (alpha, then the clamp) and the
// stores run over the summed tile, one thread per 16 consecutive m of one n.
#include "gemm_common.h"

namespace tg {

template <int DT, int R, int GM>
__global__ __launch_bounds__(256, 1) void gemm_kslice_kernel(GemmArgs p) {
    select_batch(p);
    constexpr int BM = 64, BN = 64, NW = 4;
    constexpr int ES = (DT == TG_F32) ? 4 : 2;
    constexpr int EPC = 16 / ES;
    constexpr int BKE = kRowBytes / ES;            // K elements per stage (128 bytes per row)
    constexpr int FM = BM / 32, FN = BN / 32;      // 2 x 2 blocks of 32 x 32 per wave
    constexpr int NA = BM / 8, NB = BN / 8;        // 1 KiB copies per stage: 8 rows x 128 bytes each
    constexpr int PER = NA + NB;
    constexpr int STAGE = (BM + BN) * kRowBytes;   // 16 KiB
    constexpr int RING = R * STAGE;                // per wave
    static_assert(R >= 2 && NW * RING <= 160 * 1024, "the four rings fit the LDS of a CU");
    static_assert(NW * BM * BN * 4 <= NW * RING, "the partial tiles fit where the rings were");
    static_assert((R - 1) * PER < 64, "vmcnt counts up to 63");

    __shared__ __attribute__((aligned(1024))) char smem[NW * RING];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const TileCoord tile = grouped_tile(p.tile, p.tiles_m, p.tiles_n, GM);
    const int m0 = tile.tm * BM, n0 = tile.tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    char* ring = smem + wave * RING;
    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const unsigned ring_base = __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(ring))));

    // copy sources: copy d of a stage moves rows 8d .. 8d+7 of A (d < NA)
    // or of B, whole 128-byte lines (the copy path is bound by the number of
    // line requests, so a stage covers whole lines); rows past M or N clamp
    // to the last row (their products only reach accumulators that are never
    // stored)
    const char* src[PER];
#pragma unroll
    for (int d = 0; d < PER; ++d) {
        const int j = d < NA ? d : d - NA;
        const int row = dma128_row(j, lane);
        src[d] = d < NA ? p.A + static_cast<int64_t>(min(m0 + row, M - 1)) * p.lda_b + dma128_chunk(j, lane) * kChunkBytes
                        : p.B + static_cast<int64_t>(min(n0 + row, N - 1)) * p.ldb_b + dma128_chunk(j, lane) * kChunkBytes;
    }
    // copy d of stage t into ring slot `slot`
    auto copy = [&](int d, int t, int slot) {
        const unsigned dst = __builtin_amdgcn_readfirstlane(ring_base + slot * STAGE + d * 1024);
        dma16(src[d] + static_cast<int64_t>(t) * kRowBytes, dst);
    };
    // fragments of slab q (the q-th 32 bytes of the stage's 128) from slot `slot`
    auto read = [&](int q, int slot, u32x4 (&fa)[FM], u32x4 (&fb)[FN]) {
        const char* base = ring + slot * STAGE;
#pragma unroll
        for (int j = 0; j < FM; ++j)
            fa[j] = *reinterpret_cast<const u32x4*>(base + lds_chunk_offset(32 * j + frag_row(lane), frag_chunk(lane, q)));
#pragma unroll
        for (int i = 0; i < FN; ++i)
            fb[i] = *reinterpret_cast<const u32x4*>(base + BM * kRowBytes +
                                                    lds_chunk_offset(32 * i + frag_row(lane), frag_chunk(lane, q)));
    };
    // the four slabs of the slot, each read one slab ahead of its MFMAs
    auto compute = [&](int slot) {
        u32x4 fa[2][FM], fb[2][FN];
        read(0, slot, fa[0], fb[0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < 3) read(q + 1, slot, fa[(q + 1) & 1], fb[(q + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i2 = 0; i2 < FN; ++i2)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i2][j] = mfma_slab<DT>(fb[q & 1][i2], fa[q & 1][j], acc[i2][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int nfull = K / BKE;
    // this wave's stages: wave, wave + NW, ...
    const int mine = nfull > wave ? (nfull - wave + NW - 1) / NW : 0;
    auto own = [&](int i) { return wave + NW * (i < mine - 1 ? i : mine - 1); };
    if (mine > 0) {
        // prologue: own stages 0 .. R-2 (an index past the last one reloads it,
        // so the number of copies in flight stays the same)
#pragma unroll
        for (int i = 0; i < R - 1; ++i)
#pragma unroll
            for (int d = 0; d < PER; ++d) copy(d, own(i), i);
        int slot = 0;
        for (int i = 0; i < mine; ++i) {
            // refill the slot the previous stage left (its fragments were
            // consumed by MFMAs, so its reads are complete)
            const int fill = slot == 0 ? R - 1 : slot - 1;
            const int t = own(i + R - 1);
#pragma unroll
            for (int d = 0; d < PER; ++d) copy(d, t, fill);
            wait_vm<(R - 1) * PER>();  // own stage i has landed
            compute(slot);
            slot = slot + 1 == R ? 0 : slot + 1;
        }
    }
    wait_vm<0>();  // no copy outlives the loop (the ring is reused below)

    if (K % BKE != 0 && wave == nfull % NW) {
        // ragged last stage: loaded through registers into slot 0 of this
        // wave's ring (no other wave reads it); k >= K become exact zeros
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        const int c = lane & 7;
        const int k0 = nfull * BKE + c * EPC;
#pragma unroll
        for (int i = 0; i < (BM + BN) / 8; ++i) {
            const int r = (lane >> 3) + 8 * i;  // rows 0..63 of A, then of B
            const char* row = r < BM ? p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b
                                     : p.B + static_cast<int64_t>(min(n0 + r - BM, N - 1)) * p.ldb_b;
            *reinterpret_cast<u32x4*>(ring + lds_chunk_offset(r, c)) = load_chunk_bounded<ES>(row, k0, K);
        }
        compute(0);
    }

    // partial tiles through LDS: wave w's value of (n, m) at part[w][n][m]
    __syncthreads();  // every wave is done with its ring
    float* part = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                part[(wave * BN + 32 * i + acc_row(lane, r)) * BM + 32 * j + acc_col(lane)] = acc[i][j][r];
    __syncthreads();

    // thread t: column n = t / 4 of the tile, 16 consecutive m from 16 * (t % 4)
    const int nl = tid >> 2, ml = 16 * (tid & 3);
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
        f32x4 s = *reinterpret_cast<const f32x4*>(part + nl * BM + ml + e);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const f32x4 q = *reinterpret_cast<const f32x4*>(part + (w * BN + nl) * BM + ml + e);
            s.x += q.x;
            s.y += q.y;
            s.z += q.z;
            s.w += q.w;
        }
        v[e] = s.x;
        v[e + 1] = s.y;
        v[e + 2] = s.z;
        v[e + 3] = s.w;
    }
    const float alpha = p.alpha;
    const bool relu = p.relu != 0;
    const int n = n0 + nl;
    if (n >= N) return;
    with_out_type(p.out_dtype, [&](auto out) {
        constexpr int OUT = decltype(out)::value;
        const int64_t col = static_cast<int64_t>(n) * p.ldd;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + ml + e;
            float x = v[e] * alpha;
            if (relu) x = fmaxf(x, 0.0f);
            if (m < M) store_out<OUT>(p.D, col + m, x);
        }
    });
}

template <int DT, int R, int GM>
static hipError_t launch_kslice(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_kslice_kernel<DT, R, GM>), dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tg

// Instances: (id, dtype, ring stages per wave R, group_m, eff%).  R = 2: four
// rings of two 16 KiB stages (128 KiB).  The planner only considers them when
// the output has at most half as many tiles as the GPU has CUs; there they
// measured 1.5x the 64 x 64 streaming instance (512x512x16384 bf16: 41.5 us
// against 64 us), hence the weight.
#define TG_KSLICE_LIST(X)                          \
    X(48, TG_BF16, 2, 4, 38)                       \
    X(49, TG_F16, 2, 4, 38)                        \
    X(50, TG_F32, 2, 4, 38)

#define TG_INSTANTIATE_KSLICE(id, DT, R, GM, EFF) \
    template __global__ void tg::gemm_kslice_kernel<DT, R, GM>(GemmArgs);
TG_KSLICE_LIST(TG_INSTANTIATE_KSLICE)

#ifndef __HIP_DEVICE_COMPILE__
// one wave grid cell holding the whole 64 x 64 tile, four K slices
#define TG_ENTRY_KSLICE(id, DT, R, GM, EFF)                                                                   \
    {id, DT, 64, 64, 128 / TG_ELEM_BYTES(DT), 1, 1, 64, 64, 256, R, 4 * (R) * 128 * 128, 64, 16, GM, EFF,    \
     &tg::launch_kslice<DT, R, GM>, 0, 0, 0, 0, 4},
extern const TgKernelDesc tg_entries_kslice[] = {TG_KSLICE_LIST(TG_ENTRY_KSLICE)};
extern const int tg_entries_kslice_count = sizeof(tg_entries_kslice) / sizeof(tg_entries_kslice[0]);
#endif  // __HIP_DEVICE_COMPILE__
