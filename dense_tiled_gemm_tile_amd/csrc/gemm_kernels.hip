// Tiled dense GEMM with fused alpha/ReLU epilogue for gfx950 (CDNA4).
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
// Memory roles (all operands K-contiguous, D M-contiguous):
//   A storage: BM rows of the tile are A rows m (stride lda bytes lda_b)
//   B storage: BN rows of the tile are B columns n (stride ldb bytes ldb_b)
//   MFMA "A" operand <- B rows (n), MFMA "B" operand <- A rows (m), so the
//   32 lanes of an MFMA output column group walk consecutive m: stores of one
//   accumulator register write 2 x 128 contiguous bytes of D.
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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernel_table.h"
#include "tile_math.h"

namespace tg {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// 16-byte vector that only promises 4-byte alignment: still one dwordx4 access.
typedef unsigned int u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kThreads = 256;  // 4 waves

// ---------------------------------------------------------------- loaders

// One 16-byte chunk whose elements all lie below K.
template <int LOADCLASS>
__device__ __forceinline__ u32x4 load_chunk(const char* p) {
    if constexpr (LOADCLASS >= 4) {
        return *reinterpret_cast<const u32x4_a4*>(p);
    } else {
        // 2-byte (or, for 8-bit elements, 1-byte) aligned rows: load the
        // dword-aligned 16 bytes at or below p plus, when p sits mid-dword, the
        // next dword (which starts inside the chunk), then shift by the offset.
        const uintptr_t sub = reinterpret_cast<uintptr_t>(p) & (LOADCLASS == 1 ? 3u : 2u);
        const unsigned* q = reinterpret_cast<const unsigned*>(p - sub);
        u32x4 lo = *reinterpret_cast<const u32x4_a4*>(q);
        unsigned hi = 0;
        if (sub) hi = q[4];
        const unsigned sh = static_cast<unsigned>(sub);
        u32x4 v;
        v.x = __builtin_amdgcn_alignbyte(lo.y, lo.x, sh);
        v.y = __builtin_amdgcn_alignbyte(lo.z, lo.y, sh);
        v.z = __builtin_amdgcn_alignbyte(lo.w, lo.z, sh);
        v.w = __builtin_amdgcn_alignbyte(hi, lo.w, sh);
        return v;
    }
}

// A chunk that starts at element k0 of a row and may run past K: each element
// with k >= K becomes an exact zero and is not read.
template <int ES>
__device__ __forceinline__ u32x4 load_chunk_bounded(const char* row, int k0, int K) {
    unsigned w[4];
    if constexpr (ES == 1) {
        const unsigned char* r = reinterpret_cast<const unsigned char*>(row);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            unsigned v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = k0 + 4 * d + e;
                if (k < K) v |= static_cast<unsigned>(r[k]) << (8 * e);
            }
            w[d] = v;
        }
    } else if constexpr (ES == 2) {
        const unsigned short* r = reinterpret_cast<const unsigned short*>(row);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int k = k0 + 2 * d;
            const unsigned lo = (k < K) ? r[k] : 0u;
            const unsigned hi = (k + 1 < K) ? r[k + 1] : 0u;
            w[d] = lo | (hi << 16);
        }
    } else {
        const unsigned* r = reinterpret_cast<const unsigned*>(row);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int k = k0 + d;
            w[d] = (k < K) ? r[k] : 0u;
        }
    }
    u32x4 v;
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    return v;
}

// ---------------------------------------------------------------- MFMA step

// One 128-byte K slab of the (n-block i, m-block j) accumulator: the lane's
// 16-byte fragments of two consecutive chunks (lanes 0-31 chunk 2q, lanes
// 32-63 chunk 2q+1) feed the MFMA.  A and B use the same K order, so the sum is
// the same set of products.
template <int DT>
__device__ __forceinline__ f32x16 mfma_slab(u32x4 nfrag, u32x4 mfrag, f32x16 acc) {
    if constexpr (DT == TG_BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, nfrag), __builtin_bit_cast(bf16x8, mfrag), acc, 0, 0, 0);
    } else if constexpr (DT == TG_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, nfrag), __builtin_bit_cast(f16x8, mfrag), acc, 0, 0, 0);
    } else {
        // fp32: four K=2 MFMAs, element e of each lane's 4-float fragment.
        // (Cast the whole vector: a bit-cast of a single vector element
        // lvalue reads element 0 with this compiler.)
        const f32x4 nv = __builtin_bit_cast(f32x4, nfrag);
        const f32x4 mv = __builtin_bit_cast(f32x4, mfrag);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(nv.x, mv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(nv.y, mv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(nv.z, mv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(nv.w, mv.w, acc, 0, 0, 0);
        return acc;
    }
}

// 8-bit operands: one 32x32x64 MFMA per pair of 16-byte chunks.  Lane l
// supplies row l & 31; bytes 0-15 of half-wave h = l >> 5 are k [16h, 16h+16)
// of the 64 and bytes 16-31 are k [32 + 16h, 48 + 16h), for both operands
// alike.  Half-wave h also supplies the block-scale exponent of k-block h of
// its row (low byte of sn for the n side, sm for the m side); 127 means a
// scale of 1.
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <int DT>
__device__ __forceinline__ f32x16 mfma_f8(const u32x4 (&n)[2], const u32x4 (&m)[2], f32x16 acc, int sn, int sm) {
    constexpr int FMT = (DT == TG_E4M3) ? 0 : 1;  // operand format codes: 0 e4m3, 1 e5m2
    const i32x8 a = {static_cast<int>(n[0].x), static_cast<int>(n[0].y), static_cast<int>(n[0].z),
                     static_cast<int>(n[0].w), static_cast<int>(n[1].x), static_cast<int>(n[1].y),
                     static_cast<int>(n[1].z), static_cast<int>(n[1].w)};
    const i32x8 b = {static_cast<int>(m[0].x), static_cast<int>(m[0].y), static_cast<int>(m[0].z),
                     static_cast<int>(m[0].w), static_cast<int>(m[1].x), static_cast<int>(m[1].y),
                     static_cast<int>(m[1].z), static_cast<int>(m[1].w)};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, FMT, FMT, 0, sn, 0, sm);
}

// ---------------------------------------------------------------- output

// fp32 -> bfloat16, round to nearest even (the upper 16 bits of the binary32
// after adding half an ulp of the target, plus one when the kept part is odd);
// NaN stays a quiet NaN.
__device__ __forceinline__ unsigned short bf16_rne(float f) {
    const unsigned u = __builtin_bit_cast(unsigned, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<unsigned short>((u >> 16) | 0x40u);
    return static_cast<unsigned short>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Store epilogue value v to element idx of D in output type OUT (cuTile.jl
// tutorial "Matrix Multiplication", Step 4: keep the fp32 accumulator and
// convert on the way out).  fp16 uses the hardware conversion (round to
// nearest even, overflow to infinity, subnormals kept).
template <int OUT, bool NT = false>
__device__ __forceinline__ void store_out(void* D, int64_t idx, float v) {
    if constexpr (OUT == TG_F32) {
        float* d = static_cast<float*>(D) + idx;
        if constexpr (NT) __builtin_nontemporal_store(v, d); else *d = v;
    } else if constexpr (OUT == TG_BF16) {
        unsigned short* d = static_cast<unsigned short*>(D) + idx;
        const unsigned short b = bf16_rne(v);
        if constexpr (NT) __builtin_nontemporal_store(b, d); else *d = b;
    } else {
        _Float16* d = static_cast<_Float16*>(D) + idx;
        const _Float16 h = static_cast<_Float16>(v);
        if constexpr (NT) __builtin_nontemporal_store(h, d); else *d = h;
    }
}

// Batched calls (grid y = matrix index; cuTile.jl tutorial "Matrix
// Multiplication", "Where to go from here": batched operands): move the
// operand and output bases to this workgroup's matrix.
// A split-K launch is the same mechanism with the operand bases stepping
// along K: split s covers k in [s*split_k, min((s+1)*split_k, K)) and writes
// its fp32 partial product to its own workspace matrix.
__device__ __forceinline__ void select_batch(GemmArgs& p) {
    const int64_t b = blockIdx.y;
    p.A += b * p.batch_a_b;
    p.B += b * p.batch_b_b;
    p.D = static_cast<char*>(p.D) + b * p.batch_d_b;
    if (p.split_k) p.K = min(p.split_k, p.K - static_cast<int>(b) * p.split_k);
}

// Run f with the output type as a compile-time constant (one uniform branch
// per kernel, outside the unrolled store loops).
template <typename F>
__device__ __forceinline__ void with_out_type(int out, F&& f) {
    if (out == TG_BF16)
        f(std::integral_constant<int, TG_BF16>{});
    else if (out == TG_F16)
        f(std::integral_constant<int, TG_F16>{});
    else
        f(std::integral_constant<int, TG_F32>{});
}

// Softmax over n of x = alpha*S for every row m of a 2 x 2-wave tile whose
// n range spans all of N (n0 = 0, N <= BN); `acc` as the kernels hold it
// (block (i, j), register r: m = m0 + wave_m*WTM + 32j + acc_col(lane),
// n = wave_n*WTN + 32i + acc_row(lane, r)).  Row statistics are reduced
// within a lane (its FN*16 values), across the two half-waves (lanes l and
// l^32 hold the other n of each block) and across the two waves along n
// through LDS -- the collective a row-wise epilogue needs (Tylo.jl manual,
// "Walk through GEMM", section 5).  Every reduction runs in a fixed order, so
// results repeat bit for bit.  `smem` needs 2*BM floats and must be free.
template <int BM, int WTM, int WTN, int FM, int FN>
__device__ __forceinline__ void softmax_epilogue(f32x16 (&acc)[FN][FM], const GemmArgs& p, int m0, int wave_m,
                                                 int wave_n, int lane, char* smem) {
    const float alpha = p.alpha;
    const int M = p.M, N = p.N;
    float* red = reinterpret_cast<float*>(smem);  // [2][BM]: one value per (wave_n, m)
    const float neg_inf = -__builtin_huge_valf();
    float stat[FM];
    __syncthreads();  // the LDS stages are no longer read
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        float mx = neg_inf;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = wave_n * WTN + 32 * i + acc_row(lane, r);
                const float x = acc[i][j][r] * alpha;
                acc[i][j][r] = x;
                if (n < N) mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (lane < 32) red[wave_n * BM + wave_m * WTM + 32 * j + lane] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int idx = wave_m * WTM + 32 * j + acc_col(lane);
        stat[j] = fmaxf(red[idx], red[BM + idx]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = wave_n * WTN + 32 * i + acc_row(lane, r);
                const float e = (n < N) ? expf(acc[i][j][r] - stat[j]) : 0.0f;
                acc[i][j][r] = e;
                sum += e;
            }
        const float other = __shfl_xor(sum, 32);
        sum = (lane < 32) ? sum + other : other + sum;  // same order on both halves
        if (lane < 32) red[wave_n * BM + wave_m * WTM + 32 * j + lane] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int idx = wave_m * WTM + 32 * j + acc_col(lane);
        stat[j] = red[idx] + red[BM + idx];
    }
    with_out_type(p.out_dtype, [&](auto out) {
        constexpr int OUT = decltype(out)::value;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = m0 + wave_m * WTM + 32 * j + acc_col(lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = wave_n * WTN + 32 * i + acc_row(lane, r);
                    if (m < M && n < N) store_out<OUT>(p.D, static_cast<int64_t>(n) * p.ldd + m, acc[i][j][r] / stat[j]);
                }
            }
    });
}

// ---------------------------------------------------------------- kernel

// SM = 1: the instance also carries the softmax epilogue.
template <int DT, int BM, int BN, int LOADCLASS, int MINWAVES, int SM>
__global__ __launch_bounds__(kThreads, MINWAVES) void gemm_kernel(GemmArgs p) {
    select_batch(p);
    constexpr bool F8 = (DT == TG_E4M3 || DT == TG_E5M2);
    constexpr int ES = (DT == TG_F32) ? 4 : F8 ? 1 : 2;  // element bytes
    constexpr int EPC = 16 / ES;                    // elements per 16-byte chunk
    constexpr int BKE = kRowBytes / ES;             // K elements per stage
    constexpr int WTM = BM / 2, WTN = BN / 2;       // 2 x 2 waves
    constexpr int FM = WTM / 32, FN = WTN / 32;     // 32 x 32 MFMA blocks per wave
    constexpr int RA = BM / 32, RB = BN / 32;       // staged rows per thread
    constexpr int STAGE = (BM + BN) * kRowBytes;

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave & 1, wave_n = wave >> 1;

    const TileCoord tile = tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
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
    // block scales of the lane's rows: one dword per row and stage (the four
    // 32-k blocks of the stage's 128 k), for the stage being consumed (cur)
    // and the one being loaded (nxt)
    unsigned scm_cur[FM], scn_cur[FN], scm_nxt[FM], scn_nxt[FN];
    const int nblk = (K + 31) / 32;
    auto load_scales = [&](int s) {
        if constexpr (F8) {
            if (p.scale_a) {
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int m = min(m0 + wave_m * WTM + 32 * j + frag_row(lane), M - 1);
                    scm_nxt[j] = *reinterpret_cast<const unsigned*>(p.scale_a + m * p.lds_a + 4 * s);
                }
            } else {
#pragma unroll
                for (int j = 0; j < FM; ++j) scm_nxt[j] = 0x7F7F7F7Fu;
            }
            if (p.scale_b) {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    const int n = min(n0 + wave_n * WTN + 32 * i + frag_row(lane), N - 1);
                    scn_nxt[i] = *reinterpret_cast<const unsigned*>(p.scale_b + n * p.lds_b + 4 * s);
                }
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) scn_nxt[i] = 0x7F7F7F7Fu;
            }
        }
    };
    auto next_scales = [&]() {
        if constexpr (F8) {
#pragma unroll
            for (int j = 0; j < FM; ++j) scm_cur[j] = scm_nxt[j];
#pragma unroll
            for (int i = 0; i < FN; ++i) scn_cur[i] = scn_nxt[i];
        }
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
    auto load_full = [&](int s) {
        load_scales(s);
        const int kb = s * kRowBytes + c * 16;
#pragma unroll
        for (int i = 0; i < RA; ++i) sa[i] = load_chunk<LOADCLASS>(arow[i] + kb);
#pragma unroll
        for (int i = 0; i < RB; ++i) sb[i] = load_chunk<LOADCLASS>(brow[i] + kb);
    };
    auto load_ragged = [&](int s) {
        load_scales(s);
        const int k0 = s * BKE + c * EPC;
#pragma unroll
        for (int i = 0; i < RA; ++i) sa[i] = load_chunk_bounded<ES>(arow[i], k0, K);
#pragma unroll
        for (int i = 0; i < RB; ++i) sb[i] = load_chunk_bounded<ES>(brow[i], k0, K);
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
            const bool live = 4 * s + sub < nblk;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const int sn = live ? static_cast<int>(scn_cur[i] >> (8 * sub)) : 127;
                    const int sm = live ? static_cast<int>(scm_cur[j] >> (8 * sub)) : 127;
                    acc[i][j] = mfma_f8<DT>(nf[q][i], mf[q][j], acc[i][j], sn & 0xFF, sm & 0xFF);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto compute = [&](int buf, int s) {
        if constexpr (F8) {
            compute8(buf, s);
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
                for (int j = 0; j < FM; ++j) acc[i][j] = mfma_slab<DT>(nf[q & 1][i], mf[q & 1][j], acc[i][j]);
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

// ---------------------------------------------------------------- streaming kernel
//
// For operands whose rows are 16-byte aligned: stages of 64 bytes of K per row
// go global -> LDS directly (gfx950 LDS-DMA, one 16-byte vector per lane per
// instruction, no register staging), S stages deep, so each copy is issued
// about S-2 stages before its data is consumed.  Per stage, each wave runs two
// slabs of MFMAs; the LDS reads of the next slab and the copies of a future
// stage are issued one per MFMA so that the MFMA pipe never waits for them.
// One barrier per stage, between the two slabs, both publishes stage s+1
// (every wave waited for its own copies first) and frees the buffer of stage
// s-1 for the copies issued right after it.

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 64 lanes x 16 bytes from per-lane global addresses to LDS bytes
// [lds, lds + 1024), lane t at lds + 16*t.  Inline assembly keeps the
// compiler's wait-count pass from serialising every later LDS read behind the
// copy; completion is tracked with wait_vm below.
__device__ __forceinline__ void dma16(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds)
                 : "memory", "m0");
}
// The same copy through a buffer resource: base and byte range in SGPRs
// (`rsrc`), a 32-bit per-lane offset `voff` and a wave-uniform offset `soff`.
// Lanes whose offset falls outside the range write zeros instead of reading.
// Half the per-lane address data of dma16, and no per-copy vector arithmetic.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, unsigned voff, unsigned soff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                 :
                 : "v"(voff), "s"(lds), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource over [base, base + bytes) (gfx9 layout: 48-bit base,
// stride 0, byte count, 32-bit data format word); every field wave-uniform.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, unsigned bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r.w = 0x00020000;
    return r;
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier without the LDS fence of __syncthreads(): the streaming
// pipeline orders its LDS traffic explicitly (copies by wait_vm, fragment reads
// by the waits in front of the MFMAs that consume them), so waiting for every
// in-flight fragment read here would only stall the MFMA pipe.  The memory
// clobber keeps the compiler from moving LDS reads across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" : : : "memory"); }

// The MFMAs of one slab in (n-block, m-block) order; after MFMA m the side
// operations k in [ceil(m*T/MF), ceil((m+1)*T/MF)) are issued, and a
// scheduling barrier keeps the compiler from regrouping them.
template <int DT, int FM, int FN, int T, typename Side>
__device__ __forceinline__ void slab_with_side(f32x16 (&acc)[FN][FM], const u32x4 (&fa)[FM],
                                               const u32x4 (&fb)[FN], Side&& side) {
    constexpr int MF = FM * FN;
#pragma unroll
    for (int m = 0; m < MF; ++m) {
        const int i = m / FM, j = m % FM;
        acc[i][j] = mfma_slab<DT>(fb[i], fa[j], acc[i][j]);
#pragma unroll
        for (int k = (m * T + MF - 1) / MF; k < ((m + 1) * T + MF - 1) / MF; ++k) side(k);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int DT, int BM, int BN, int WM, int WN, int S, int GM>
__global__ __launch_bounds__(64 * WM * WN, (WM * WN) / 4) void gemm_stream_kernel(GemmArgs p) {
    select_batch(p);
    constexpr int NW = WM * WN;                 // waves per workgroup
    constexpr int NT = 64 * NW;
    constexpr int ES = (DT == TG_F32) ? 4 : 2;
    constexpr int EPC = 16 / ES;
    constexpr int BKE = kRow64Bytes / ES;       // K elements per stage
    constexpr int WTM = BM / WM, WTN = BN / WN; // output owned by one wave
    constexpr int FM = WTM / 32, FN = WTN / 32; // 32 x 32 MFMA blocks per wave
    constexpr int NA = BM / (16 * NW);          // 1 KiB copies of A per wave per stage
    constexpr int NB = BN / (16 * NW);
    constexpr int PER = NA + NB;
    constexpr int NR = FM + FN;                 // fragment reads per slab
    constexpr int STAGE = (BM + BN) * kRow64Bytes;
    static_assert(NA * 16 * NW == BM && NB * 16 * NW == BN, "copies must tile the stage");
    static_assert(S >= 3, "at least one stage in flight beyond the next");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int wave_m = wave % WM, wave_n = wave / WM;

    const TileCoord tile = tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM);
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
        asrc[i] = p.A + static_cast<int64_t>(min(m0 + dma_row(j, lane), M - 1)) * p.lda_b +
                  dma_chunk(j, lane) * kChunkBytes;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int j = wave * NB + i;
        bsrc[i] = p.B + static_cast<int64_t>(min(n0 + dma_row(j, lane), N - 1)) * p.ldb_b +
                  dma_chunk(j, lane) * kChunkBytes;
    }
    // copy d of stage t into buffer b
    auto copy = [&](int d, int t, int b) {
        const unsigned dst = __builtin_amdgcn_readfirstlane(lds_base + b * STAGE);
        if (d < NA)
            dma16(asrc[d] + t * kRow64Bytes, dst + (wave * NA + d) * 1024);
        else
            dma16(bsrc[d - NA] + t * kRow64Bytes, dst + BM * kRow64Bytes + (wave * NB + d - NA) * 1024);
    };

    // ---- fragment read offsets within a stage; block steps are 32 rows
    int mread[2], nread[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        mread[q] = wave_m * WTM * kRow64Bytes + lds64_chunk_offset(frag_row(lane), frag_chunk(lane, q));
        nread[q] = (BM + wave_n * WTN) * kRow64Bytes + lds64_chunk_offset(frag_row(lane), frag_chunk(lane, q));
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
            fa[blk] = *reinterpret_cast<const u32x4*>(base + mread[q] + blk * 32 * kRow64Bytes);
        else
            fb[blk] = *reinterpret_cast<const u32x4*>(base + nread[q] + blk * 32 * kRow64Bytes);
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nfull = K / BKE;
    u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];

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
        for (int r = 0; r < NR; ++r) read(r, 0, 0, fa0, fb0);

        int buf = 0;           // buffer of stage s
        int fill = S - 1;      // buffer that receives stage s + S - 1
        for (int s = 0; s < nfull; ++s) {
            // slab 0 of stage s; meanwhile read slab 1 of stage s
            slab_with_side<DT, FM, FN, NR>(acc, fa0, fb0, [&](int k) { read(k, 1, buf, fa1, fb1); });
            wait_vm<(S - 3) * PER>();  // this wave's copies of stage s+1 have landed
            barrier();                 // ... and everyone's; stage s-1's buffer is free
            const int nbuf = (buf + 1 == S) ? 0 : buf + 1;
            const int tload = min(s + S - 1, nfull - 1);
            // slab 1 of stage s; meanwhile read slab 0 of stage s+1 (on the last
            // stage this reads a buffer whose values go unused), then copy stage s+S-1
            slab_with_side<DT, FM, FN, NR + PER>(acc, fa1, fb1, [&](int k) {
                if (k < NR)
                    read(k, 0, nbuf, fa0, fb0);
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
        const int c = tid & 3;
        const int k0 = nfull * BKE + c * EPC;
        char* base = smem;
#pragma unroll
        for (int i = 0; i < BM * 4 / NT; ++i) {
            const int r = (tid >> 2) + (NT / 4) * i;
            const char* row = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
            *reinterpret_cast<u32x4*>(base + lds64_chunk_offset(r, c)) = load_chunk_bounded<ES>(row, k0, K);
        }
#pragma unroll
        for (int i = 0; i < BN * 4 / NT; ++i) {
            const int r = (tid >> 2) + (NT / 4) * i;
            const char* row = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
            *reinterpret_cast<u32x4*>(base + BM * kRow64Bytes + lds64_chunk_offset(r, c)) =
                load_chunk_bounded<ES>(row, k0, K);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int r = 0; r < NR; ++r) read(r, q, 0, fa0, fb0);
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = mfma_slab<DT>(fb0[i], fa0[j], acc[i][j]);
        }
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

template <int DT, int BM, int BN, int WM, int WN, int S, int GM>
static hipError_t launch_stream(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_stream_kernel<DT, BM, BN, WM, WN, S, GM>),
                       dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)),
                       dim3(64 * WM * WN), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- wide-row streaming kernel
//
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
// only 4-byte aligned, so the plain-store twins 43/44 carry it), bit 2 =
// the same for bf16/fp16 D, whose direct stores would write 64-byte halves of
// lines; bit 3 = the instance also carries the softmax epilogue (kept out of
// the plain instances, whose epilogue it would bloat); bit 4 = interior tiles
// transpose 4 x 4 register groups across lane quads and store 4 consecutive m
// per lane as one 8-byte vector for 16-bit D (measured: the bf16-D epilogue
// drops from about 31k to 21k cycles against the LDS transpose), bit 5 = the
// same for fp32 D as 16-byte vectors (measured slower than direct stores:
// fp32 D is bound by the write burst, and the shuffles add VALU work), bit 6 =
// 8-bit operands with block scales (their loads sit in the main loop, and the
// waits the compiler puts before their use also wait for copies, so the
// instances without scales do not carry them).
template <int DT, int GM, int NS, int RS, int ADDR, int SCHED, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_wide_kernel(GemmArgs p) {
    select_batch(p);
    constexpr int BM = 256, BN = 256, WM = 2;
    constexpr bool F8 = (DT == TG_E4M3 || DT == TG_E5M2);
    constexpr int ES = (DT == TG_F32) ? 4 : F8 ? 1 : 2;
    constexpr int EPC = 16 / ES;
    constexpr int BKE = kRowBytes / ES;          // K elements per stage
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

    __shared__ __attribute__((aligned(1024))) char smem[NS * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave % WM, wave_n = wave / WM;

    const TileCoord tile = tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, GM);
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
        }
    }
    // copy i of operand o (0: A, 1: B) of stage t into slot `slot`
    auto copy = [&](int o, int i, int t, int slot) {
        const unsigned dst = __builtin_amdgcn_readfirstlane(lds_base + slot * SLOT + (wave * NC + i) * 1024);
        if constexpr (ADDR == 0)
            dma16(src[o][i] + static_cast<int64_t>(t) * kRowBytes, dst);
        else
            dma16_buf(rsrc[o], voff[o][i], __builtin_amdgcn_readfirstlane(t * kRowBytes), dst);
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
    if constexpr (F8) {
        // 8-bit operands: a stage (128 k) is two 32x32x64 MFMAs per block.
        // The fragments of slabs 2p and 2p + 1 (chunks 4p + h and 4p + 2 + h
        // of half-wave h) together feed MFMA pair p; pair 0 runs while slabs
        // 2 and 3 are read and the copies of slabs 0-2 of the 16-bit schedule
        // go out (12), pair 1 after the barrier while slabs 0 and 1 of the
        // next stage are read and the last 4 copies go out, so the copy
        // order and the wait counts are those of the 16-bit schedule.  Block
        // scales (when given) come from the lane's rows, as in the
        // register-staged kernel.
        static_assert(SCHED == 1 && NS == 5, "the 8-bit schedule follows the spread copy schedule");
        constexpr bool SC = (EPI & 64) != 0;  // the instance applies block scales
        const int nk = nfull + ((K % BKE) != 0 ? 1 : 0);  // stages including a ragged one
        u32x4 g[4][FM], h[4][FN];
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
                const u32x4 nn[2] = {h[2 * pp][i], h[2 * pp + 1][i]};
                const u32x4 mm[2] = {g[2 * pp][j], g[2 * pp + 1][j]};
                if constexpr (SC) {
                    const int sn = live ? static_cast<int>((scn[i] >> (8 * sub)) & 0xFFu) : 127;
                    const int sm = live ? static_cast<int>((scm[j] >> (8 * sub)) & 0xFFu) : 127;
                    acc[i][j] = mfma_f8<DT>(nn, mm, acc[i][j], sn, sm);
                } else {
                    acc[i][j] = mfma_f8<DT>(nn, mm, acc[i][j], 127, 127);
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
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                read(r, 0, 0, 1, g[0], h[0]);
                read(r, 1, 0, 1, g[1], h[1]);
            }
            load_scales(0);
            int slot0 = 0;
            for (int s = 0; s < nfull; ++s) {
                const int sa = slot0, sb = wrap(slot0 + 1);
                const int na = wrap(slot0 + 2), nb = wrap(slot0 + 3);
                const int slot_h0 = wrap(slot0 + NS - 1);
                const int t1 = min(s + 1, nfull - 1), t2 = min(s + 2, nfull - 1);
                pair(0, s, [&](int m) {
                    if (m < NR) read(m, 2, sa, sb, g[2], h[2]); else read(m - NR, 3, sa, sb, g[3], h[3]);
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
                    if (m < NR) read(m, 0, na, nb, g[0], h[0]); else read(m - NR, 1, na, nb, g[1], h[1]);
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
#pragma unroll
            for (int i = 0; i < BM / 32; ++i) {
                const int r = stage_row(tid, i);
                const char* arow = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
                const char* brow = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
                *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) = load_chunk_bounded<ES>(arow, k0, K);
                *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) =
                    load_chunk_bounded<ES>(brow, k0, K);
            }
            if (nfull == 0) load_scales(0);  // otherwise loaded at the end of the last full stage
            __syncthreads();
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    read(r, 2 * pp, 0, 1, g[2 * pp], h[2 * pp]);
                    read(r, 2 * pp + 1, 0, 1, g[2 * pp + 1], h[2 * pp + 1]);
                }
                pair(pp, nfull, [](int) {});
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
                *reinterpret_cast<u32x4*>(smem + lds_chunk_offset(r, c)) = load_chunk_bounded<ES>(arow, k0, K);
                *reinterpret_cast<u32x4*>(smem + SLOT + lds_chunk_offset(r, c)) = load_chunk_bounded<ES>(brow, k0, K);
            }
            __syncthreads();
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
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
    const bool quad = (EPI & 16) && (p.out_dtype != TG_F32 || (EPI & 32)) && interior && (p.ldd & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.D) & (p.out_dtype == TG_F32 ? 15u : 7u)) == 0;
    if (quad) {
        // Interior tile: transpose each 4 x 4 group (4 lanes of a quad = 4
        // consecutive m, 4 registers = 4 consecutive n) in registers with two
        // DPP butterfly steps, so each lane holds 4 consecutive m of one n and
        // stores them as one 16-byte (fp32) or 8-byte (16-bit) vector: a
        // quarter of the store instructions, each writing whole 128-byte
        // (fp32) or 64-byte (16-bit) row pieces.
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
                        if constexpr (OUT == TG_F32) {
                            const f32x4 v = {x[0], x[1], x[2], x[3]};
                            f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(p.D) + idx);
                            if constexpr (EPI & 1) __builtin_nontemporal_store(v, d); else *d = v;
                        } else {
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
        static_assert((EPI & 4) == 0 || 256 * PITCH16 <= NS * SLOT, "16-bit tile fits the ring");
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
        static_assert(EPI < 2 || 128 * PITCH <= NS * SLOT, "transpose buffer fits the ring");
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

template <int DT, int GM, int NS, int RS, int ADDR, int SCHED, int EPI>
static hipError_t launch_wide(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_wide_kernel<DT, GM, NS, RS, ADDR, SCHED, EPI>),
                       dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- hybrid kernel
//
// On gfx950 an LDS read issued on a SIMD more often than about once per 128
// MFMA cycles slows that SIMD's MFMA pipe (twice that rate halves it), whatever
// wave it comes from, while vector-memory loads and LDS-DMA copies issue almost
// for free.  A 128 x 128 wave tile with both operands in LDS needs twice that
// read rate, so here only the A side (the m rows) goes through LDS, staged by
// LDS-DMA S stages deep; the B side (the n rows) is loaded by each wave
// straight from global memory (L2/L1) into registers in MFMA operand layout,
// P stages ahead, through a ring of P+1 stages of fragments.  16x16x32 MFMAs
// are used so that each direct load reads 16 rows x 64 contiguous bytes (one
// fully used 64-byte sector per row) instead of 32 rows x 32 bytes.  One
// barrier per stage publishes the next A stage and frees the oldest.

// The MFMA is written as inline assembly with the accumulator tied in place
// ("+a"): with the builtin, the register allocator does not keep the result
// in the accumulator's registers for this many 16x16 accumulators and adds
// chains of AGPR moves that serialise on MFMA completion.  In this kernel the
// operands come only from loads (waited by vmcnt/lgkmcnt), each accumulator
// is touched once per stage, and mfma16_drain() pads before any other read of
// the accumulators, which covers the MFMA hazards the compiler cannot see.
template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 afrag, u32x4 bfrag, f32x4 acc) {
    if constexpr (DT == TG_BF16)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(afrag), "v"(bfrag));
    else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(afrag), "v"(bfrag));
    return acc;
}

// Wait states after the last MFMA before its results are read by other
// instructions (more than the 16x16x32 pass count requires).
__device__ __forceinline__ void mfma16_drain() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

template <int DT, int S, int P>
__global__ __launch_bounds__(256, 1) void gemm_hybrid_kernel(GemmArgs p) {
    select_batch(p);
    static_assert(DT == TG_BF16 || DT == TG_F16, "16-bit operands");
    constexpr int BM = 256, BN = 256;
    constexpr int EPC = 8;                   // elements per 16-byte chunk
    constexpr int BKE = kRow64Bytes / 2;     // K elements per stage
    constexpr int WTM = 128, WTN = 128;      // 2 x 2 waves
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int NA = BM / 64;              // 1 KiB A copies per wave per stage
    constexpr int ASTAGE = BM * kRow64Bytes;
    constexpr int G = P + 1;                 // B fragment ring, in stages
    constexpr int OPS = FN + NA;             // vector-memory operations per stage
    static_assert(P >= S - 3, "the steady-state copy wait assumes P >= S - 3");
    static_assert(S >= 3, "at least one stage in flight beyond the next");
    // copies of stage t are the last vector-memory operations of stage t-S+1;
    // waiting for stage s+1 at the start of stage s leaves the operations of
    // stages s-S+3 .. s-1 in flight
    constexpr int WAIT_FIRST = (S - 2) * NA + P * FN;
    constexpr int WAIT_STEADY = (S - 3) * OPS;
    static_assert(WAIT_FIRST < 64 && WAIT_STEADY < 64, "vmcnt is 6 bits");
    constexpr int LDS = (S * ASTAGE > (BM + BN) * kRow64Bytes) ? S * ASTAGE : (BM + BN) * kRow64Bytes;

    __shared__ __attribute__((aligned(1024))) char smem[LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave & 1, wave_n = wave >> 1;

    const TileCoord tile = tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
    const int m0 = tile.tm * BM, n0 = tile.tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    const unsigned lds_base = __builtin_amdgcn_readfirstlane(
        static_cast<unsigned>(reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) char*)(smem))));

    // ---- A copies (rows past M clamp to the last row)
    const char* asrc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int j = wave * NA + i;
        asrc[i] = p.A + static_cast<int64_t>(min(m0 + dma_row(j, lane), M - 1)) * p.lda_b +
                  dma_chunk(j, lane) * kChunkBytes;
    }
    auto copy = [&](int d, int t, int b) {
        const unsigned dst = __builtin_amdgcn_readfirstlane(lds_base + b * ASTAGE);
        dma16(asrc[d] + t * kRow64Bytes, dst + (wave * NA + d) * 1024);
    };
    // ---- A fragment reads: block j covers rows wave_m*WTM + 16j .. +15
    const int aread = wave_m * WTM * kRow64Bytes + lds64_chunk_offset(frag16_row(lane), frag16_chunk(lane));
    auto read_a = [&](int j, int b, u32x4 (&fa)[FM]) {
        fa[j] = *reinterpret_cast<const u32x4*>(smem + b * ASTAGE + aread + j * 16 * kRow64Bytes);
    };
    // ---- B fragments straight from global memory: stage t of row block i is
    // the 16 bytes at k = 32t + 8*(lane/16) of row n0 + wave_n*WTN + 16i + lane%16
    // (the same k order as the A fragments read from LDS)
    const char* bsrc[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i)
        bsrc[i] = p.B + static_cast<int64_t>(min(n0 + wave_n * WTN + 16 * i + frag16_row(lane), N - 1)) * p.ldb_b +
                  frag16_chunk(lane) * kChunkBytes;
    u32x4 fb[G][FN];
    auto load_b = [&](int i, int t, int slot) {
        fb[slot][i] = *reinterpret_cast<const u32x4*>(bsrc[i] + t * kRow64Bytes);
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nfull = K / BKE;
    u32x4 fa[FM];  // A fragments of the current stage, refilled in place

    if (nfull > 0) {
        // prologue: A stages 0 .. S-2, then B stages 0 .. P-1 (indices past the
        // end repeat the last one, keeping the number of operations in flight
        // the same every stage)
#pragma unroll
        for (int t = 0; t < S - 1; ++t)
#pragma unroll
            for (int d = 0; d < NA; ++d) copy(d, min(t, nfull - 1), t);
#pragma unroll
        for (int t = 0; t < P; ++t)
#pragma unroll
            for (int i = 0; i < FN; ++i) load_b(i, min(t, nfull - 1), t);
        wait_vm<WAIT_FIRST>();
        barrier();
#pragma unroll
        for (int j = 0; j < FM; ++j) read_a(j, 0, fa);

        int nbuf = 1;      // A buffer of stage s+1
        int fill = S - 1;  // A buffer that receives stage s + S - 1
        // Stage s; u = s mod G picks the B ring slot.  MFMAs run m-block by
        // m-block: once the eight MFMAs of A fragment j are issued, fragment j
        // of stage s+1 is read into the same registers.  Between MFMAs go one
        // B load (stage s+P) per m-block and the NA copies (stage s+S-1), so
        // every group of eight MFMAs carries at most one LDS read, one load
        // and one copy.  A of stage s was read during stage s-1, so at the
        // barrier that opens stage s every wave is done with stage s-1's buffer.
        auto stage = [&](int s, int u) {
            const int cur = u % G, pf = (u + P) % G;
            const int tb = min(s + P, nfull - 1);
            const int tload = min(s + S - 1, nfull - 1);
            wait_vm<WAIT_STEADY>();  // this wave's copies of stage s+1 have landed
            barrier();               // ... and everyone's
#pragma unroll
            for (int j = 0; j < FM; ++j) {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    acc[i][j] = mfma16<DT>(fb[cur][i], fa[j], acc[i][j]);
                    if (i == 2) load_b(j, tb, pf);
                    if (i == 5 && j < NA) copy(j, tload, fill);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // on the last stage this reads a buffer whose values go unused
                read_a(j, nbuf, fa);
            }
            nbuf = (nbuf + 1 == S) ? 0 : nbuf + 1;
            fill = (fill + 1 == S) ? 0 : fill + 1;
        };
        // whole ring turns without guards, then the last nfull mod G stages
        int s0 = 0;
        for (; s0 + G <= nfull; s0 += G) {
#pragma unroll
            for (int u = 0; u < G; ++u) stage(s0 + u, u);
        }
#pragma unroll
        for (int u = 0; u < G - 1; ++u)
            if (s0 + u < nfull) stage(s0 + u, u);
        wait_vm<0>();  // no copy outlives the loop
    }

    if (K % BKE != 0) {
        // ragged last stage, both operands through LDS with exact zeros past K
        __syncthreads();
        const int c = tid & 3;
        const int k0 = nfull * BKE + c * EPC;
#pragma unroll
        for (int i = 0; i < BM / 64; ++i) {
            const int r = (tid >> 2) + 64 * i;
            const char* row = p.A + static_cast<int64_t>(min(m0 + r, M - 1)) * p.lda_b;
            *reinterpret_cast<u32x4*>(smem + lds64_chunk_offset(r, c)) = load_chunk_bounded<2>(row, k0, K);
        }
#pragma unroll
        for (int i = 0; i < BN / 64; ++i) {
            const int r = (tid >> 2) + 64 * i;
            const char* row = p.B + static_cast<int64_t>(min(n0 + r, N - 1)) * p.ldb_b;
            *reinterpret_cast<u32x4*>(smem + BM * kRow64Bytes + lds64_chunk_offset(r, c)) =
                load_chunk_bounded<2>(row, k0, K);
        }
        __syncthreads();
        u32x4 fbt[FN];
#pragma unroll
        for (int j = 0; j < FM; ++j) read_a(j, 0, fa);
#pragma unroll
        for (int i = 0; i < FN; ++i)
            fbt[i] = *reinterpret_cast<const u32x4*>(
                smem + (BM + wave_n * WTN + 16 * i) * kRow64Bytes +
                lds64_chunk_offset(frag16_row(lane), frag16_chunk(lane)));
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = mfma16<DT>(fbt[i], fa[j], acc[i][j]);
    }

    mfma16_drain();

    // ---- epilogue: alpha, optional ReLU, store by ownership
    const float alpha = p.alpha;
    const bool relu = p.relu != 0;
    const bool interior = (m0 + BM <= M) && (n0 + BN <= N);
    with_out_type(p.out_dtype, [&](auto out) {
        constexpr int OUT = decltype(out)::value;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = m0 + wave_m * WTM + 16 * j + acc16_col(lane);
                const int nb = n0 + wave_n * WTN + 16 * i;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = nb + acc16_row(lane, r);
                    float v = acc[i][j][r] * alpha;
                    if (relu) v = fmaxf(v, 0.0f);
                    if (interior || (m < M && n < N)) store_out<OUT>(p.D, static_cast<int64_t>(n) * p.ldd + m, v);
                }
            }
        }
    });
}

template <int DT, int S, int P>
static hipError_t launch_hybrid(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_hybrid_kernel<DT, S, P>), dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- table

template <int DT, int BM, int BN, int LC, int MW, int SM>
static hipError_t launch(const GemmArgs& a, int64_t grid, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, LC, MW, SM>), dim3(static_cast<unsigned>(grid), static_cast<unsigned>(batch)),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- split-K reduction
//
// One thread per 4 consecutive m of one output column n: the fp32 partial
// products of the splits are added in split order (so every launch gives the
// same bits), then alpha, the clamp and the conversion of the output type.
// Workspace layout: split s, element (m, n) at ws[s*M*N + n*M + m].
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits, int M,
                                                            int N, void* D, int64_t ldd, float alpha, int relu) {
    const int mq = (M + 3) / 4;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (t >= static_cast<int64_t>(mq) * N) return;
    const int n = static_cast<int>(t / mq);
    const int m = static_cast<int>(t % mq) * 4;
    const int64_t plane = static_cast<int64_t>(M) * N;
    const float* src = ws + static_cast<int64_t>(n) * M + m;
    const int cnt = min(4, M - m);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((M & 3) == 0) {
        // whole 16-byte groups (the workspace base is 16-byte aligned)
        for (int s = 0; s < splits; ++s) {
            const f32x4 q = *reinterpret_cast<const f32x4*>(src + s * plane);
            acc[0] += q.x;
            acc[1] += q.y;
            acc[2] += q.z;
            acc[3] += q.w;
        }
    } else {
        for (int s = 0; s < splits; ++s) {
            const float* q = src + s * plane;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < cnt) acc[e] += q[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < cnt) {
            float v = acc[e] * alpha;
            if (relu) v = fmaxf(v, 0.0f);
            store_out<OUT>(D, static_cast<int64_t>(n) * ldd + m + e, v);
        }
    }
}


// ---------------------------------------------------------------- staged operand copy
//
// Rows of A (rows [0, M)) and then of B (rows [M, rows)) copied into dense
// rows of cpr 16-byte chunks each, so that every copied row starts 16-byte
// aligned and holds a whole number of 128-byte K stages; the elements from K
// to the end of a copied row are exact zeros.  One wave per row at a time,
// lanes on consecutive chunks (1 KiB per wave instruction on both sides).
// A chunk that lies wholly below K takes the shifting 16-byte load (a
// source row is only element-aligned); the chunk that straddles K reads its
// elements one by one.
template <int ES>
__global__ __launch_bounds__(256) void stage_rows_kernel(const char* __restrict__ A, int64_t lda_b, int64_t M,
                                                         const char* __restrict__ B, int64_t ldb_b, int64_t rows,
                                                         int K, int64_t cpr, char* __restrict__ dstA,
                                                         char* __restrict__ dstB) {
    constexpr int EPC = 16 / ES;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
    const int64_t full = K / EPC;  // chunks entirely below K
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); r < rows; r += nwaves) {
        const bool in_a = r < M;
        const int64_t rr = in_a ? r : r - M;
        const char* src = in_a ? A + rr * lda_b : B + rr * ldb_b;
        char* dst = (in_a ? dstA : dstB) + rr * cpr * 16;
        for (int64_t c = lane; c < cpr; c += 64) {
            u32x4 v;
            if (c < full) {
                v = load_chunk<(ES == 1 ? 1 : ES == 2 ? 2 : 4)>(src + c * 16);
            } else if (c * EPC < K) {
                v = load_chunk_bounded<ES>(src, static_cast<int>(c * EPC), K);
            } else {
                v.x = v.y = v.z = v.w = 0u;
            }
            *reinterpret_cast<u32x4*>(dst + c * 16) = v;
        }
    }
}

}  // namespace tg

// Row softmax over n of an fp32 D in place: one thread per m (consecutive
// threads read consecutive m of each row n, so every pass is coalesced); max,
// then the sum of exponentials, then the normalised values, each pass in
// increasing n.
__global__ __launch_bounds__(256) void tg_softmax_rows_kernel(float* D, int M, int N, int64_t ldd) {
    const int m = blockIdx.x * 256 + threadIdx.x;
    if (m >= M) return;
    float mx = -__builtin_huge_valf();
    for (int n = 0; n < N; ++n) mx = fmaxf(mx, D[static_cast<int64_t>(n) * ldd + m]);
    float sum = 0.0f;
    for (int n = 0; n < N; ++n) sum += expf(D[static_cast<int64_t>(n) * ldd + m] - mx);
    for (int n = 0; n < N; ++n) {
        float* d = D + static_cast<int64_t>(n) * ldd + m;
        *d = expf(*d - mx) / sum;
    }
}

hipError_t tg_softmax_rows(float* D, int M, int N, int64_t ldd, hipStream_t stream) {
    hipLaunchKernelGGL(tg_softmax_rows_kernel, dim3(static_cast<unsigned>((M + 255) / 256)), dim3(256), 0, stream, D,
                       M, N, ldd);
    return hipGetLastError();
}

hipError_t tg_splitk_reduce(const float* ws, int splits, int M, int N, void* D, int64_t ldd, float alpha,
                            int relu, int out_dtype, hipStream_t stream) {
    const int64_t threads = static_cast<int64_t>((M + 3) / 4) * N;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if (out_dtype == TG_BF16)
        hipLaunchKernelGGL(tg::splitk_reduce_kernel<TG_BF16>, grid, dim3(256), 0, stream, ws, splits, M, N, D, ldd,
                           alpha, relu);
    else if (out_dtype == TG_F16)
        hipLaunchKernelGGL(tg::splitk_reduce_kernel<TG_F16>, grid, dim3(256), 0, stream, ws, splits, M, N, D, ldd,
                           alpha, relu);
    else
        hipLaunchKernelGGL(tg::splitk_reduce_kernel<TG_F32>, grid, dim3(256), 0, stream, ws, splits, M, N, D, ldd,
                           alpha, relu);
    return hipGetLastError();
}

hipError_t tg_stage_operands(const char* A, int64_t lda_b, int64_t M, const char* B, int64_t ldb_b, int64_t N, int K,
                             int es, int64_t row_bytes, char* dstA, char* dstB, hipStream_t stream) {
    const int64_t rows = M + N;
    const int64_t blocks = (rows + 3) / 4;
    const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
    const int64_t cpr = row_bytes / 16;
    if (es == 1)
        hipLaunchKernelGGL(tg::stage_rows_kernel<1>, grid, dim3(256), 0, stream, A, lda_b, M, B, ldb_b, rows, K, cpr,
                           dstA, dstB);
    else if (es == 2)
        hipLaunchKernelGGL(tg::stage_rows_kernel<2>, grid, dim3(256), 0, stream, A, lda_b, M, B, ldb_b, rows, K, cpr,
                           dstA, dstB);
    else
        hipLaunchKernelGGL(tg::stage_rows_kernel<4>, grid, dim3(256), 0, stream, A, lda_b, M, B, ldb_b, rows, K, cpr,
                           dstA, dstB);
    return hipGetLastError();
}

// Kernel instances.
//   register-staged: (id, dtype, BM, BN, min row alignment class, min waves per SIMD, group_m, eff%)
//   streaming:       (id, dtype, BM, BN, waves along m, waves along n, LDS stages, group_m, eff%)
//   hybrid:          (id, dtype, A stages in LDS, B prefetch stages, group_m, eff%), 256 x 256
// eff% is the expected MFMA efficiency the host plan chooser weighs tiles by
// (instances with the 2-byte shifting loader measure about 0.8x their 4-byte
// twins).  The 64 x 64 and 128 x 128 streaming instances (45-48) keep 7
// stages of copies in flight and win where few tiles each run a long K
// (kernel trace, bf16: 512x512x16384 64 us against 109 us for the
// register-staged 64 x 64; 2048^3 26.5 us against 30.0 us for the
// register-staged 128 x 128); their weights tie with or just beat those
// register-staged twins, whose plans they take over for aligned rows.  fp32
// operands: the wide kernel reaches 96 % of the fp32 MFMA peak at 4096^3
// (911 us), whose 64-cycle MFMAs hide its copy and barrier overheads; the
// 128 x 128 streaming instance (49) takes 2048^3 in 143.5 us against 162 us
// for the register-staged 128 x 128.
#define TG_RS_LIST(X)                           \
    X(2, TG_BF16, 256, 256, 4, 1, 4, 0, 70)     \
    X(3, TG_BF16, 256, 256, 2, 1, 4, 0, 56)     \
    X(4, TG_F16, 256, 256, 4, 1, 4, 0, 70)      \
    X(5, TG_F16, 256, 256, 2, 1, 4, 0, 56)      \
    X(6, TG_BF16, 128, 128, 4, 2, 4, 1, 45)     \
    X(7, TG_BF16, 128, 128, 2, 2, 4, 1, 36)     \
    X(8, TG_F16, 128, 128, 4, 2, 4, 1, 45)      \
    X(9, TG_F16, 128, 128, 2, 2, 4, 1, 36)      \
    X(10, TG_F32, 128, 128, 4, 2, 4, 1, 45)     \
    X(30, TG_BF16, 64, 64, 4, 2, 4, 1, 25)      \
    X(31, TG_F16, 64, 64, 4, 2, 4, 1, 25)       \
    X(32, TG_F32, 64, 64, 4, 2, 4, 1, 25)       \
    X(33, TG_BF16, 64, 64, 2, 2, 4, 1, 20)      \
    X(34, TG_F16, 64, 64, 2, 2, 4, 1, 20)       \
    X(37, TG_BF16, 256, 256, 4, 1, 4, 1, 69)    \
    X(38, TG_BF16, 256, 256, 2, 1, 4, 1, 55)    \
    X(39, TG_F16, 256, 256, 4, 1, 4, 1, 69)     \
    X(40, TG_F16, 256, 256, 2, 1, 4, 1, 55)     \
    X(50, TG_E4M3, 256, 256, 4, 1, 4, 0, 70)    \
    X(51, TG_E4M3, 256, 256, 1, 1, 4, 0, 56)    \
    X(52, TG_E4M3, 128, 128, 4, 2, 4, 0, 45)    \
    X(53, TG_E4M3, 64, 64, 4, 2, 4, 0, 25)      \
    X(54, TG_E4M3, 64, 64, 1, 2, 4, 0, 20)      \
    X(55, TG_E5M2, 256, 256, 4, 1, 4, 0, 70)    \
    X(56, TG_E5M2, 256, 256, 1, 1, 4, 0, 56)    \
    X(57, TG_E5M2, 128, 128, 4, 2, 4, 0, 45)    \
    X(58, TG_E5M2, 64, 64, 4, 2, 4, 0, 25)      \
    X(59, TG_E5M2, 64, 64, 1, 2, 4, 0, 20)
#define TG_STREAM_LIST(X)                       \
    X(0, TG_BF16, 256, 256, 2, 4, 4, 4, 100)    \
    X(1, TG_F16, 256, 256, 2, 4, 4, 4, 100)     \
    X(11, TG_BF16, 256, 256, 2, 2, 4, 4, 90)    \
    X(12, TG_F16, 256, 256, 2, 2, 4, 4, 90)     \
    X(45, TG_BF16, 64, 64, 2, 2, 8, 4, 25)      \
    X(46, TG_F16, 64, 64, 2, 2, 8, 4, 25)       \
    X(47, TG_BF16, 128, 128, 2, 2, 8, 4, 46)    \
    X(48, TG_F16, 128, 128, 2, 2, 8, 4, 46)     \
    X(49, TG_F32, 128, 128, 2, 2, 8, 4, 50)

#define TG_HYBRID_LIST(X)                       \
    X(13, TG_BF16, 5, 2, 4, 75)                 \
    X(14, TG_F16, 5, 2, 4, 75)

#define TG_WIDE_LIST(X)                         \
    X(15, TG_BF16, 4, 5, 16, 0, 0, 0, 105)      \
    X(16, TG_F16, 4, 5, 16, 0, 0, 0, 105)       \
    X(17, TG_F32, 4, 5, 16, 0, 0, 0, 93)        \
    X(18, TG_BF16, 4, 4, 16, 0, 0, 0, 10)       \
    X(19, TG_BF16, 4, 5, 8, 0, 0, 0, 10)        \
    X(20, TG_BF16, 4, 5, 8, 1, 0, 0, 10)        \
    X(21, TG_BF16, 4, 5, 16, 1, 0, 0, 10)       \
    X(22, TG_BF16, 4, 5, 16, 1, 1, 17, 107)     \
    X(23, TG_BF16, 4, 5, 8, 1, 1, 5, 10)        \
    X(24, TG_F16, 4, 5, 16, 1, 1, 17, 107)      \
    X(25, TG_F32, 4, 5, 16, 1, 1, 5, 96)        \
    X(26, TG_BF16, 4, 5, 16, 1, 1, 0, 10)       \
    X(27, TG_BF16, 4, 5, 16, 1, 1, 2, 10)       \
    X(28, TG_BF16, 4, 5, 16, 1, 1, 3, 10)       \
    X(29, TG_BF16, 4, 5, 16, 1, 1, 1, 10)       \
    X(35, TG_BF16, 4, 5, 16, 1, 1, 13, 106)     \
    X(36, TG_F16, 4, 5, 16, 1, 1, 13, 106)      \
    X(41, TG_BF16, 4, 5, 16, 1, 1, 49, 10)      \
    X(42, TG_F16, 4, 5, 16, 1, 1, 5, 10)        \
    X(43, TG_BF16, 4, 5, 16, 1, 1, 18, 107)     \
    X(44, TG_F16, 4, 5, 16, 1, 1, 18, 107)      \
    X(60, TG_E4M3, 4, 5, 16, 1, 1, 17, 107)     \
    X(61, TG_E5M2, 4, 5, 16, 1, 1, 17, 107)     \
    X(62, TG_E4M3, 4, 5, 16, 1, 1, 81, 90)      \
    X(63, TG_E5M2, 4, 5, 16, 1, 1, 81, 90)

// Explicit instantiation, seen by both the device and the host pass.
#define TG_INSTANTIATE_RS(id, DT, BM, BN, LC, MW, GM, SM, EFF) \
    template __global__ void tg::gemm_kernel<DT, BM, BN, LC, MW, SM>(GemmArgs);
#define TG_INSTANTIATE_STREAM(id, DT, BM, BN, WM, WN, S, GM, EFF) \
    template __global__ void tg::gemm_stream_kernel<DT, BM, BN, WM, WN, S, GM>(GemmArgs);
#define TG_INSTANTIATE_HYBRID(id, DT, S, P, GM, EFF) \
    template __global__ void tg::gemm_hybrid_kernel<DT, S, P>(GemmArgs);
TG_RS_LIST(TG_INSTANTIATE_RS)
TG_STREAM_LIST(TG_INSTANTIATE_STREAM)
TG_HYBRID_LIST(TG_INSTANTIATE_HYBRID)
#define TG_INSTANTIATE_WIDE(id, DT, GM, NS, RS, ADDR, SCHED, EPI, EFF) \
    template __global__ void tg::gemm_wide_kernel<DT, GM, NS, RS, ADDR, SCHED, EPI>(GemmArgs);
TG_WIDE_LIST(TG_INSTANTIATE_WIDE)

// The table holds host launch functions, so it exists only in the host pass.
#ifndef __HIP_DEVICE_COMPILE__
#define TG_ES(DT) ((DT) == TG_F32 ? 4 : ((DT) == TG_E4M3 || (DT) == TG_E5M2) ? 1 : 2)
#define TG_ENTRY_RS(id, DT, BM, BN, LC, MW, GM, SM, EFF)                                            \
    {id, DT, BM, BN, 128 / TG_ES(DT), 2, 2, (BM) / 2, (BN) / 2, 256, 2, 2 * ((BM) + (BN)) * 128,    \
     ((BM) / 2) * ((BN) / 2) / 64, LC, GM, EFF, &tg::launch<DT, BM, BN, LC, MW, SM>, 0, SM, 0,               \
     ((DT) == TG_E4M3 || (DT) == TG_E5M2) ? 1 : 0},
#define TG_ENTRY_STREAM(id, DT, BM, BN, WM, WN, S, GM, EFF)                                         \
    {id, DT, BM, BN, 64 / TG_ES(DT), WM, WN, (BM) / (WM), (BN) / (WN), 64 * (WM) * (WN), S,           \
     (S) * ((BM) + (BN)) * 64, ((BM) / (WM)) * ((BN) / (WN)) / 64, 16, GM, EFF,                    \
     &tg::launch_stream<DT, BM, BN, WM, WN, S, GM>},

#define TG_ENTRY_HYBRID(id, DT, S, P, GM, EFF)                                                      \
    {id, DT, 256, 256, 64 / TG_ES(DT), 2, 2, 128, 128, 256, S,                                      \
     ((S) * 256 * 64 > 512 * 64 ? (S) * 256 * 64 : 512 * 64), 256, 16, GM, EFF,                     \
     &tg::launch_hybrid<DT, S, P>},

#define TG_ENTRY_WIDE(id, DT, GM, NS, RS, ADDR, SCHED, EPI, EFF)                                    \
    {id, DT, 256, 256, 128 / TG_ES(DT), 2, 2, 128, 128, 256, NS, (NS) * 256 * 128, 256, 16, GM, EFF,   \
     &tg::launch_wide<DT, GM, NS, RS, ADDR, SCHED, EPI>, (ADDR) ? (int64_t(1) << 23) : 0, ((EPI) & 8) ? 1 : 0, \
     (EPI) & 1, ((EPI) & 64) ? 1 : 0},

static const TgKernelDesc kUnsorted[] = {TG_STREAM_LIST(TG_ENTRY_STREAM) TG_RS_LIST(TG_ENTRY_RS)
                                             TG_HYBRID_LIST(TG_ENTRY_HYBRID) TG_WIDE_LIST(TG_ENTRY_WIDE)};
constexpr int kCount = sizeof(kUnsorted) / sizeof(kUnsorted[0]);

// The table is indexed by kernel id.
struct TgTable {
    TgKernelDesc k[kCount];
    TgTable() {
        for (int i = 0; i < kCount; ++i) k[kUnsorted[i].id] = kUnsorted[i];
    }
};
static const TgTable kTable;
extern "C" const TgKernelDesc* const tg_kernel_table = kTable.k;
extern "C" const int tg_kernel_table_size = kCount;
#endif  // __HIP_DEVICE_COMPILE__
