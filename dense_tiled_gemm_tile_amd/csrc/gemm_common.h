// Device building blocks shared by every GEMM kernel of the library: operand
// loaders, the MFMA steps, the epilogue's output conversion and stores, the
// batch/split selection of a workgroup, the row-softmax epilogue, and the
// LDS-DMA copy primitives with their explicit wait counts.
//
// Common conventions (all operands K-contiguous, D M-contiguous):
//   A storage: BM rows of a tile are A rows m (stride lda bytes lda_b)
//   B storage: BN rows of a tile are B columns n (stride ldb bytes ldb_b)
//   MFMA "A" operand <- B rows (n), MFMA "B" operand <- A rows (m), so the
//   32 lanes of an MFMA output column group walk consecutive m: stores of one
//   accumulator register write 2 x 128 contiguous bytes of D (Tylo.jl manual,
//   "Walk through GEMM", section 5: store by accumulator ownership).
// LDS rows hold 128 (or 64) bytes of K with their 16-byte chunks in XOR-
// swizzled slots (tile_math.h), so fragment reads and stage writes of
// consecutive rows at one logical chunk never share a bank group.
#pragma once

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
// with k >= K becomes an exact zero and is not read.  Every load reads an
// element below K (the index is clamped to K - 1, the value then replaced by
// zero), so the loads carry no branches and go out back to back.  K >= 1.
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
                const unsigned x = r[min(k, K - 1)];
                v |= (k < K ? x : 0u) << (8 * e);
            }
            w[d] = v;
        }
    } else if constexpr (ES == 2) {
        const unsigned short* r = reinterpret_cast<const unsigned short*>(row);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int k = k0 + 2 * d;
            const unsigned lo = r[min(k, K - 1)], hi = r[min(k + 1, K - 1)];
            w[d] = (k < K ? lo : 0u) | ((k + 1 < K ? hi : 0u) << 16);
        }
    } else {
        const unsigned* r = reinterpret_cast<const unsigned*>(row);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int k = k0 + d;
            const unsigned x = r[min(k, K - 1)];
            w[d] = k < K ? x : 0u;
        }
    }
    u32x4 v;
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    return v;
}

// A chunk of 4-bit (e2m1) elements, two per byte with the low nibble first,
// that starts at element k0 (a multiple of 32) of a row and may run past K:
// elements with k >= K become exact zeros.  Every load reads a byte that
// holds an element below K (clamped, as above).  K >= 1.
__device__ __forceinline__ u32x4 load_chunk_bounded_e2m1(const char* row, int k0, int K) {
    const unsigned char* r = reinterpret_cast<const unsigned char*>(row);
    const int last = (K - 1) / 2;  // the last byte holding an element below K
    unsigned w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        unsigned v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + 8 * d + 2 * e;  // the byte's low element
            const unsigned x = r[min(k / 2, last)];
            v |= (k + 1 < K ? x : k < K ? (x & 0xFu) : 0u) << (8 * e);
        }
        w[d] = v;
    }
    u32x4 v;
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    return v;
}

// Sixteen bytes of a packed row from byte b0 on, of which only the first
// `nbits` bits of the row hold elements below K: every later bit becomes
// zero (a 6-bit element past K then decodes to +0).  Every load reads a byte
// that holds bits below nbits (clamped, as above).  nbits >= 1.
__device__ __forceinline__ u32x4 load_chunk_bounded_bits(const char* row, int64_t b0, int64_t nbits) {
    const unsigned char* r = reinterpret_cast<const unsigned char*>(row);
    const int64_t last = (nbits - 1) / 8;
    unsigned w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        unsigned v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t b = b0 + 4 * d + e;
            const int64_t left = nbits - 8 * b;  // bits of this byte below K
            const unsigned x = r[b < last ? b : last];
            v |= (left >= 8 ? x : left > 0 ? (x & ((1u << left) - 1u)) : 0u) << (8 * e);
        }
        w[d] = v;
    }
    u32x4 v;
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    return v;
}

// ---------------------------------------------------------------- MFMA step

typedef int i32x8 __attribute__((ext_vector_type(8)));

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 6-bit (e2m3, FMT 2; e3m2, FMT 3) operands: one 32x32x64 MFMA per 24-byte
// fragment, given as three 8-byte pieces in order.  Lane l supplies row
// l & 31; half-wave h = l >> 5 supplies k [32h, 32h + 32) of the 64, element i
// in bits [6i, 6i + 6) of the 24 bytes, for both operands alike, and the
// block-scale exponent of its row's k-block h (low byte of sn / sm).
template <int FMT>
__device__ __forceinline__ f32x16 mfma_f6(const u32x2 (&n)[3], const u32x2 (&m)[3], f32x16 acc, int sn, int sm) {
    const i32x8 a = {static_cast<int>(n[0].x), static_cast<int>(n[0].y), static_cast<int>(n[1].x),
                     static_cast<int>(n[1].y), static_cast<int>(n[2].x), static_cast<int>(n[2].y), 0, 0};
    const i32x8 b = {static_cast<int>(m[0].x), static_cast<int>(m[0].y), static_cast<int>(m[1].x),
                     static_cast<int>(m[1].y), static_cast<int>(m[2].x), static_cast<int>(m[2].y), 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, FMT, FMT, 0, sn, 0, sm);
}

// 4-bit (e2m1) operands: one 32x32x64 MFMA per 16-byte fragment.  Lane l
// supplies row l & 31; half-wave h = l >> 5 supplies k [32h, 32h + 32) of the
// 64, element i of the fragment in bits [4i, 4i + 4), for both operands alike
// (so a fragment is one 16-byte chunk of the row), and the block-scale
// exponent of its row's k-block h: byte SEL of sn for the n side and of sm
// for the m side (127 means a scale of 1).
template <int SEL = 0>
__device__ __forceinline__ f32x16 mfma_f4(u32x4 n, u32x4 m, f32x16 acc, int sn, int sm) {
    const i32x8 a = {static_cast<int>(n.x), static_cast<int>(n.y), static_cast<int>(n.z), static_cast<int>(n.w),
                     0, 0, 0, 0};
    const i32x8 b = {static_cast<int>(m.x), static_cast<int>(m.y), static_cast<int>(m.z), static_cast<int>(m.w),
                     0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 4, 4, SEL, sn, SEL, sm);
}

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
    } else if constexpr (DT == TG_E2M1) {
        return mfma_f4(nfrag, mfrag, acc, 127, 127);
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
    // A batch (or split-K) of an even number of matrices from six on may run
    // on a grid of matrices (x) by tiles (y): workgroups go to the XCDs
    // round-robin in x-major order, so matrix b's tiles land on 8 / gcd(count,
    // 8) XCDs (for a multiple of kXcdCount, matrix b runs whole on XCD b mod 8
    // and no operand byte is fetched into more than one XCD's L2); the tiles
    // of a matrix follow the grouped walk.
    int64_t b;
    if (p.xcd_batches) {
        b = blockIdx.x;
        p.tile = blockIdx.y;
    } else {
        b = blockIdx.y;
        p.tile = xcd_order(blockIdx.x, gridDim.x);
    }
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

// ---------------------------------------------------------------- LDS-DMA copies and waits

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

}  // namespace tg
