// Auxiliary kernels of the library: the split-K reduction (fp32 partial
// products added in split order, then the epilogue), the staged operand copy
// (misaligned rows into 16-byte aligned, zero-padded rows) and the row
// softmax over n of an fp32 D (the second pass when one tile cannot span N).
#include <atomic>
#include <mutex>

#include "gemm_common.h"

namespace tg {

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
    // partials of split s at src + s * plane, added in split order; the loads
    // of eight splits go out together (one round trip each batch, not one per
    // split), the additions keep their order, so the sum has the same bits
    constexpr int BATCH = 8;
    auto load4 = [&](int s) {
        f32x4 q = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* x = src + s * plane;
        if ((M & 3) == 0) {
            q = *reinterpret_cast<const f32x4*>(x);  // whole 16-byte groups (16-byte aligned base)
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < cnt) q[e] = x[e];
        }
        return q;
    };
    auto add4 = [&](const f32x4& q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += q[e];
    };
    int s = 0;
    for (; s + BATCH <= splits; s += BATCH) {
        f32x4 q[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) q[u] = load4(s + u);
#pragma unroll
        for (int u = 0; u < BATCH; ++u) add4(q[u]);
    }
    for (; s < splits; ++s) add4(load4(s));
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

// ---------------------------------------------------------------- static scratch
//
// Device memory the library itself holds, for callers that cannot allocate
// (tile_gemm_splitk_noalloc keeps its fp32 partial products here): one array
// per GPU, loaded with the library's code object and kept until the process
// ends.  In host code the array's name is only a stand-in for the device
// symbol, never a device address, so the address is looked up once per
// device (with that device current) and only that address reaches kernels.
// Every call on a GPU shares its array: calls that overlap on one GPU race.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kTgStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t tg_static_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}
