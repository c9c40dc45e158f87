// C ABI of the tiled GEMM library: argument validation, the host plan chooser
// and the launch.
//
// The plan is chosen on the host from the problem and the operands' alignment
// (Tylo.jl manual, "Walk through GEMM", section 1: the configuration runs on
// the host and picks a compiled kernel, while problem sizes and leading
// strides stay runtime kernel arguments).  The 16-byte vector staging needs
// every operand row start to be at least 4-byte aligned; the caller's pointers
// and strides decide the class, and 2-byte aligned rows take the shifting
// loader (section 3: the caller establishes pointer alignment; the plan must
// respect it).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "kernel_table.h"
#include "tile_math.h"
#include "tile_gemm.h"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxGrid = int64_t(1) << 24;
constexpr int64_t kMaxBatch = 65535;              // grid y
constexpr int64_t kMaxBatchStride = int64_t(1) << 40;
constexpr int kMaxSplits = 256;
constexpr int kAutoSplitMax = 64;

// Matrices of a batched call: batch >= 1, element distances between
// consecutive A, B and D matrices (0 = the same matrix for every entry).
struct Batch {
    int64_t batch = 1, stride_a = 0, stride_b = 0, stride_d = 0;
};
constexpr int kCusPerGpu = 256;
constexpr int64_t kMaxGridY = 65535;  // largest grid y dimension

// Whether `count` matrices (a batch, or the splits of a split-K) of `tiles`
// tiles each run on a grid of matrices by tiles (select_batch): matrix b's
// tiles then go to 8 / gcd(count, 8) of the XCDs (one for a multiple of
// eight), so fewer L2s fetch its operands.  For an even count from six on,
// when the tiles fit the grid's y dimension (one box, same bits: 12 x
// 512x512x2048 22.4 against 28.1 us, 20 x 256x256x4096 32.7 against 53.9,
// 12 x 1024^3 32.5 against 35.5, 6 x 1024^3 25.9 against 26.9; 2 and 4
// products of 1024^3 or 2048^3 neither gained nor lost).
int whole_matrices_per_xcd(int64_t count, int64_t tiles) {
    return (count >= 6 && count % 2 == 0 && tiles <= kMaxGridY) ? 1 : 0;
}

// Time model of the staging decision: seconds per unit of plan_cost per K
// stage (fitted to the 256x256 streaming kernel on an 8192^3 bf16 product),
// the HBM rate of the staging copy (measured: 286 MB read and written for
// 12289x5003x4099 bf16 in 54 us), and the cost of one more launch.
constexpr double kSecondsPerCostStage = 2.5e-11;
constexpr double kCopyBytesPerSecond = 5.0e12;
constexpr double kLaunchSeconds = 6e-6;

// Bits per element of an operand or output type (0: unknown).
int elem_bits(int dtype) {
    switch (dtype) {
        case TG_E2M1: return 4;
        case TG_E2M3:
        case TG_E3M2: return 6;
        case TG_E4M3:
        case TG_E5M2: return 8;
        case TG_BF16:
        case TG_F16: return 16;
        case TG_F32: return 32;
        default: return 0;
    }
}

// Bytes of an element type (1 for the packed 4-bit format: its pointers need
// byte alignment only).
int elem_size(int dtype) {
    const int b = elem_bits(dtype);
    return b >= 8 ? b / 8 : (b ? 1 : 0);
}

// Bytes spanned by `elems` consecutive elements (rounded up for packed types).
int64_t bytes_of(int64_t elems, int dtype) { return (elems * elem_bits(dtype) + 7) / 8; }

// Types D may have.
bool out_type_ok(int dtype) { return dtype == TG_F32 || dtype == TG_BF16 || dtype == TG_F16; }

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

int validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
             int64_t ldb, const void* D, int64_t ldd, int dtype, int out_dtype, const Batch& bt) {
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return TG_ERR_DIMS;
    if (bt.batch < 0 || bt.batch > kMaxBatch) return TG_ERR_DIMS;
    const int es = elem_size(dtype);
    const int os = out_type_ok(out_dtype) ? elem_size(out_dtype) : 0;
    if (!es || !os) return TG_ERR_DTYPE;
    const int64_t kmin = K > 1 ? K : 1;
    if (lda < kmin || ldb < kmin || ldd < (M > 1 ? M : 1)) return TG_ERR_LD;
    if (bt.stride_a < 0 || bt.stride_b < 0 || bt.stride_d < 0 || bt.stride_a > kMaxBatchStride ||
        bt.stride_b > kMaxBatchStride || bt.stride_d > kMaxBatchStride)
        return TG_ERR_LD;
    // packed types: every operand row (and matrix) starts on a byte
    const int eb = elem_bits(dtype);
    if (eb < 8 && (((lda * eb) | (ldb * eb) | (bt.stride_a * eb) | (bt.stride_b * eb)) & 7)) return TG_ERR_LD;
    if (M == 0 || N == 0 || bt.batch == 0) return TG_OK;
    // the output matrices of a batch must not overlap one another
    if (bt.batch > 1 && bt.stride_d < (N - 1) * ldd + M) return TG_ERR_LD;
    const bool reads = K > 0;
    if (!D || (reads && (!A || !B))) return TG_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(D) & uintptr_t(os - 1)) ||
        (reads && ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & uintptr_t(es - 1))))
        return TG_ERR_ALIGN;
    if (reads) {
        // whole spans of the batch (conservative for interleaved layouts)
        const int64_t last = bt.batch - 1;
        const uintptr_t d0 = reinterpret_cast<uintptr_t>(D);
        const uintptr_t d1 = d0 + uintptr_t(last * bt.stride_d + (N - 1) * ldd + M) * uintptr_t(os);
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(A);
        const uintptr_t a1 = a0 + uintptr_t(bytes_of(last * bt.stride_a + (M - 1) * lda + K, dtype));
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(B);
        const uintptr_t b1 = b0 + uintptr_t(bytes_of(last * bt.stride_b + (N - 1) * ldb + K, dtype));
        if (overlaps(d0, d1, a0, a1) || overlaps(d0, d1, b0, b1)) return TG_ERR_ALIAS;
    }
    return TG_OK;
}

// Byte alignment class shared by every operand row start (of every matrix of
// a batch): 16, 4, 2 or (8- and 4-bit operands) 1.
int row_class(int64_t M, int64_t N, const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
              const Batch& bt) {
    uintptr_t bits = reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B);
    if (M > 1) bits |= uintptr_t(bytes_of(lda, dtype));
    if (N > 1) bits |= uintptr_t(bytes_of(ldb, dtype));
    if (bt.batch > 1) bits |= uintptr_t(bytes_of(bt.stride_a, dtype)) | uintptr_t(bytes_of(bt.stride_b, dtype));
    if ((bits & 15u) == 0) return 16;
    if ((bits & 3u) == 0) return 4;
    if ((bits & 1u) == 0) return 2;
    return 1;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Relative cost of a plan: each CU works through ceil(tiles / CUs) tiles one
// after another (co-resident workgroups share the CU's MFMA pipes), each tile
// costing its area divided by the instance's expected MFMA efficiency.
double plan_cost(const TgKernelDesc& k, int64_t M, int64_t N, int64_t batch) {
    const int64_t tiles = cdiv(M, k.block_m) * cdiv(N, k.block_n) * (batch > 1 ? batch : 1);
    return double(cdiv(tiles, kCusPerGpu)) * double(k.block_m) * double(k.block_n) / (0.01 * k.eff_pct);
}

bool usable(const TgKernelDesc& k, int dtype, int cls, int64_t row_stride) {
    return k.dtype == dtype && cls >= k.load_class && (k.max_row_stride == 0 || row_stride <= k.max_row_stride);
}

// Whether every D column (and every D matrix of a batch) starts on a
// 128-byte line, so that a tile's column pieces are whole lines.
bool d_lines_aligned(const void* D, int64_t ldd, int os, const Batch& bt) {
    uintptr_t bits = reinterpret_cast<uintptr_t>(D) | uintptr_t(ldd * os);
    if (bt.batch > 1) bits |= uintptr_t(bt.stride_d * os);
    return (bits & 127u) == 0;
}

// d_lines: D columns start on 128-byte lines.  When they do not, the tiles'
// column pieces end in partial lines that a neighbouring tile completes
// later, and nontemporal stores of them measure about 20 % slower on the whole
// product than ordinary ones; such instances are then weighed down.
// Instances whose every wave holds the whole tile and a share of K (the
// K-sliced kernel) only pay when most CUs would otherwise idle (at most half
// as many tiles as CUs; measured: 512x512x16384 41 us against 64 us,
// 1024x1024x4096 a tie, 1024^3 slower).
// Instances marked power_bound (the 16x16x32 wide kernel) need K loops of at
// least 16 stages: their MFMAs cost less energy, which pays when the power
// limit sets the clock, and since their loop issues its copies in groups
// and knows its ring slots at compile time it also matches the 32x32x16
// kernel at a given clock (one box: 8192x8192x1024 904 against 899
// TFLOP/s, 4096x4096x1024 958-965 against 886-898, 3072^3 on 144 CUs
// 986-1014 against 946-990, 6144x6144x1536 973 against 932); below 16
// stages the two trade places (8192x8192x512 604-606 against 630,
// 4096x4096x512 651-653 against 629-647) and the 32x32x16 kernel stays.
constexpr int kPowerBoundStages = 16;
int choose(int64_t M, int64_t N, int64_t batch, int64_t K, int dtype, int cls, int64_t row_stride,
           bool d_lines = true) {
    int best = -1;
    double best_cost = 0;
    for (int i = 0; i < tg_kernel_count(); ++i) {
        const TgKernelDesc& k = tg_kernel(i);
        if (!usable(k, dtype, cls, row_stride)) continue;
        if (k.power_bound && cdiv(K, k.block_k) < kPowerBoundStages) continue;
        if (k.k_slices > 1 && k.waves_m * k.waves_n == 1 &&
            cdiv(M, k.block_m) * cdiv(N, k.block_n) * batch > kCusPerGpu / 2)
            continue;
        // among equal costs prefer the instance that needs the strongest alignment
        double c = plan_cost(k, M, N, batch) * (1.0 + 0.001 / k.load_class);
        if (k.nt_store && !d_lines) c *= 1.25;
        if (best < 0 || c < best_cost) { best = i; best_cost = c; }
    }
    return best;
}

void describe(const TgKernelDesc& k, int64_t M, int64_t N, tile_gemm_plan_info* out) {
    memset(out, 0, sizeof *out);
    out->kernel_id = k.id;
    out->dtype = k.dtype;
    out->block_m = k.block_m;
    out->block_n = k.block_n;
    out->block_k = k.block_k;
    out->waves_m = k.waves_m;
    out->waves_n = k.waves_n;
    out->wave_tile_m = k.wave_tile_m;
    out->wave_tile_n = k.wave_tile_n;
    out->threads = k.threads;
    out->stages = k.stages;
    out->lds_bytes = k.lds_bytes;
    out->acc_per_lane = k.acc_per_lane;
    out->load_class = k.load_class;
    out->group_m = k.group_m;
    out->k_slices = k.k_slices > 0 ? k.k_slices : 1;
    out->block_scales = k.block_scales;
    if (M > 0 && N > 0) {
        out->tiles_m = cdiv(M, k.block_m);
        out->tiles_n = cdiv(N, k.block_n);
        out->grid = out->tiles_m * out->tiles_n;
    }
}

// Staged operands: A and B copied into rows of staged_row_bytes (a whole
// number of 128-byte K stages, zeros past K) that start 16-byte aligned.
int64_t staged_row_bytes(int64_t K, int es) { return cdiv(K * es, 128) * 128; }

int64_t staged_b_offset(int64_t M, int64_t K, int es) { return cdiv(M * staged_row_bytes(K, es), 256) * 256; }

int64_t staged_bytes(int64_t M, int64_t N, int64_t K, int es) {
    return staged_b_offset(M, K, es) + N * staged_row_bytes(K, es);
}

double plan_seconds(const TgKernelDesc& k, int64_t M, int64_t N, int64_t K) {
    return kSecondsPerCostStage * plan_cost(k, M, N, 1) * double(cdiv(K, k.block_k));
}

struct Staging {
    bool on = false;
    int staged_id = -1;     // instance for the staged operands
    int64_t row_bytes = 0;  // bytes per staged row
};

// Whether a single product runs on staged copies of its operands (mode 1:
// always; -1: when the operand rows are not all 16-byte aligned and the
// staged plan plus the copy is expected to beat the direct plan).  The copy
// costs one read and one write of both operands at HBM speed and a launch.
Staging decide_staging(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda, const void* B,
                       int64_t ldb, bool d_lines, int mode) {
    Staging st;
    if (mode == 0 || M == 0 || N == 0 || K == 0 || elem_bits(dtype) < 8) return st;
    const int es = elem_size(dtype);
    const int64_t rb = staged_row_bytes(K, es);
    if (rb / es > kMaxDim) return st;
    const int sid = choose(M, N, 1, rb / es, dtype, 16, rb, d_lines);
    if (sid < 0) return st;
    if (mode != 1) {
        const int cls = row_class(M, N, A, lda, B, ldb, dtype, Batch());
        if (cls == 16) return st;
        const int did = choose(M, N, 1, K, dtype, cls, (lda > ldb ? lda : ldb) * es, d_lines);
        if (did >= 0) {
            const double copy = double((M + N) * (K * es + rb)) / kCopyBytesPerSecond + kLaunchSeconds;
            const double staged = plan_seconds(tg_kernel(sid), M, N, rb / es) + copy;
            if (staged >= plan_seconds(tg_kernel(did), M, N, K)) return st;
        }
    }
    st.on = true;
    st.staged_id = sid;
    st.row_bytes = rb;
    return st;
}

// The plan of a direct launch on the operands as given (no staging).
int plan(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda, const void* B,
         int64_t ldb, const void* D, int64_t ldd, int out_dtype, int kernel_id, tile_gemm_plan_info* out,
         const Batch& bt = Batch(), int64_t splits = 1) {
    const int rc = validate(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, bt);
    if (rc) return rc;
    const int cls = row_class(M, N, A, lda, B, ldb, dtype, bt);
    const int64_t row_stride = bytes_of(lda > ldb ? lda : ldb, dtype);
    const bool d_lines = d_lines_aligned(D, ldd, elem_size(out_dtype), bt);
    int id = kernel_id;
    if (id < 0) {
        id = choose(M, N, bt.batch * splits, cdiv(K, splits), dtype, cls, row_stride, d_lines);
        if (id < 0) return TG_ERR_PLAN;
    } else if (id >= tg_kernel_count() || !usable(tg_kernel(id), dtype, cls, row_stride)) {
        return TG_ERR_PLAN;
    }
    describe(tg_kernel(id), M, N, out);
    out->load_class = cls;
    if (out->grid > kMaxGrid) return TG_ERR_DIMS;
    return TG_OK;
}

// gfx950 check, cached per device (0 unknown, 1 yes, 2 no).
std::atomic<int> g_arch_ok[64];

int device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return TG_ERR_DEVICE;
    }
    if (dev < 64) {
        int v = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (v == 1) return TG_OK;
        if (v == 2) return TG_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return TG_ERR_DEVICE;
    }
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? TG_OK : TG_ERR_DEVICE;
}

// Block scales of 8-bit operands (none when both pointers are null).
struct Scales {
    const unsigned char* a = nullptr;
    const unsigned char* b = nullptr;
    int64_t lds_a = 0, lds_b = 0;
};

int launch_batched(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
                   int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b, void* D, int64_t ldd,
                   int64_t stride_d, int64_t batch, int dtype, int out_dtype, void* stream, int kernel_id,
                   const Scales& sc = Scales());

// Whether tile_gemm_staged copies the operands (mode 1: always; -1: when the
// plan says the copy pays and the workspace suffices; 0: never).  *rc gets
// TG_ERR_WORKSPACE (mode 1 without a usable workspace) or TG_ERR_ALIAS (the
// workspace overlaps an operand).
Staging staged_decision(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                        const void* D, int64_t ldd, int dtype, int out_dtype, const void* workspace,
                        int64_t workspace_bytes, int mode, int* rc) {
    *rc = TG_OK;
    if (mode == 1 && elem_bits(dtype) < 8 && M > 0 && N > 0 && K > 0) {
        *rc = TG_ERR_DTYPE;  // packed operands are never staged
        return Staging();
    }
    Staging st = decide_staging(M, N, K, dtype, A, lda, B, ldb, d_lines_aligned(D, ldd, elem_size(out_dtype), Batch()),
                                mode);
    if (!st.on) return st;
    const int es = elem_size(dtype);
    const int64_t need = staged_bytes(M, N, K, es);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)) {
        if (mode == 1) *rc = TG_ERR_WORKSPACE;
        st.on = false;
        return st;
    }
    const int os = elem_size(out_dtype);
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + uintptr_t(need);
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(D), d1 = d0 + uintptr_t((N - 1) * ldd + M) * uintptr_t(os);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(A), a1 = a0 + uintptr_t((M - 1) * lda + K) * uintptr_t(es);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(B), b1 = b0 + uintptr_t((N - 1) * ldb + K) * uintptr_t(es);
    if (overlaps(w0, w1, d0, d1) || overlaps(w0, w1, a0, a1) || overlaps(w0, w1, b0, b1)) {
        *rc = TG_ERR_ALIAS;
        st.on = false;
    }
    return st;
}

// A single product on staged operand copies in the caller's workspace, when
// `mode` and the plan say so; otherwise the direct plan.
int gemm_staged(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda, const void* B,
                int64_t ldb, void* D, int64_t ldd, int dtype, int out_dtype, void* stream, void* workspace,
                int64_t workspace_bytes, int mode) {
    int rc = validate(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, Batch());
    if (rc) return rc;
    const Staging st = staged_decision(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, workspace,
                                       workspace_bytes, mode, &rc);
    if (rc) return rc;
    if (!st.on)
        return launch_batched(M, N, K, alpha, relu, A, lda, 0, B, ldb, 0, D, ldd, 0, 1, dtype, out_dtype, stream,
                              -1);
    rc = device_ok();
    if (rc) return rc;
    const int es = elem_size(dtype);
    char* sa = static_cast<char*>(workspace);
    char* sb = sa + staged_b_offset(M, K, es);
    const hipError_t err = tg_stage_operands(static_cast<const char*>(A), lda * es, M, static_cast<const char*>(B),
                                             ldb * es, N, static_cast<int>(K), es, st.row_bytes, sa, sb,
                                             static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return TG_ERR_LAUNCH;
    const int64_t kp = st.row_bytes / es;  // the padding holds exact zeros
    return launch_batched(M, N, kp, alpha, relu, sa, kp, 0, sb, kp, 0, D, ldd, 0, 1, dtype, out_dtype, stream,
                          st.staged_id);
}

// The fused softmax instance for a tile_gemm_softmax call (*id = -1: two
// launches, the plain product and the row pass).
int softmax_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                 const void* D, int64_t ldd, int dtype, int out_dtype, int kernel_id, int* id) {
    *id = -1;
    const int rc = validate(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, Batch());
    if (rc) return rc;
    if (M == 0 || N == 0) return TG_OK;
    const int cls = row_class(M, N, A, lda, B, ldb, dtype, Batch());
    const int64_t row_stride = bytes_of(lda > ldb ? lda : ldb, dtype);
    // fused: an instance whose tile spans all of N
    if (kernel_id >= 0) {
        if (kernel_id >= tg_kernel_count()) return TG_ERR_PLAN;
        const TgKernelDesc& k = tg_kernel(kernel_id);
        if (!usable(k, dtype, cls, row_stride) || !k.softmax || k.block_n < N) return TG_ERR_PLAN;
        *id = kernel_id;
    } else {
        double best = 0;
        for (int i = 0; i < tg_kernel_count(); ++i) {
            const TgKernelDesc& k = tg_kernel(i);
            if (!usable(k, dtype, cls, row_stride) || !k.softmax || k.block_n < N) continue;
            const double c = plan_cost(k, M, N, 1) * (1.0 + 0.001 / k.load_class);
            if (*id < 0 || c < best) { *id = i; best = c; }
        }
    }
    if (*id < 0 && out_dtype != TG_F32) return TG_ERR_DIMS;  // the two-pass path writes fp32 logits
    if (*id >= 0 && cdiv(M, tg_kernel(*id).block_m) > kMaxGrid) return TG_ERR_DIMS;
    return TG_OK;
}

// Validation of a tile_gemm_scaled call and its instance: with block scales
// only instances that apply them may run it (*kernel_id -1 = the cheapest such
// instance); without scales the call is tile_gemm_out's.
int scaled_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* scale_a, int64_t lds_a,
                const void* B, int64_t ldb, const void* scale_b, int64_t lds_b, const void* D, int64_t ldd, int dtype,
                int out_dtype, int* kernel_id, Scales* sc) {
    const int rc = validate(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, Batch());
    if (rc) return rc;
    if (!scale_a && !scale_b) return TG_OK;
    if (elem_bits(dtype) > 8) return TG_ERR_DTYPE;
    // 8- and 6-bit: whole dwords per 128-k stage, 4*ceil(K/128) bytes per
    // row, 4-byte aligned; 4-bit: whole 16-byte pieces per two 256-k stages,
    // 16*ceil(K/512) bytes per row, 16-byte aligned
    const bool f4 = elem_bits(dtype) == 4;
    const int64_t unit = f4 ? 16 : 4;
    const int64_t need = unit * cdiv(K, f4 ? 512 : 128);
    if ((scale_a && (lds_a < need || (lds_a % unit))) || (scale_b && (lds_b < need || (lds_b % unit))))
        return TG_ERR_LD;
    if ((reinterpret_cast<uintptr_t>(scale_a) | reinterpret_cast<uintptr_t>(scale_b)) & uintptr_t(unit - 1))
        return TG_ERR_ALIGN;
    if (M > 0 && N > 0 && K > 0) {
        const uintptr_t d0 = reinterpret_cast<uintptr_t>(D);
        const uintptr_t d1 = d0 + uintptr_t((N - 1) * ldd + M) * uintptr_t(elem_size(out_dtype));
        if (scale_a) {
            const uintptr_t s0 = reinterpret_cast<uintptr_t>(scale_a), s1 = s0 + uintptr_t((M - 1) * lds_a + need);
            if (overlaps(d0, d1, s0, s1)) return TG_ERR_ALIAS;
        }
        if (scale_b) {
            const uintptr_t s0 = reinterpret_cast<uintptr_t>(scale_b), s1 = s0 + uintptr_t((N - 1) * lds_b + need);
            if (overlaps(d0, d1, s0, s1)) return TG_ERR_ALIAS;
        }
    }
    sc->a = static_cast<const unsigned char*>(scale_a);
    sc->b = static_cast<const unsigned char*>(scale_b);
    sc->lds_a = lds_a;
    sc->lds_b = lds_b;
    // instances with 32-bit row offsets also address 256 rows of scales that way
    auto scale_rows_fit = [&](const TgKernelDesc& k) {
        return !k.max_row_stride || !((scale_a && lds_a > k.max_row_stride) || (scale_b && lds_b > k.max_row_stride));
    };
    if (*kernel_id >= 0) {
        if (*kernel_id >= tg_kernel_count() || !tg_kernel(*kernel_id).block_scales) return TG_ERR_PLAN;
        return scale_rows_fit(tg_kernel(*kernel_id)) ? TG_OK : TG_ERR_PLAN;
    }
    const int cls = row_class(M, N, A, lda, B, ldb, dtype, Batch());
    const int64_t row_stride = bytes_of(lda > ldb ? lda : ldb, dtype);
    const bool d_lines = d_lines_aligned(D, ldd, elem_size(out_dtype), Batch());
    double best = 0;
    for (int i = 0; i < tg_kernel_count(); ++i) {
        const TgKernelDesc& k = tg_kernel(i);
        if (!k.block_scales || !usable(k, dtype, cls, row_stride) || !scale_rows_fit(k)) continue;
        double cost = plan_cost(k, M, N, 1) * (1.0 + 0.001 / k.load_class);
        if (k.nt_store && !d_lines) cost *= 1.25;
        if (*kernel_id < 0 || cost < best) { *kernel_id = i; best = cost; }
    }
    return *kernel_id < 0 ? TG_ERR_PLAN : TG_OK;
}

}  // namespace

extern "C" {

int tile_gemm_query_plan(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                         const void* B, int64_t ldb, const float* D, int64_t ldd, tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    return plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, TG_F32, -1, out);
}

int tile_gemm_query_plan_batched(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                                 int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b,
                                 const void* D, int64_t ldd, int64_t stride_d, int64_t batch, int out_dtype,
                                 int kernel_id, tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    Batch bt;
    bt.batch = batch;
    bt.stride_a = stride_a;
    bt.stride_b = stride_b;
    bt.stride_d = stride_d;
    const int rc = plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id, out, bt);
    if (rc == TG_OK) out->grid *= (batch > 0 ? batch : 0);
    return rc;
}

int tile_gemm_query_plan_out(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                             const void* B, int64_t ldb, const void* D, int64_t ldd, int out_dtype,
                             int kernel_id, tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    return plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id, out);
}

int tile_gemm_batched(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A,
                      int64_t lda, int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b,
                      void* D, int64_t ldd, int64_t stride_d, int64_t batch, int dtype, int out_dtype,
                      void* stream, int kernel_id) {
    return launch_batched(M, N, K, alpha, relu, A, lda, stride_a, B, ldb, stride_b, D, ldd, stride_d, batch, dtype,
                          out_dtype, stream, kernel_id);
}

}  // extern "C"

namespace {

int launch_batched(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
                   int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b, void* D, int64_t ldd,
                   int64_t stride_d, int64_t batch, int dtype, int out_dtype, void* stream, int kernel_id,
                   const Scales& sc) {
    Batch bt;
    bt.batch = batch;
    bt.stride_a = stride_a;
    bt.stride_b = stride_b;
    bt.stride_d = stride_d;
    tile_gemm_plan_info pl;
    int rc = plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id, &pl, bt);
    if (rc) return rc;
    if (M == 0 || N == 0 || batch == 0) return TG_OK;
    rc = device_ok();
    if (rc) return rc;
    GemmArgs a{};  // every field starts at zero (split_k = 0: no split)
    a.A = static_cast<const char*>(A);
    a.B = static_cast<const char*>(B);
    a.D = D;
    a.lda_b = bytes_of(lda, dtype);
    a.ldb_b = bytes_of(ldb, dtype);
    a.ldd = ldd;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.alpha = alpha;
    a.relu = relu ? 1 : 0;
    a.tiles_m = static_cast<int>(pl.tiles_m);
    a.tiles_n = static_cast<int>(pl.tiles_n);
    a.group_m = pl.group_m;
    a.out_dtype = out_dtype;
    a.batch_a_b = bytes_of(stride_a, dtype);
    a.batch_b_b = bytes_of(stride_b, dtype);
    a.batch_d_b = stride_d * elem_size(out_dtype);
    a.scale_a = sc.a;
    a.scale_b = sc.b;
    a.lds_a = sc.lds_a;
    a.lds_b = sc.lds_b;
    // an even number of products from six on runs on a grid of products (x)
    // by tiles (y); with a multiple of eight each product is whole on one XCD
    // (one box: 32 x 256x256x4096 40.6 against 76.9 us, 24 x 1024x1024x2048
    // 98-99 against 112-113, 16 x 1024^3 39-40 against 44-45; the same bits)
    a.xcd_batches = whole_matrices_per_xcd(batch, pl.grid);
    const hipError_t err =
        a.xcd_batches ? tg_kernel(pl.kernel_id).launch(a, batch, static_cast<int>(pl.grid), static_cast<hipStream_t>(stream))
                      : tg_kernel(pl.kernel_id).launch(a, pl.grid, static_cast<int>(batch), static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int64_t tile_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int splits) {
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim || splits < 0 || splits > kMaxSplits) return -1;
    if (splits == 0) splits = kAutoSplitMax;
    if (splits <= 1 || M == 0 || N == 0) return 0;
    return int64_t(splits) * M * N * 4;
}

}  // extern "C"

namespace {

// Split-K product; `use_static` puts the partials in the library's static
// scratch array instead of `workspace` (whose checks then do not apply).
int splitk_impl(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda, const void* B,
                int64_t ldb, void* D, int64_t ldd, int dtype, int out_dtype, int splits, void* workspace,
                int64_t workspace_bytes, void* stream, int kernel_id, bool use_static) {
    if (use_static) workspace_bytes = kTgStaticScratchBytes;
    if (splits < 0 || splits > kMaxSplits) return TG_ERR_DIMS;
    if (splits == 0) {
        // automatic: split only when the output has fewer tiles than the chip
        // has CUs and every split keeps at least 16 stages of K; about 32
        // stages of K a split, but at least enough splits to give every CU a
        // workgroup (the best measured count, within a few percent, for 256^2
        // to 1024x512 outputs with K of 8192 to 32768)
        tile_gemm_plan_info p1;
        const int rc = plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id, &p1);
        if (rc) return rc;
        const int64_t tiles = p1.tiles_m * p1.tiles_n, stages = p1.block_k ? K / p1.block_k : 0;
        int64_t s = 1;
        if (tiles > 0 && tiles < kCusPerGpu && stages >= 64) {
            s = stages / 32;
            const int64_t fill = cdiv(kCusPerGpu, tiles);
            if (s < fill) s = fill;
            if (s > stages / 16) s = stages / 16;
            if (s > kAutoSplitMax) s = kAutoSplitMax;
            // never more than the workspace holds
            const int64_t fit = (M > 0 && N > 0 && (workspace || use_static)) ? workspace_bytes / (M * N * 4) : 0;
            if (s > fit) s = fit;
            // a multiple of the XCD count, so that every split runs whole on one XCD
            if (s >= tg::kXcdCount) s -= s % tg::kXcdCount;
        }
        splits = static_cast<int>(s < 1 ? 1 : s);
    }
    if (splits == 1)
        return launch_batched(M, N, K, alpha, relu, A, lda, 0, B, ldb, 0, D, ldd, 0, 1, dtype, out_dtype, stream,
                              kernel_id);
    // the first launch is a batch of `splits` products over K ranges; the
    // plan weighs all their workgroups
    tile_gemm_plan_info pl;
    int rc = plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id, &pl, Batch(), splits);
    if (rc) return rc;
    if (M == 0 || N == 0) return TG_OK;
    const int64_t bk = pl.block_k;
    const int64_t stages = cdiv(K, bk);
    const int64_t chunk = cdiv(stages, splits) * bk;         // K elements per split, whole stages
    const int64_t used = K > 0 ? cdiv(K, chunk) : 1;        // splits that get at least one element
    const int64_t need = used * M * N * 4;
    if (use_static) {
        if (need > kTgStaticScratchBytes) return TG_ERR_WORKSPACE;
    } else {
        if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15u))
            return TG_ERR_WORKSPACE;
        const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + uintptr_t(need);
        const int os = elem_size(out_dtype);
        const uintptr_t d0 = reinterpret_cast<uintptr_t>(D), d1 = d0 + uintptr_t((N - 1) * ldd + M) * uintptr_t(os);
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(A), a1 = a0 + uintptr_t(bytes_of((M - 1) * lda + K, dtype));
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(B), b1 = b0 + uintptr_t(bytes_of((N - 1) * ldb + K, dtype));
        if (overlaps(w0, w1, d0, d1) || (K > 0 && (overlaps(w0, w1, a0, a1) || overlaps(w0, w1, b0, b1))))
            return TG_ERR_ALIAS;
    }
    rc = device_ok();
    if (rc) return rc;
    if (use_static && tg_static_scratch(&workspace) != hipSuccess) {
        (void)hipGetLastError();
        return TG_ERR_LAUNCH;
    }
    GemmArgs a{};  // every field starts at zero (split_k = 0: no split)
    a.A = static_cast<const char*>(A);
    a.B = static_cast<const char*>(B);
    a.D = workspace;
    a.lda_b = bytes_of(lda, dtype);
    a.ldb_b = bytes_of(ldb, dtype);
    a.ldd = M;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.alpha = 1.0f;
    a.relu = 0;
    a.tiles_m = static_cast<int>(pl.tiles_m);
    a.tiles_n = static_cast<int>(pl.tiles_n);
    a.group_m = pl.group_m;
    a.out_dtype = TG_F32;
    a.batch_a_b = bytes_of(chunk, dtype);  // whole stages: whole bytes
    a.batch_b_b = bytes_of(chunk, dtype);
    a.batch_d_b = M * N * 4;
    a.split_k = static_cast<int>(chunk);
    // with an even number of splits from six on the grid is splits (x) by
    // tiles (y); with a multiple of eight each XCD runs whole splits and reads
    // only its own K ranges of A and B
    a.xcd_batches = whole_matrices_per_xcd(used, pl.grid);
    hipError_t err = hipSuccess;
    if (K > 0 && a.xcd_batches)
        err = tg_kernel(pl.kernel_id).launch(a, used, static_cast<int>(pl.grid), static_cast<hipStream_t>(stream));
    else if (K > 0)
        err = tg_kernel(pl.kernel_id).launch(a, pl.grid, static_cast<int>(used), static_cast<hipStream_t>(stream));
    if (err == hipSuccess)
        err = tg_splitk_reduce(static_cast<const float*>(workspace), K > 0 ? static_cast<int>(used) : 0,
                               static_cast<int>(M), static_cast<int>(N), D, ldd, alpha, relu ? 1 : 0, out_dtype,
                               static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}


}  // namespace

extern "C" {

int tile_gemm_splitk(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
                     const void* B, int64_t ldb, void* D, int64_t ldd, int dtype, int out_dtype, int splits,
                     void* workspace, int64_t workspace_bytes, void* stream, int kernel_id) {
    return splitk_impl(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, splits, workspace,
                       workspace_bytes, stream, kernel_id, false);
}

int tile_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
                             const void* B, int64_t ldb, void* D, int64_t ldd, int dtype, int out_dtype, int splits,
                             void* stream, int kernel_id) {
    return splitk_impl(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, splits, nullptr, 0, stream,
                       kernel_id, true);
}

int tile_gemm_softmax(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda, const void* B,
                      int64_t ldb, void* D, int64_t ldd, int dtype, int out_dtype, void* stream, int kernel_id) {
    int id = -1;
    int rc = softmax_plan(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, kernel_id, &id);
    if (rc) return rc;
    if (M == 0 || N == 0) return TG_OK;
    if (id < 0) {
        // two passes: the logits alpha*S into an fp32 D, then the row softmax in place
        rc = tile_gemm_out(M, N, K, alpha, 0, A, lda, B, ldb, D, ldd, dtype, TG_F32, stream, -1);
        if (rc) return rc;
        const hipError_t err = tg_softmax_rows(static_cast<float*>(D), static_cast<int>(M), static_cast<int>(N), ldd,
                                               static_cast<hipStream_t>(stream));
        return err == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
    }
    rc = device_ok();
    if (rc) return rc;
    const TgKernelDesc& k = tg_kernel(id);
    GemmArgs a{};
    a.A = static_cast<const char*>(A);
    a.B = static_cast<const char*>(B);
    a.D = D;
    a.lda_b = bytes_of(lda, dtype);
    a.ldb_b = bytes_of(ldb, dtype);
    a.ldd = ldd;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.alpha = alpha;
    a.tiles_m = static_cast<int>(cdiv(M, k.block_m));
    a.tiles_n = 1;
    a.group_m = k.group_m;
    a.out_dtype = out_dtype;
    a.epi = TG_EPI_SOFTMAX;
    const hipError_t err = k.launch(a, a.tiles_m, 1, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

int tile_gemm_query_plan_softmax(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, const void* D, int64_t ldd, int out_dtype,
                                 int kernel_id, tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    memset(out, 0, sizeof *out);
    int id = -1;
    const int rc = softmax_plan(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, kernel_id, &id);
    if (rc) return rc;
    if (id >= 0) {
        describe(tg_kernel(id), M, N, out);
        out->tiles_n = 1;  // one tile spans N
        out->grid = out->tiles_m;
    } else {
        out->kernel_id = -1;  // two launches: the plain product, then the row pass
        out->dtype = dtype;
    }
    return TG_OK;
}

int tile_gemm_out(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A,
                  int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd, int dtype,
                  int out_dtype, void* stream, int kernel_id) {
    return launch_batched(M, N, K, alpha, relu, A, lda, 0, B, ldb, 0, D, ldd, 0, 1, dtype, out_dtype, stream,
                          kernel_id);
}

int tile_gemm_staged(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
                     const void* B, int64_t ldb, void* D, int64_t ldd, int dtype, int out_dtype, void* workspace,
                     int64_t workspace_bytes, void* stream, int mode) {
    if (mode < -1 || mode > 1) return TG_ERR_PLAN;
    return gemm_staged(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, out_dtype, stream, workspace,
                       workspace_bytes, mode);
}

int tile_gemm_scaled(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
                     const void* scale_a, int64_t lds_a, const void* B, int64_t ldb, const void* scale_b,
                     int64_t lds_b, void* D, int64_t ldd, int dtype, int out_dtype, void* stream, int kernel_id) {
    Scales sc;
    const int rc = scaled_plan(M, N, K, A, lda, scale_a, lds_a, B, ldb, scale_b, lds_b, D, ldd, dtype, out_dtype,
                               &kernel_id, &sc);
    if (rc) return rc;
    return launch_batched(M, N, K, alpha, relu, A, lda, 0, B, ldb, 0, D, ldd, 0, 1, dtype, out_dtype, stream,
                          kernel_id, sc);
}

int tile_gemm_query_plan_scaled(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                                const void* scale_a, int64_t lds_a, const void* B, int64_t ldb, const void* scale_b,
                                int64_t lds_b, const void* D, int64_t ldd, int out_dtype, int kernel_id,
                                tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    Scales sc;
    const int rc = scaled_plan(M, N, K, A, lda, scale_a, lds_a, B, ldb, scale_b, lds_b, D, ldd, dtype, out_dtype,
                               &kernel_id, &sc);
    if (rc) return rc;
    return plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, kernel_id, out);
}

int tile_gemm_query_plan_staged(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                                const void* B, int64_t ldb, const void* D, int64_t ldd, int out_dtype,
                                const void* workspace, int64_t workspace_bytes, int mode, tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    if (mode < -1 || mode > 1) return TG_ERR_PLAN;
    int rc = validate(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, Batch());
    if (rc) return rc;
    const Staging st = staged_decision(M, N, K, A, lda, B, ldb, D, ldd, dtype, out_dtype, workspace,
                                       workspace_bytes, mode, &rc);
    if (rc) return rc;
    if (!st.on) return plan(M, N, K, dtype, A, lda, B, ldb, D, ldd, out_dtype, -1, out);
    describe(tg_kernel(st.staged_id), M, N, out);
    out->staged = 1;
    return out->grid > kMaxGrid ? TG_ERR_DIMS : TG_OK;
}

int64_t tile_gemm_staged_workspace_bytes(int64_t M, int64_t N, int64_t K, int dtype) {
    const int es = elem_bits(dtype) >= 8 ? elem_size(dtype) : 0;  // packed operands are never staged
    if (!es || M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
    if (M == 0 || N == 0 || K == 0) return 0;
    return staged_bytes(M, N, K, es);
}

int tile_gemm_ex(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A,
                 int64_t lda, const void* B, int64_t ldb, float* D, int64_t ldd, int dtype,
                 void* stream, int kernel_id) {
    return tile_gemm_out(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, TG_F32, stream, kernel_id);
}

int tile_gemm(int64_t M, int64_t N, int64_t K, float alpha, int relu, const void* A, int64_t lda,
              const void* B, int64_t ldb, float* D, int64_t ldd, int dtype, void* stream) {
    return tile_gemm_out(M, N, K, alpha, relu, A, lda, B, ldb, D, ldd, dtype, TG_F32, stream, -1);
}

int tile_gemm_kernel_count(void) { return tg_kernel_count(); }

int tile_gemm_kernel_info(int kernel_id, tile_gemm_plan_info* out) {
    if (!out) return TG_ERR_NULL;
    if (kernel_id < 0 || kernel_id >= tg_kernel_count()) return TG_ERR_PLAN;
    describe(tg_kernel(kernel_id), 0, 0, out);
    return TG_OK;
}

const char* tile_gemm_strerror(int code) {
    switch (code) {
        case TG_OK: return "success";
        case TG_ERR_DIMS: return "invalid dimensions (negative, above 2^30, or grid too large)";
        case TG_ERR_LD: return "leading stride too small (lda,ldb >= max(1,K); ldd >= max(1,M))";
        case TG_ERR_NULL: return "null pointer for an operand that is read or written";
        case TG_ERR_ALIGN: return "pointer not aligned to its element size";
        case TG_ERR_DTYPE: return "unknown operand or output dtype";
        case TG_ERR_ALIAS: return "output overlaps an input operand";
        case TG_ERR_LAUNCH: return "HIP kernel launch failed";
        case TG_ERR_DEVICE: return "no current gfx950 HIP device";
        case TG_ERR_PLAN: return "kernel instance unknown or not valid for these operands";
        case TG_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown status";
    }
}

int tile_gemm_abi_version(void) { return TILE_GEMM_ABI_VERSION; }

}  // extern "C"
