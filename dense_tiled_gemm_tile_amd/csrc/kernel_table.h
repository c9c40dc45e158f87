// Internal interface between the host plan/ABI layer and the kernel
// instances: the argument block every GEMM kernel takes and the static table
// describing each compiled instance.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_gemm.h"

struct GemmArgs {
    const char* A;   // a[m,k] at A + m*lda_b + k*s (4-bit: nibble k of the row, low first)
    const char* B;   // b[k,n] at B + n*ldb_b + k*s
    void* D;         // d[m,n] at element m + n*ldd of D, in type out_dtype
    int64_t lda_b;   // A leading stride in bytes
    int64_t ldb_b;   // B leading stride in bytes
    int64_t ldd;     // D leading stride in elements
    int M, N, K;
    float alpha;
    int relu;
    int tiles_m, tiles_n, group_m;
    int out_dtype;   // element type of D: TG_F32, TG_BF16 or TG_F16
    int64_t batch_a_b, batch_b_b, batch_d_b;  // byte distance between consecutive matrices (grid y)
    int split_k;     // split-K partial products: K elements per split (grid y = split, or grid x
                     // with xcd_batches), 0 = off
    int xcd_batches; // 1: grid x is the matrix (or split) and grid y the tile (see select_batch)
    int tile;        // set on the device by select_batch: the workgroup's tile in the grouped walk
    int epi;         // epilogue: 0 = alpha then optional ReLU per element, 1 = softmax over n
    // 8- and 4-bit operands: block-scale exponents (2^(e-127) per 32 consecutive k),
    // byte m*lds_a + k/32 for A row m and n*lds_b + k/32 for B column n;
    // nullptr = no scales
    const unsigned char* scale_a;
    const unsigned char* scale_b;
    int64_t lds_a, lds_b;
};

enum { TG_EPI_POINTWISE = 0, TG_EPI_SOFTMAX = 1 };

// Row softmax over n of an fp32 D, in place (second pass when one tile
// cannot span N).
hipError_t tg_softmax_rows(float* D, int M, int N, int64_t ldd, hipStream_t stream);

// Second phase of a split-K call: D = epilogue(sum over splits of the fp32
// partial products), summed in split order.
hipError_t tg_splitk_reduce(const float* ws, int splits, int M, int N, void* D, int64_t ldd, float alpha,
                            int relu, int out_dtype, hipStream_t stream);

// Staged operand copy: the M rows of A (byte stride lda_b) and the N rows of B
// (ldb_b), K elements of es bytes each, into dense rows of row_bytes (a
// multiple of 128) at dstA and dstB (16-byte aligned), zero past K.
hipError_t tg_stage_operands(const char* A, int64_t lda_b, int64_t M, const char* B, int64_t ldb_b, int64_t N, int K,
                             int es, int64_t row_bytes, char* dstA, char* dstB, hipStream_t stream);

// The library's static scratch array (one per GPU, for callers that cannot
// allocate): its size, and its device address on the current device (looked
// up once per device; no allocation).
constexpr int64_t kTgStaticScratchBytes = int64_t(TILE_GEMM_STATIC_SCRATCH_BYTES);
hipError_t tg_static_scratch(void** ptr);

typedef hipError_t (*TgLaunchFn)(const GemmArgs&, int64_t grid, int batch, hipStream_t stream);

struct TgKernelDesc {
    int id;
    int dtype;         // tile_gemm_dtype
    int block_m, block_n, block_k;
    int waves_m, waves_n;
    int wave_tile_m, wave_tile_n;
    int threads;
    int stages;
    int lds_bytes;
    int acc_per_lane;
    int load_class;    // minimum byte alignment of operand row starts (16, 4 or 2)
    int group_m;
    int eff_pct;       // expected MFMA efficiency, weighs tiles in the plan chooser
    TgLaunchFn launch;
    int64_t max_row_stride;  // largest lda/ldb in bytes the instance can address (0: any)
    int softmax;             // 1: the epilogue can also take a softmax over n (N <= block_n)
    int nt_store;            // 1: D is written with nontemporal stores
    int block_scales;        // 1: 8- or 4-bit instance that applies block scales (GemmArgs::scale_a/b)
    int k_slices;            // groups of waves that split K inside a workgroup, each over the whole tile (0: 1)
    int power_bound;         // 1: considered only for K loops of at least kPowerBoundStages stages (the
                             // 16x16x32 wide kernel; below that it and the 32x32x16 one trade places)
};

// Element bits of an operand type (the 4- and 6-bit formats are packed).
#define TG_ELEM_BITS(DT)                                                                        \
    ((DT) == TG_F32 ? 32 : ((DT) == TG_E4M3 || (DT) == TG_E5M2) ? 8 : (DT) == TG_E2M1 ? 4      \
     : ((DT) == TG_E2M3 || (DT) == TG_E3M2) ? 6 : 16)
// K elements in one 128-byte row segment of a wide-kernel stage (6-bit: a
// stage is 128 elements, 96 bytes).
#define TG_WIDE_STAGE_K(DT) (TG_ELEM_BITS(DT) == 6 ? 128 : 1024 / TG_ELEM_BITS(DT))
// Element bytes of an operand type of at least 8 bits.
#define TG_ELEM_BYTES(DT) (TG_ELEM_BITS(DT) / 8)

// The instances each kernel translation unit contributes (host pass only).
extern const TgKernelDesc tg_entries_wide16[];
extern const int tg_entries_wide16_count;
extern const TgKernelDesc tg_entries_wide32[];
extern const int tg_entries_wide32_count;
extern const TgKernelDesc tg_entries_wide8[];
extern const int tg_entries_wide8_count;
extern const TgKernelDesc tg_entries_stream[];
extern const int tg_entries_stream_count;
extern const TgKernelDesc tg_entries_rs[];
extern const int tg_entries_rs_count;
extern const TgKernelDesc tg_entries_kslice[];
extern const int tg_entries_kslice_count;
extern const TgKernelDesc tg_entries_wide4[];
extern const int tg_entries_wide4_count;
extern const TgKernelDesc tg_entries_wide6[];
extern const int tg_entries_wide6_count;
extern const TgKernelDesc tg_entries_wide_m16[];
extern const int tg_entries_wide_m16_count;

// The instance table, indexed by kernel id (ids are 0 .. tg_kernel_count()-1).
int tg_kernel_count();
const TgKernelDesc& tg_kernel(int id);
