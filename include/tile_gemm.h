/*
 * tile_gemm — tiled dense GEMM with fused alpha/ReLU epilogue for AMD MI355X
 * (gfx950, CDNA4), C ABI.
 *
 * Operation (Tylo.jl manual, "Walk through GEMM": opening paragraph, section 2
 * "Bind runtime global arrays" and section 5 "Apply the epilogue and store by
 * ownership"):
 *
 *     D = alpha * A * B,  optionally followed by D = max(D, 0)  (ReLU)
 *
 * with FP32 accumulation.  All coordinates are zero-based; s is the operand
 * element size (1 for the 8-bit formats, 2 for bf16/fp16, 4 for fp32):
 *
 *   A is logically (M,K), stored K-contiguous:  a[m,k] at byte A + (m*lda + k)*s
 *   B is logically (K,N), stored K-contiguous:  b[k,n] at byte B + (k + n*ldb)*s
 *   D is logically (M,N), fp32, M-contiguous:   d[m,n] at byte D + (m + n*ldd)*4
 *
 * The 4-bit (TG_E2M1) and 6-bit (TG_E2M3, TG_E3M2) formats are packed:
 * element i of an operand array holds bits [w*i, w*i + w) of the array read
 * as a little-endian bit string (w = 4 or 6), i.e. a 4-bit a[m,k] is the low
 * nibble of byte A + (m*lda + k)/2 when m*lda + k is even and the high nibble
 * otherwise, and four 6-bit elements fill three bytes (b[k,n] likewise at
 * index k + n*ldb).  Every row must start on a byte, so lda and ldb are even
 * (4-bit) or multiples of 4 (6-bit) (TG_ERR_LD), and the pointers need only
 * byte alignment.  Strides and sizes count elements.
 *
 * For 0 <= m < M and 0 <= n < N the call writes
 *
 *     d[m,n] = relu ? max(alpha * S, 0) : alpha * S,   S = sum_{k<K} a[m,k]*b[k,n]
 *
 * (alpha is applied to the fp32 accumulator, then the clamp).  No other byte
 * of D is written: the padding rows m >= M of each D column are left alone.
 * There is no beta; prior contents of D are irrelevant.  K = 0 writes zeros;
 * M = 0 or N = 0 is a no-op.  Ragged edges are handled inside the kernel:
 * operand elements with k >= K are never read and contribute exactly zero
 * (cuTile.jl tutorial "Matrix Multiplication", section "Sizes that are not a
 * multiple of the tile shape").
 *
 * Ownership: A, B and D are device pointers owned by the caller and only
 * borrowed for the duration of the enqueued kernels (Tylo.jl manual, "Walk
 * through GEMM", section 2: the kernel's views borrow storage the caller
 * owns).  The library allocates no device memory, never synchronises a
 * stream or the device, and keeps no pointer of the caller's after the call
 * returns: the kernels are enqueued on `stream` (a hipStream_t; NULL means
 * the default stream) and the call returns after the enqueue (section 4:
 * no hidden allocation).  Scratch space, where an entry point needs it
 * (split-K partial products, staged operand copies), is a workspace the
 * caller passes in.  D must not overlap A or B.  The library's only shared
 * state is an immutable instance table and a per-device architecture check,
 * so calls from several host threads may run concurrently; work enqueued on
 * one stream runs in the order of the calls.
 *
 * Alignment: pointers must be aligned to their element size.  Nothing
 * stronger is required.  When the operand rows are not all 16-byte aligned
 * (odd lda/ldb, offset views), the plan takes a kernel whose loads need only
 * 4- or 2-byte aligned rows (Tylo.jl manual, "Walk through GEMM", section 3:
 * the caller establishes the alignment and the plan must respect it);
 * tile_gemm_staged can instead copy the operands into aligned rows in a
 * caller workspace first.
 *
 * Errors: every entry point returns 0 on success or one of the negative
 * tile_gemm_status codes below; no exception or abort crosses the ABI.
 * Argument validation happens before any HIP call, so invalid arguments are
 * reported even on a machine without a GPU.
 */
#ifndef TILE_GEMM_H
#define TILE_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of A and B (both the same), and of D for tile_gemm_out.
 * tile_gemm and tile_gemm_ex always write fp32 D. */
enum tile_gemm_dtype {
    TG_BF16 = 1, /* bfloat16 operands, bf16 MFMA */
    TG_F16 = 2,  /* IEEE binary16 operands, fp16 MFMA */
    TG_F32 = 3,  /* IEEE binary32 operands, fp32 MFMA (full fp32 products) */
    TG_E4M3 = 4, /* 8-bit float operands (1-4-3, bias 7, no infinity), 8-bit MFMA */
    TG_E5M2 = 5, /* 8-bit float operands (1-5-2, bias 15, IEEE-style), 8-bit MFMA */
    TG_E2M1 = 6, /* 4-bit float operands (the MX FP4 element: 1-2-1, bias 1, values
                    0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, no infinity or
                    NaN), packed two per byte, 4-bit MFMA */
    TG_E2M3 = 7, /* 6-bit float operands (MX FP6 E2M3: 1-2-3, bias 1, largest 7.5,
                    no infinity or NaN), packed four per three bytes, 6-bit MFMA */
    TG_E3M2 = 8  /* 6-bit float operands (MX FP6 E3M2: 1-3-2, bias 3, largest 28,
                    no infinity or NaN), packed as TG_E2M3 */
};

enum tile_gemm_status {
    TG_OK = 0,
    TG_ERR_DIMS = -1,   /* M, N or K negative or above 2^30, or more than 2^24 tiles */
    TG_ERR_LD = -2,     /* lda < max(1,K), ldb < max(1,K) or ldd < max(1,M), or a
                           packed operand row that does not start on a byte */
    TG_ERR_NULL = -3,   /* NULL pointer for an operand that is read or written */
    TG_ERR_ALIGN = -4,  /* pointer not aligned to its element size */
    TG_ERR_DTYPE = -5,  /* dtype or out_dtype not one of tile_gemm_dtype */
    TG_ERR_ALIAS = -6,  /* D's byte range overlaps A's or B's */
    TG_ERR_LAUNCH = -7, /* the HIP launch failed (hipGetLastError) */
    TG_ERR_DEVICE = -8, /* no current HIP device, or it is not gfx950 */
    TG_ERR_PLAN = -9,   /* requested kernel id unknown or not valid for the call */
    TG_ERR_WORKSPACE = -10 /* workspace missing, misaligned or too small */
};

/* The host plan for one call (what the kernel will be launched with). */
typedef struct tile_gemm_plan_info {
    int32_t kernel_id;     /* index of the compiled kernel instance */
    int32_t dtype;         /* tile_gemm_dtype */
    int32_t block_m;       /* macro-tile extent along m (A rows) */
    int32_t block_n;       /* macro-tile extent along n (B columns) */
    int32_t block_k;       /* K elements staged per pipeline stage */
    int32_t waves_m;       /* wave grid of one workgroup */
    int32_t waves_n;
    int32_t wave_tile_m;   /* output extent owned by one wave */
    int32_t wave_tile_n;
    int32_t threads;       /* threads per workgroup (64 per wave) */
    int32_t stages;        /* LDS buffering stages */
    int32_t lds_bytes;     /* static LDS per workgroup */
    int32_t acc_per_lane;  /* fp32 accumulators held by each lane */
    int32_t load_class;    /* 16, 4 or 2: byte alignment of every operand row start */
    int32_t group_m;       /* tile-rows per group in the grouped tile order */
    int32_t staged;        /* always 0 for a query (tile_gemm_staged decides per call) */
    int32_t k_slices;      /* groups of waves of a workgroup that each take 1/k_slices of K over the whole tile */
    int32_t block_scales;  /* 1: the instance applies block scales (tile_gemm_scaled) */
    int64_t tiles_m;       /* ceil(M / block_m) */
    int64_t tiles_n;       /* ceil(N / block_n) */
    int64_t grid;          /* workgroups launched = tiles_m * tiles_n */
} tile_gemm_plan_info;

/*
 * D = alpha*A*B (+ReLU if relu != 0), fp32 accumulation, enqueued on `stream`.
 * M, N, K: problem sizes (>= 0).  lda, ldb: operand leading strides in
 * elements (>= max(1,K)); ldd: output leading stride in elements (>= max(1,M)).
 * dtype: tile_gemm_dtype of A and B.  Returns TG_OK or a tile_gemm_status.
 */
int tile_gemm(int64_t M, int64_t N, int64_t K, float alpha, int relu,
              const void* A, int64_t lda, const void* B, int64_t ldb,
              float* D, int64_t ldd, int dtype, void* stream);

/*
 * As tile_gemm, but with an explicit kernel instance (kernel_id from
 * tile_gemm_query_plan or tile_gemm_kernel_count; -1 = the automatic
 * choice).  For tests and tuning: every instance computes the same result.
 * Returns TG_ERR_PLAN if the instance does not exist, has another dtype, or
 * needs a stronger row alignment than the operands have.
 */
int tile_gemm_ex(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                 const void* A, int64_t lda, const void* B, int64_t ldb,
                 float* D, int64_t ldd, int dtype, void* stream, int kernel_id);

/*
 * As tile_gemm_ex, with D of element type out_dtype (TG_F32, TG_BF16 or
 * TG_F16): d[m,n] at byte D + (m + n*ldd)*out_size, out_size 4 or 2.  The
 * accumulation and the epilogue stay fp32 (alpha, then the clamp); the
 * epilogue value is then rounded to nearest-even in out_dtype (fp16: values
 * beyond its range become +-inf, subnormals are kept) on the way out (cuTile.jl
 * tutorial "Matrix Multiplication", Step 4: keep the Float32 accumulator and
 * convert on the way out).  D must be aligned to out_size; everything else is
 * as for tile_gemm, and out_dtype TG_F32 is exactly tile_gemm_ex.
 */
int tile_gemm_out(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  void* D, int64_t ldd, int dtype, int out_dtype,
                  void* stream, int kernel_id);

/*
 * Batched: `batch` independent products D_b = alpha*A_b*B_b (+ReLU), b = 0 ..
 * batch-1, in one launch (cuTile.jl tutorial "Matrix Multiplication", "Where to
 * go from here": batched operands).  Matrix b of A starts stride_a elements
 * after matrix b-1 (likewise B with stride_b, D with stride_d, in elements of
 * their own types); a stride of 0 reuses one A or B for every product.  Each
 * product is exactly the tile_gemm_out product of its matrices.
 * Extra checks: 0 <= batch <= 65535 (TG_ERR_DIMS); strides >= 0 and at most
 * 2^40, and with batch > 1, stride_d >= (N-1)*ldd + M so the outputs do not
 * overlap (TG_ERR_LD); D's whole span must not overlap A's or B's whole span
 * (TG_ERR_ALIAS).  batch = 0 is a no-op.
 */
int tile_gemm_batched(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                      const void* A, int64_t lda, int64_t stride_a,
                      const void* B, int64_t ldb, int64_t stride_b,
                      void* D, int64_t ldd, int64_t stride_d, int64_t batch,
                      int dtype, int out_dtype, void* stream, int kernel_id);

/*
 * Split-K (for problems with few output tiles and a long K): K is cut into
 * `splits` contiguous ranges of whole pipeline stages; each range's fp32
 * partial product goes to the caller's workspace in a first launch, and a
 * second launch on the same stream adds the partials in split order (so the
 * result is the same bits on every call), applies alpha and the clamp and
 * stores D in out_dtype.  The epilogue thus runs after the reduction, never on
 * partial sums.
 *
 * splits: 1 .. 256 requested (fewer are used when K has fewer stages; 1 is the
 * plain product), or 0 for an automatic choice (no split unless the output
 * has fewer tiles than the GPU has CUs and K has at least 64 stages; then
 * about 32 stages per split but at least one workgroup per CU, at least 16
 * stages per split, at most 64 splits, never more than `workspace_bytes`
 * holds, and from 8 on a multiple of 8, so that every split runs whole on one
 * XCD); workspace: device
 * memory of at least
 * tile_gemm_splitk_workspace_bytes(M, N, splits) bytes, 16-byte aligned, not
 * overlapping A, B or D, owned by the caller and reusable once the stream has
 * passed the call (its prior contents are irrelevant).  The library still
 * allocates nothing.  Errors as tile_gemm_out, plus TG_ERR_DIMS for splits out
 * of range and TG_ERR_WORKSPACE for a missing, misaligned or short workspace.
 */
int tile_gemm_splitk(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                     const void* A, int64_t lda, const void* B, int64_t ldb,
                     void* D, int64_t ldd, int dtype, int out_dtype, int splits,
                     void* workspace, int64_t workspace_bytes, void* stream, int kernel_id);

/*
 * As tile_gemm_splitk, for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * allocation): the fp32 partial products live in the library's own static
 * scratch array of TILE_GEMM_STATIC_SCRATCH_BYTES per GPU (part of the
 * library's code object, held on each GPU it runs on until the process
 * ends) instead of a caller workspace.  The call allocates nothing and
 * synchronises nothing.  Every call on one GPU shares that GPU's array, so
 * calls that can overlap on one GPU (several streams, several host threads)
 * race and must be ordered by the caller; a call fully ordered after another
 * on the stream is safe (each call writes every partial it reads).
 * Errors as tile_gemm_splitk, and TG_ERR_WORKSPACE when the partials of the
 * requested split (splits * M * N * 4 bytes for the splits that get work)
 * exceed the scratch; splits = 0 chooses automatically within the scratch.
 */
int tile_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                             const void* A, int64_t lda, const void* B, int64_t ldb,
                             void* D, int64_t ldd, int dtype, int out_dtype, int splits,
                             void* stream, int kernel_id);

/* Bytes of the static scratch array tile_gemm_splitk_noalloc uses (32 MiB). */
#define TILE_GEMM_STATIC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * Softmax over n (a row-wise epilogue; Tylo.jl manual, "Walk through GEMM",
 * section 5, on replacing the pointwise ReLU by a softmax, which needs a
 * reduction across the waves that share a row):
 *
 *     x[m,n] = alpha * S[m,n]  (fp32),
 *     d[m,n] = exp(x[m,n] - max_n' x[m,n']) / sum_n' exp(x[m,n'] - max_n' x[m,n'])
 *
 * for every row m, over the N columns.  When one tile of a softmax-capable
 * instance spans N (N <= 256 for 16-bit operands, N <= 128 for fp32), it is
 * fused into the GEMM's epilogue and D may be fp32, bf16 or fp16
 * (out_dtype).  Otherwise it runs as two launches on the stream -- the fp32
 * logits into D, then the row softmax in place -- which needs out_dtype
 * TG_F32 (else TG_ERR_DIMS).  kernel_id forces a fused instance (-1 = auto).
 * Other rules as tile_gemm_out.
 */
int tile_gemm_softmax(int64_t M, int64_t N, int64_t K, float alpha,
                      const void* A, int64_t lda, const void* B, int64_t ldb,
                      void* D, int64_t ldd, int dtype, int out_dtype,
                      void* stream, int kernel_id);

/*
 * 8-bit (TG_E4M3, TG_E5M2), 6-bit (TG_E2M3, TG_E3M2) and 4-bit (TG_E2M1)
 * operands with optional block scales: every 32 consecutive k of an A row (and of a B column) share one
 * unsigned 8-bit exponent e, and the elements of that block stand for their
 * decoded value times 2^(e - 127) (e = 255: NaN).  The pages name
 * block-scaled 8-bit and 4-bit matmuls (cuTile.jl tutorial "Matrix
 * Multiplication", "Where to go from here") without defining them; this is
 * the plain reading of the MX formats, and the product then is
 *
 *     d[m,n] = epilogue(alpha * sum_k a[m,k]*sa[m,k/32] * b[k,n]*sb[n,k/32])
 *
 * accumulated in fp32 on the scaled MFMA (which applies the scales itself).
 * Scale of A row m, block j: byte scale_a[m*lds_a + j]; of B column n:
 * scale_b[n*lds_b + j].  8- and 6-bit operands: lds_a, lds_b >= 4*ceil(K/128) and
 * multiples of 4, scale pointers 4-byte aligned (the kernels read the four
 * scales of each 128-k stage as one dword); 4-bit operands: lds_a, lds_b >=
 * 16*ceil(K/512) and multiples of 16, scale pointers 16-byte aligned (the
 * kernels copy the sixteen scales of two 256-k stages as one 16-byte piece);
 * otherwise TG_ERR_LD / TG_ERR_ALIGN.  Scales of blocks past ceil(K/32) are
 * read but ignored.  Either pointer may be NULL (no scale on
 * that side); scales with 16-bit or fp32 operands give TG_ERR_DTYPE; the
 * scales must not overlap D (TG_ERR_ALIAS).  kernel_id as tile_gemm_ex
 * (only instances that apply block scales accept scales; others give
 * TG_ERR_PLAN).  Other rules as tile_gemm_out.
 */
int tile_gemm_scaled(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                     const void* A, int64_t lda, const void* scale_a, int64_t lds_a,
                     const void* B, int64_t ldb, const void* scale_b, int64_t lds_b,
                     void* D, int64_t ldd, int dtype, int out_dtype, void* stream, int kernel_id);

/*
 * A single product on staged operand copies: a first launch copies the M rows
 * of A and the N rows of B into `workspace`, each row starting 16-byte aligned
 * and holding K rounded up to a whole 128-byte K stage (64 bf16/fp16 or 32
 * fp32 elements) with exact zeros past K; the product then runs on the copies
 * with the widest loads, and the zero padding adds exact zeros to every sum
 * (the same zero-fill of the ragged K edge the bounded path does in place;
 * cuTile.jl tutorial "Matrix Multiplication", section "Sizes that are not a
 * multiple of the tile shape"; Tylo.jl manual, "Walk through GEMM", section 3:
 * the vector width a kernel may use depends on the alignment of the rows it
 * reads).  Layout of the workspace: A's copy at byte 0 (row m at
 * m*row_bytes), B's copy at the next 256-byte boundary after M*row_bytes,
 * row_bytes = 128*ceil(K*s/128).
 *
 * mode 1: always stage (TG_ERR_WORKSPACE when workspace is NULL, not 256-byte
 * aligned or shorter than tile_gemm_staged_workspace_bytes); mode -1: stage
 * only when the operand rows are not all 16-byte aligned and the time model
 * of the plan says the copy pays for itself, and run the direct plan when the
 * workspace does not suffice; mode 0: never (as tile_gemm_out).  workspace:
 * device memory owned by the caller, not overlapping A, B or D
 * (TG_ERR_ALIAS), reusable once the stream has passed the call.  M, N or K
 * = 0 never stages.  Packed 4- and 6-bit operands are never staged (mode 1
 * gives TG_ERR_DTYPE; mode -1 runs the direct plan).  Other rules and errors
 * as tile_gemm_out with kernel_id -1.
 */
int tile_gemm_staged(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                     const void* A, int64_t lda, const void* B, int64_t ldb,
                     void* D, int64_t ldd, int dtype, int out_dtype,
                     void* workspace, int64_t workspace_bytes, void* stream, int mode);

/* Workspace bytes tile_gemm_staged needs for these sizes (0 when M, N or K
 * is 0; -1 for an unknown or packed dtype or sizes out of range). */
int64_t tile_gemm_staged_workspace_bytes(int64_t M, int64_t N, int64_t K, int dtype);

/* Workspace a split-K call needs: splits * M * N * 4 bytes (0 for splits = 1
 * or an empty output; splits = 0: enough for any automatic choice, i.e. 64
 * splits; -1 for negative or oversized arguments). */
int64_t tile_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int splits);

/*
 * Host-only: validate the arguments exactly as tile_gemm does and describe the
 * plan it would launch (no HIP call is made; pointers are only inspected for
 * alignment and overlap).  For tests and tuning.
 */
int tile_gemm_query_plan(int64_t M, int64_t N, int64_t K, int dtype,
                         const void* A, int64_t lda, const void* B, int64_t ldb,
                         const float* D, int64_t ldd, tile_gemm_plan_info* out);

/* Host-only: as tile_gemm_query_plan, for a tile_gemm_out call with D of
 * element type out_dtype and an explicit kernel instance (kernel_id -1 = the
 * automatic choice; TG_ERR_PLAN as for tile_gemm_ex).  The plan does not
 * depend on out_dtype except through the D line alignment it weighs. */
int tile_gemm_query_plan_out(int64_t M, int64_t N, int64_t K, int dtype,
                             const void* A, int64_t lda, const void* B, int64_t ldb,
                             const void* D, int64_t ldd, int out_dtype, int kernel_id,
                             tile_gemm_plan_info* out);

/* Host-only: the plan of a tile_gemm_batched call; `grid` counts the
 * workgroups of all products (tiles_m * tiles_n * batch). */
int tile_gemm_query_plan_batched(int64_t M, int64_t N, int64_t K, int dtype,
                                 const void* A, int64_t lda, int64_t stride_a,
                                 const void* B, int64_t ldb, int64_t stride_b,
                                 const void* D, int64_t ldd, int64_t stride_d, int64_t batch,
                                 int out_dtype, int kernel_id, tile_gemm_plan_info* out);

/* Host-only: the plan of a tile_gemm_softmax call after the same validation:
 * the fused instance (grid = tiles along m; one tile spans N), or kernel_id
 * -1 when the call runs as two launches (the fp32 logits, then the row pass). */
int tile_gemm_query_plan_softmax(int64_t M, int64_t N, int64_t K, int dtype,
                                 const void* A, int64_t lda, const void* B, int64_t ldb,
                                 const void* D, int64_t ldd, int out_dtype, int kernel_id,
                                 tile_gemm_plan_info* out);

/* Host-only: the plan of a tile_gemm_scaled call after the same validation
 * (with scales, the instance that applies them). */
int tile_gemm_query_plan_scaled(int64_t M, int64_t N, int64_t K, int dtype,
                                const void* A, int64_t lda, const void* scale_a, int64_t lds_a,
                                const void* B, int64_t ldb, const void* scale_b, int64_t lds_b,
                                const void* D, int64_t ldd, int out_dtype, int kernel_id,
                                tile_gemm_plan_info* out);

/* Host-only: the plan of a tile_gemm_staged call after the same validation:
 * staged = 1 and the product on the staged copies (load_class 16, the instance
 * chosen for rows of the rounded-up K) when the copy runs, else the direct
 * plan. */
int tile_gemm_query_plan_staged(int64_t M, int64_t N, int64_t K, int dtype,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                const void* D, int64_t ldd, int out_dtype,
                                const void* workspace, int64_t workspace_bytes, int mode,
                                tile_gemm_plan_info* out);

/* Number of compiled kernel instances (valid kernel ids are 0 .. count-1). */
int tile_gemm_kernel_count(void);

/* Static description of kernel instance `kernel_id` (grid fields are 0). */
int tile_gemm_kernel_info(int kernel_id, tile_gemm_plan_info* out);

/* Static string for a status code ("unknown status" for codes not listed). */
const char* tile_gemm_strerror(int code);

/* ABI version of this header (bumped on any incompatible change). */
int tile_gemm_abi_version(void);

#define TILE_GEMM_ABI_VERSION 9

#ifdef __cplusplus
}
#endif

#endif /* TILE_GEMM_H */
