/*
 * rfp4.h -- C ABI of librfp4.so: ROCmFP4 quantized-weight decode, GEMV and GEMM on
 * AMD Instinct MI355X (gfx950).
 *
 * Weight format: "Feasibility Report: Porting ROCmFP4 to Atlas", section "What is
 * ROCmFP4?".
 *   - "Block Layout": a block holds 32 weights as 16 bytes `qs` of packed 4-bit
 *     indices followed by the scale byte(s). Dual-scale (Q4_0_ROCMFP4): two scale
 *     bytes, one per 16-weight half, 18 bytes, 4.50 bits per weight. Fast single-
 *     scale (Q4_0_ROCMFP4_FAST): one scale byte for the block, 17 bytes, 4.25 bits.
 *   - "Codebook10 Value Table": an index selects one of
 *     {0,1,2,3,4,6,8,10, 0,-1,-2,-3,-4,-6,-8,-10}.
 *   - "Scale Format": scale bytes are finite unsigned E4M3 decoded to half-scale
 *     fp32; row validation rejects non-finite bytes once, so the hot path does not
 *     check them.
 * Conventions this library fixes where the page is silent:
 *   - index t (0..15) is the low nibble of qs[t], index t+16 its high nibble;
 *   - decoded scale S(b) = E4M3(b & 0x7F) / 2 (bit 7 ignored; exponent field 0 is
 *     the E4M3 subnormal m * 2^-9; 0x7F decodes by the same bit formula to 240);
 *   - weight = codebook[index] * S (IEEE product, so -10 * 0 = -0.0);
 *   - a matrix W of n rows and k columns is n rows of k/32 blocks, back to back;
 *     block j of a row holds columns 32j..32j+31; row stride = (k/32) * block bytes.
 *
 * General rules for every entry point:
 *   - All pointers except rfp4_validate's `w_host` are device pointers. The caller
 *     owns every buffer it passes. No entry point frees memory or synchronizes a
 *     stream or the device. The dequant, encoder and validation entry points never
 *     allocate; rfp4_gemm and rfp4_gemv(_multi) allocate a workspace at its first need
 *     (see there) and keep it; rfp4_gemm_dequant uses rocBLAS, which keeps handles and
 *     workspace of its own. Global state: per-device caches of the CU count and of
 *     kernel attributes (atomics), the workspaces and the rocBLAS handles (behind
 *     mutexes), so calls from several threads are safe. Nothing reads the
 *     environment.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls are
 *     asynchronous and ordered on that stream; a fault in a kernel surfaces at the
 *     caller's next synchronization.
 *   - Every argument check runs before any HIP call, so argument errors are
 *     reported without touching the GPU. Scale bytes are NOT checked on these hot
 *     paths: call rfp4_validate once when the weights are loaded.
 *   - Alignment: W must start on a 16-byte boundary (RFP4_ERR_UNSUPPORTED
 *     otherwise); its rows may have any length, so k is any multiple of 32 and rows
 *     need not start on a 16-byte boundary. The activations x and A and the outputs
 *     y and C need 4-byte alignment, with an even leading dimension for x and A (every
 *     16-bit activation row then starts on a 4-byte boundary); any ldy and ldc are
 *     accepted. Rows that are not 16-byte aligned are read with the same vector loads
 *     at some cost in load cycles. The dequant outputs and the encoder's buffers keep
 *     the 16-byte rule stated with those calls (they are written and read with
 *     16-byte vector accesses).
 *   - Sizes: 1 <= n, m and 32 <= k, with n, m, k <= 2^31 - 1 and W at most 2^40
 *     bytes (RFP4_ERR_SHAPE otherwise); buffers are addressed with 64-bit offsets.
 */
#ifndef RFP4_H
#define RFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef RFP4_API
#define RFP4_API __attribute__((visibility("default")))
#endif

typedef enum rfp4_status {
  RFP4_OK = 0,
  RFP4_ERR_NULL = 1,             /* a required pointer is NULL */
  RFP4_ERR_SHAPE = 2,            /* n, m or k out of range, k % 32 != 0, batch
                                    outside 1..8, or a leading dimension too small */
  RFP4_ERR_UNSUPPORTED = 3,      /* unknown layout or dtype, or an alignment rule broken */
  RFP4_ERR_NONFINITE_SCALE = 4,  /* rfp4_validate found a non-finite scale byte */
  RFP4_ERR_HIP = 5,              /* the HIP runtime reported an error at launch */
  RFP4_ERR_SCRATCH = 6           /* rfp4_gemm_noalloc: the forced plan's partial sums need
                                    more than RFP4_GEMM_SCRATCH_BYTES */
} rfp4_status;

typedef enum rfp4_layout {
  RFP4_DUAL = 0, /* Q4_0_ROCMFP4: qs[16], e[2]; 18 bytes per 32 weights */
  RFP4_FAST = 1  /* Q4_0_ROCMFP4_FAST: qs[16], e; 17 bytes per 32 weights */
} rfp4_layout;

typedef enum rfp4_dtype {
  RFP4_F16 = 0,  /* IEEE binary16 */
  RFP4_BF16 = 1, /* bfloat16 */
  RFP4_F32 = 2   /* IEEE binary32 (quantizer input only) */
} rfp4_dtype;

/* Bytes per 32-weight block ("Block Layout"): 18 (dual), 17 (fast), 0 for an
 * unknown layout. */
RFP4_API size_t rfp4_block_bytes(int layout);

/* Bytes of one weight row of k columns: (k / 32) * rfp4_block_bytes(layout);
 * -1 if the layout is unknown or k is not a positive multiple of 32. */
RFP4_API int64_t rfp4_row_bytes(int layout, int64_t k);

/* Static, human-readable text for a status code (never NULL). */
RFP4_API const char* rfp4_status_string(int status);

/* Row validation ("Scale Format": non-finite scale bytes are rejected when the
 * weights are loaded). Host memory: `w_host` holds n rows of packed blocks. A scale
 * byte is non-finite when its low seven bits are all ones (0x7F or 0xFF); index
 * bytes are never rejected. On RFP4_ERR_NONFINITE_SCALE, *first_bad_block (if the
 * pointer is not NULL) receives the row-major number (row * k/32 + block) of the
 * first offending block; on RFP4_OK it receives -1. Runs on the calling thread. */
RFP4_API rfp4_status rfp4_validate(const uint8_t* w_host, int layout, int64_t n, int64_t k,
                          int64_t* first_bad_block);

/* Dequantization, the page's "reference decoder" ("Integration Options", Option 1):
 * out[r * ldo + c] = weight (r, c) as fp32, bit-exact (every codebook value times
 * every decoded scale is representable in fp32). `out` has n rows of ldo floats,
 * ldo >= k, ldo % 4 == 0. */
RFP4_API rfp4_status rfp4_dequant(const void* w, int layout, int64_t n, int64_t k, float* out,
                         int64_t ldo, void* stream);

/* Dequantization to bf16: out[r * ldo + c] = weight (r, c) as bf16 bits, bit-exact
 * (every codebook value times every decoded scale is a bf16 value; signs of zero as
 * rfp4_dequant). `out` has n rows of ldo bf16 values, ldo >= k, ldo % 8 == 0,
 * 16-byte aligned, n * ldo <= 2^39. */
RFP4_API rfp4_status rfp4_dequant_bf16(const void* w, int layout, int64_t n, int64_t k,
                                       uint16_t* out, int64_t ldo, void* stream);

/* Decode matvec, the page's decode hot path ("Kernel System": gemv; "Integration
 * Options", Option 2): for b < batch and r < n,
 *   y[b * ldy + r] = sum_c weight(r, c) * x[b * ldx + c]
 * with x of dtype xdtype (RFP4_F16 or RFP4_BF16), products formed exactly and summed
 * in fp32, y fp32. 1 <= batch <= 8, ldx >= k (ldx even), ldy >= n.
 * Kernel choice (each sums in its own fp32 order, so the last bits differ between
 * them; rfp4_gemv_multi_ex can force one):
 *   - batch 1: a dot-product kernel; launches with the dual layout, f16 activations,
 *     k = 5120, every matrix's rows a multiple of 16 and at least two 16-row tiles per
 *     CU spread evenly over the CUs (the busiest at most 7 % above the average) run a
 *     batch-1 matrix-core kernel ("tall") instead;
 *   - batch 2: a matrix-core kernel of 16-row tiles when the launch has 4096 to 65536
 *     rows in all, otherwise the dot-product kernel;
 *   - batches 3 to 8: the matrix-core kernel, except one matrix of at most 1024 rows
 *     and k <= 6144 up to batch 6 (the dot-product kernel).
 * Workspace: when a launch's tiles leave the CUs short of work (long rows: every part
 * keeps at least 5 chunks of 16 units, a unit being two blocks when k / 32 is even and
 * one otherwise) the tile kernel gives each tile's k range to 2 to 4 workgroups whose
 * fp32 partial sums meet in a device workspace of fixed size (2 MiB + 4 KiB) that the library
 * allocates once per (device, stream) at its first need and keeps until the process
 * ends; the parts are added in a fixed order, so results are deterministic. The
 * workspace is never freed or reallocated, and no call synchronizes. It is never
 * allocated while the stream is being captured into a graph (the launch then runs
 * unsplit, which changes the last bits), so call once on a stream before capturing on
 * it. A captured split launch uses the capturing stream's workspace: replay such a
 * graph only ordered with that stream's other work and with its own other replays. */
RFP4_API rfp4_status rfp4_gemv(const void* w, int layout, int64_t n, int64_t k, const void* x,
                      int xdtype, int64_t batch, int64_t ldx, float* y, int64_t ldy,
                      void* stream);

/* Several decode matvecs that share one activation batch, in one launch: the page's
 * gemv_gate_up ("Kernel System"), also used for q/k/v. For i < count, part i computes
 *   y[i][b * ldy[i] + r] = sum_c weight_i(r, c) * x[b * ldx + c],  r < n[i], b < batch
 * as rfp4_gemv does for w[i], with the same layout and k for every part and the same
 * accuracy (the kernel and lane mapping, and so the fp32 summation order, are chosen
 * for the launch as a whole; with the same mapping the results equal separate
 * rfp4_gemv calls bit for bit). The row groups of all parts are split evenly over the
 * CUs, so small matrices (k/v) ride along with large ones. `w`, `n`, `y` and `ldy` are
 * host arrays of `count` entries (1 <= count <= RFP4_MAX_GEMV_PARTS) holding device
 * pointers and sizes; the total row count must be <= 2^31 - 1. Every part is checked
 * as in rfp4_gemv before any HIP call. Workspace as rfp4_gemv. */
#define RFP4_MAX_GEMV_PARTS 8
RFP4_API rfp4_status rfp4_gemv_multi(int count, const void* const* w, const int64_t* n,
                                     int layout, int64_t k, const void* x, int xdtype,
                                     int64_t batch, int64_t ldx, float* const* y,
                                     const int64_t* ldy, void* stream);

/* Weight-only 4-bit GEMM for prefill ("Kernel System": w4a16_gemm):
 *   c[i * ldc + r] = bf16_rne( sum_q a[i * lda + q] * weight(r, q) ),  i < m, r < n
 * i.e. C = A * W^T with A (m x k, bf16, row-major) and C (m x n, bf16, row-major);
 * weight tiles are decoded to bf16 in LDS and multiplied on the matrix cores with
 * fp32 accumulation. lda >= k (lda even), ldc >= n, and
 * m * lda, m * ldc <= 2^39 (RFP4_ERR_SHAPE otherwise).
 * Balance: the columns of C are split between 256 x 256 tiles and trailing strips of
 * 128 x 128 tiles, and the k range of either kind of tile may be split in two or more
 * parts, as a cost model of the launch picks (at most 512 MiB of partial sums). Split
 * tiles write fp32 partial sums to a device workspace that the library allocates per
 * (device, stream) at the first need and enlarges (at least doubling) when a launch
 * needs more; a final kernel adds the parts in a fixed order and rounds to bf16.
 * Nothing is ever freed or synchronized: an outgrown workspace is kept, unused, until
 * the process ends, so a graph captured earlier still owns valid memory. No workspace
 * is allocated or enlarged while the stream is being captured (the split is then
 * skipped, which changes the last bits), so call once with the largest shape before
 * capturing; a captured split launch uses the workspace the capturing stream had,
 * so replay such a graph only ordered with that stream's other work and with its own
 * other replays. Results are deterministic for a given shape and CU count. */
RFP4_API rfp4_status rfp4_gemm(const void* w, int layout, int64_t n, int64_t k, const void* a,
                      int64_t m, int64_t lda, void* c, int64_t ldc, void* stream);

/* Forcing a kernel or plan (tests and experiments). The default entry points choose
 * every kernel, lane mapping, split and tiling themselves; the _ex variants below take
 * an rfp4_force that overrides some of those choices. NULL, or a zero-filled struct,
 * gives exactly the default entry point's behaviour. Forcing changes only which
 * kernel runs and in which fp32 summation order, never what is computed. A field
 * outside its listed values gives RFP4_ERR_UNSUPPORTED before any HIP call. */
typedef enum rfp4_gemv_kernel {
  RFP4_GEMV_KERNEL_AUTO = 0,    /* the default choice */
  RFP4_GEMV_KERNEL_DOT = 1,     /* the dot-product kernel, at every batch */
  RFP4_GEMV_KERNEL_TILES = 2,   /* the matrix-core kernel of 16-row tiles, at every batch */
  RFP4_GEMV_KERNEL_TALL = 3,    /* the batch-1 tall matrix-core kernel wherever its shape
                                   rules allow (dual, f16, batch 1, k = 5120 or 6144, every
                                   matrix's rows a multiple of 16), else the default */
  RFP4_GEMV_KERNEL_NO_TALL = 4  /* the default choice without the tall kernel */
} rfp4_gemv_kernel;

typedef enum rfp4_gemm_plan {
  RFP4_GEMM_PLAN_AUTO = 0,     /* the cost model's choice */
  RFP4_GEMM_PLAN_MAIN = 1,     /* 256 x 256 tiles only, k unsplit */
  RFP4_GEMM_PLAN_MSPLIT2 = 2,  /* 256 x 256 tiles only, k split 2, 3 or 4 ways (fewer */
  RFP4_GEMM_PLAN_MSPLIT3 = 3,  /*   where k has too few 128-column steps) */
  RFP4_GEMM_PLAN_MSPLIT4 = 4,
  RFP4_GEMM_PLAN_TAIL = 5,     /* 128 x 128 tiles only, k unsplit, split 2 or 4 ways */
  RFP4_GEMM_PLAN_TAIL2 = 6,
  RFP4_GEMM_PLAN_TAIL4 = 7,
  RFP4_GEMM_PLAN_NOSPLIT = 8   /* the cost model's choice among plans without a k split */
} rfp4_gemm_plan;

typedef struct rfp4_force {
  int32_t gemv_kernel;         /* rfp4_gemv_kernel */
  int32_t gemv_unit_blocks;    /* dot-product kernel: consecutive blocks per lane unit, 1
                                  or 2, together with gemv_lanes_per_row; 0 = the default
                                  mapping (a pair mapping on an odd k / 32 is ignored) */
  int32_t gemv_lanes_per_row;  /* dot-product kernel: lanes per weight row, a power of two
                                  from 1 to 64 (0 with gemv_unit_blocks = 0) */
  int32_t gemv_splits;         /* tile kernel: parts of each tile's k range, 1 to 4
                                  (fewer where a row has fewer chunks; launches with two
                                  tiles per workgroup, batches above 4 on many rows, are
                                  not split); 0 = default */
  int32_t gemm_plan;           /* rfp4_gemm_plan */
  int32_t gemv_split_combine;  /* tile kernel with a split k range: 0 = the default (the
                                  last part polls, a bounded number of times, until the
                                  others have counted themselves, then adds all parts);
                                  1 = no polling: every part stores and counts itself
                                  and the part that counts last adds all parts (the
                                  default's fallback). Both add the parts in part order,
                                  so outputs are bitwise equal. */
} rfp4_force;

/* rfp4_gemv_multi with `force` (may be NULL); rfp4_gemv is count = 1. */
RFP4_API rfp4_status rfp4_gemv_multi_ex(int count, const void* const* w, const int64_t* n,
                                        int layout, int64_t k, const void* x, int xdtype,
                                        int64_t batch, int64_t ldx, float* const* y,
                                        const int64_t* ldy, const rfp4_force* force,
                                        void* stream);

/* rfp4_gemm with `force` (may be NULL). */
RFP4_API rfp4_status rfp4_gemm_ex(const void* w, int layout, int64_t n, int64_t k, const void* a,
                                  int64_t m, int64_t lda, void* c, int64_t ldc,
                                  const rfp4_force* force, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. rfp4_gemm_ex with the same arguments,
 * checks and result, except where its split plans keep their fp32 partial sums: in a
 * static device array of RFP4_GEMM_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends, not in a workspace. No call allocates, frees or
 * synchronizes anything. The cost model chooses among the plans whose partial sums fit
 * the array (where rfp4_gemm's plan fits, that is the same plan, and the outputs are
 * bit-identical); a forced plan (force->gemm_plan) that needs more is rejected with
 * RFP4_ERR_SCRATCH before any launch. Every call on one GPU shares that GPU's array and
 * leaves its contents behind (the partial sums are written before they are read, so
 * nothing needs clearing): calls that overlap in time on one GPU (other streams, other
 * threads, graph replays running concurrently) race on it and must be ordered by the
 * caller. The first call on a device looks up the array's device address (no
 * allocation). */
#define RFP4_GEMM_SCRATCH_BYTES (32u << 20)
RFP4_API rfp4_status rfp4_gemm_noalloc(const void* w, int layout, int64_t n, int64_t k,
                                       const void* a, int64_t m, int64_t lda, void* c,
                                       int64_t ldc, const rfp4_force* force, void* stream);

/* Dequantize-then-multiply prefill, the comparison baseline of rfp4_gemm ("Kernel
 * System" lists dequantize + dense GEMM beside the fused w4a16_gemm): W is expanded
 * to bf16 into the caller's buffer `wbuf` (n rows of ldw bf16 values, ldw >= k,
 * ldw % 8 == 0, 16-byte aligned; it holds rfp4_dequant_bf16's result afterwards) and
 * C = A W^T is computed by rocBLAS's dense bf16 GEMM (fp32 accumulation, bf16
 * output), on `stream`. Same arguments and checks as rfp4_gemm otherwise. rocBLAS is
 * loaded at the first call (RFP4_ERR_UNSUPPORTED if it cannot be); one rocBLAS handle
 * is kept per (device, stream), and rocBLAS may hold workspace memory of its own. */
RFP4_API rfp4_status rfp4_gemm_dequant(const void* w, int layout, int64_t n, int64_t k,
                                       const void* a, int64_t m, int64_t lda, void* c,
                                       int64_t ldc, uint16_t* wbuf, int64_t ldw, void* stream);

/* Quantization, the encoder that the converter of "Integration Options" (Option 2,
 * and Phase B of "The Automation Pipeline") needs in order to write 4-bit blocks.
 * The page defines only the decoder ("What is ROCmFP4?": Block Layout, Codebook10
 * Value Table, Scale Format), so the encoder is the plainest one that decoder
 * supports: for each scale group (16 weights dual, 32 fast) the scale byte is the
 * smallest b in 0..126 with 10 * S(b) >= max |w| (S the decoded scale; 126 when
 * none reaches, so the non-finite byte is never written), and each weight takes the
 * codebook entry nearest to w / S(b), ties to the smaller magnitude, with zero
 * always written as index 0. Every decision is an exact fp32 comparison, so the
 * result is deterministic bytes. A NaN or infinity makes its group saturate
 * (b = 126); NaN weights are written as index 0, infinities as +-10.
 * `src` holds n rows of k values of dtype src_dtype (RFP4_F32, RFP4_BF16 or
 * RFP4_F16) with a row stride of lds elements (lds >= k; src 16-byte aligned and
 * lds * element size a multiple of 16; n * lds <= 2^39). `w_out` receives
 * n * rfp4_row_bytes(layout, k) bytes, rows back to back (16-byte aligned; k need
 * only be a multiple of 32 here). */
RFP4_API rfp4_status rfp4_quantize(const void* src, int src_dtype, int64_t n, int64_t k,
                                   int64_t lds, int layout, void* w_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RFP4_H */
