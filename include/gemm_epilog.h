/*
 * gemm_epilog.h - C ABI of the fused GEMM + epilogue library for AMD Instinct MI355X (gfx950).
 *
 * One call computes D = epilogue(A . B) in a single HIP kernel: the bias add, the
 * activation, the ReLU mask or the masked bias gradient are applied to the fp32
 * accumulators before the only store of D.
 *
 * Sources (web pages describing the method):
 *  [P1] "Fusing bias addition via the nvmath-python epilog mechanism: parameter
 *       configuration and engineering practice guide" (blog.hotdry.top).
 *  [P2] "nvmath-python wraps cuBLASLt: low-overhead matmul and bias-fusion primitives
 *       for PyTorch" (blog.hotdry.top).
 *  [P3] "Fusing epilogs with matrix multiplication using nvmath-python" (itzkxy.com).
 *  [P4] "Dissecting nvmath-python: a seamless bridge between NumPy and cuBLASLt"
 *       (blog.hotdry.top).
 *  [P5] "Operator fusion in AI inference compilers: implementation and trade-offs"
 *       (mqxn.cn).
 *
 * Lifecycle ([P4] paragraph on the plan-execute-free lifecycle; [P2] body, plan and
 * execute steps; [P1] paragraph 4, second item): gemm_epilog_plan validates the
 * problem, picks a kernel configuration and allocates the plan's workspace once;
 * gemm_epilog_execute only enqueues work and may be called any number of times;
 * gemm_epilog_free releases the plan.
 *
 * Layouts. Every matrix is dense row-major with no leading-dimension padding:
 *   A (m, k), B (k, n), D (m, n). bias and bgrad hold m values, one per row of D:
 *   the bias has shape (m,) or (m, 1) and is added to every column ([P1] paragraph 2;
 *   [P2] body, initialisation example).
 *   The ReLU mask (aux) is uint32 words [ceil(m/32)][n], row-major: bit (i % 32) of
 *   word (i / 32, j) is 1 exactly when the pre-activation at (i, j) is > 0; bits of
 *   rows i >= m are 0. The pages keep this mask opaque ([P1] paragraph 3, [P3]
 *   section on the fused forward epilogs); this layout is the library's own.
 *
 * Arithmetic. Products are accumulated in fp32 whatever the storage type ([P2] body,
 * plan step: FP32 accumulator with FP16 inputs/outputs; [P5] section 4.3). Every
 * narrowing conversion rounds to nearest even. The order of the k reduction is the
 * kernel's own; results agree with a plain ascending-k fp32 sum to rounding.
 *
 * Ownership and threading. The caller owns every tensor pointer and the stream; the
 * plan owns only its workspace. A plan may be used from one stream at a time (its
 * workspace is shared between executes). All pointers passed to execute are device
 * pointers of the device that was current at plan time.
 *
 * Errors. Every argument check runs on the host before any HIP call, so invalid
 * arguments never launch a kernel. Faults inside a kernel surface at the caller's
 * next synchronisation, as for any asynchronous HIP work ([P1] paragraph 4, third
 * item: execute is asynchronous and the caller synchronises the stream).
 */
#ifndef GEMM_EPILOG_H_
#define GEMM_EPILOG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ge_plan* ge_handle_t; /* opaque; owned by the library */

/* Storage types. */
typedef enum { GE_F32 = 0, GE_F16 = 1, GE_BF16 = 2 } ge_dtype_t;

/* ab: type of A and B; d: type of D (must equal ab); vec: type of bias / bgrad
 * (equal to d, or GE_F32) - [P1] paragraph 4, first item: with fp16 A and B the
 * bias is fp16 or fp32. Accumulation is always fp32. */
typedef struct {
  ge_dtype_t ab;
  ge_dtype_t d;
  ge_dtype_t vec;
} ge_dtypes_t;

typedef enum {
  /* D = A.B (no epilogue); also the first kernel of the unfused chain. */
  GE_EPILOG_NONE = 0,
  /* D = max(A.B + bias, 0)  ([P2] body, plan step; [P3] section on the fused forward epilogs). */
  GE_EPILOG_RELU_BIAS = 1,
  /* D = gelu(A.B + bias), tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
   * ([P1] final paragraph and [P2] "other epilogs" paragraph name GELU_BIAS). */
  GE_EPILOG_GELU_BIAS = 2,
  /* RELU_BIAS that also writes the packed ReLU mask to aux ([P1] paragraph 3; [P3]
   * section on the fused forward epilogs). */
  GE_EPILOG_RELU_AUX_BIAS = 3,
  /* Backward: D = mask ? A.B : 0 using the mask in aux, and bgrad[i] = sum over j of
   * that masked fp32 product, before D's rounding ([P3] section "The DRELU_BGRAD path
   * in the backward pass"). No bias input. */
  GE_EPILOG_DRELU_BGRAD = 4,
  /* D = A.B + bias ([P1] paragraph 2). */
  GE_EPILOG_BIAS = 5,
  /* Measurement baseline: three kernels GEMM -> T1, T1 + bias -> T2, max(T2, 0) -> D,
   * with T1 and T2 in D's type held in the plan's workspace ([P5] section 2.2 diagram
   * of the chain before fusion). */
  GE_EPILOG_RELU_BIAS_UNFUSED = 100,
  /* Measurement baseline of the backward: the three steps DRELU_BGRAD does in one call
   * ([P3] section "The DRELU_BGRAD path in the backward pass"), each as its own kernel
   * as in [P5] section 2.2: GEMM -> T1 in D's type (held in the plan's workspace);
   * D = T1 where the forward activation in aux is > 0, else +0; bgrad[i] = the sum of
   * row i of the stored D. The unfused forward writes no bit mask, so aux holds its ReLU
   * output. No bias input. */
  GE_EPILOG_DRELU_BGRAD_UNFUSED = 101
} ge_epilog_t;

typedef enum {
  GE_OK = 0,
  GE_ERR_INVALID_VALUE = 1, /* m, n or k out of range; unknown enum value */
  GE_ERR_NOT_SUPPORTED = 2, /* dtype combination or shape outside the supported set */
  GE_ERR_NULL_POINTER = 3,  /* a pointer the epilogue needs is NULL */
  GE_ERR_MISALIGNED = 4,    /* a pointer violates its alignment rule */
  GE_ERR_ALLOC = 5,         /* host or device allocation failed in plan */
  GE_ERR_HIP = 6,           /* a HIP runtime call failed (launch, device query) */
  GE_ERR_SCRATCH = 7        /* gemm_epilog_execute_noalloc: the problem needs more workspace
                               than the static scratch holds */
} ge_status_t;

/*
 * gemm_epilog_plan - validate a problem and build its plan.
 *   m, n, k : problem sizes, 1 <= m <= 2^31 - 1, 1 <= n, k <= 2^20.
 *             n and k must be multiples of 8 for fp16/bf16 and of 4 for fp32
 *             (16-byte rows); otherwise GE_ERR_NOT_SUPPORTED. m is arbitrary.
 *   dt      : storage types (see ge_dtypes_t).
 *   ep      : epilogue.
 *   out     : receives the handle; untouched on error.
 * Allocates the workspace on the current device: the per-tile bias-gradient
 * partial sums for DRELU_BGRAD, T1 and T2 for RELU_BIAS_UNFUSED, T1 for
 * DRELU_BGRAD_UNFUSED, nothing otherwise.
 * Environment (tuning experiments): GE_TILE=S|M|L|LH|LM|LM4|LMD|L3|LW forces a tile configuration;
 * GE_GROUP_M=g (1..1024) sets how many m-tiles share one group of the tile order;
 * GE_STREAMK=0 keeps a sparse last round of tiles whole instead of splitting its k loop;
 * GE_SK_RUN=r sets the k-tiles per split run (at least one run per compute unit);
 * GE_PERSIST=0 launches one workgroup per tile instead of the persistent kernel;
 * GE_LOG=1 prints each plan's configuration and workspace size to stderr.
 */
ge_status_t gemm_epilog_plan(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep,
                             ge_handle_t* out);

/* Storage order of an operand ([P3] section "The DRELU_BGRAD path in the backward
 * pass", second paragraph: the backward's weight transpose and gradient layout must
 * match the matmul call; its FAQ: the rest of the backward pass, such as the weight
 * gradient, is outside DRELU_BGRAD). The product always uses A as (m, k) and B as
 * (k, n); GE_OP_T says the operand is passed as its transpose:
 *   op_a = GE_OP_T: the A pointer holds a row-major (k, m) matrix At, A[i][kk] = At[kk][i]
 *                   (e.g. dX = W^T . dY with W passed as stored);
 *   op_b = GE_OP_T: the B pointer holds a row-major (n, k) matrix Bt, B[kk][j] = Bt[j][kk]
 *                   (e.g. dW = dZ . X^T with X passed as stored). */
typedef enum { GE_OP_N = 0, GE_OP_T = 1 } ge_op_t;

/*
 * gemm_epilog_plan_ex - gemm_epilog_plan with the storage order of A and B.
 *   op_a, op_b : GE_OP_N or GE_OP_T (anything else: GE_ERR_INVALID_VALUE).
 * GE_OP_T needs fp16 or bf16 operands (fp32: GE_ERR_NOT_SUPPORTED). With op_a =
 * GE_OP_T, m follows the rules of n: a multiple of 8 and at most 2^20, else
 * GE_ERR_NOT_SUPPORTED. Every other argument, rule and error is that of
 * gemm_epilog_plan, which equals gemm_epilog_plan_ex(..., GE_OP_N, GE_OP_N, out).
 * Plans with a transposed operand run the 256 x 256 tile (the persistent kernel
 * included) and the 128 x 128 tiles with eight waves (LM, and LMD for a small grid
 * with 24 or more k-tiles), but never split their k loop; the 192 x 256, 128 x 256
 * and four-wave 128 x 128 tiles take untransposed operands only. GE_TILE may pick
 * L, LH, LM or LMD.
 */
ge_status_t gemm_epilog_plan_ex(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_op_t op_a,
                                ge_op_t op_b, ge_handle_t* out);

/*
 * gemm_epilog_execute - enqueue the planned computation on `stream` and return.
 *   A, B   : device inputs (m,k) and (k,n), type dt.ab, 16-byte aligned; (k,m) for A
 *            and (n,k) for B when the plan was made with op_a / op_b = GE_OP_T.
 *   bias   : device, m values of type dt.vec, aligned to its element size.
 *            Read by BIAS, RELU_BIAS, GELU_BIAS, RELU_AUX_BIAS, RELU_BIAS_UNFUSED;
 *            ignored (may be NULL) otherwise.
 *   D      : device output (m,n), type dt.d, 16-byte aligned.
 *   aux    : device mask words, gemm_epilog_aux_bytes(m,n) bytes, 16-byte aligned.
 *            Written by RELU_AUX_BIAS, read by DRELU_BGRAD, ignored otherwise.
 *            For DRELU_BGRAD_UNFUSED instead the forward activation, (m,n) of type
 *            dt.d, 16-byte aligned, read.
 *   bgrad  : device output, m values of type dt.vec, aligned to its element size.
 *            Written by DRELU_BGRAD and DRELU_BGRAD_UNFUSED, ignored otherwise.
 *   stream : a hipStream_t; NULL means the null stream.
 * Every output element in range is written; nothing outside the stated extents is.
 * Returns GE_ERR_HIP if a launch fails.
 * An execute enqueues kernel launches only (no memset, no host synchronisation), so it
 * may be captured into a HIP graph and replayed; replays of one plan must not overlap,
 * as for any two executes of a plan.
 */
ge_status_t gemm_epilog_execute(ge_handle_t h, const void* A, const void* B, const void* bias, void* D,
                                void* aux, void* bgrad, void* stream);

/*
 * gemm_epilog_autotune - time the kernel configurations that can run this plan on the
 * caller's own operands and keep the fastest in the plan. The plan's configuration
 * comes from a fixed per-shape table; this is the measured search that [P1] (final
 * paragraph: hand tuning through the algorithm heuristic) and [P2] (body, plan step:
 * the plan picks the best algorithm for the problem) describe. It runs on the real
 * data because the matrix cores' clock under the power limit depends on the values.
 *   h, A, B, bias, D, aux, bgrad, stream : as for gemm_epilog_execute (same rules and
 *            errors, checked first). D, aux and bgrad are written: on return they hold
 *            what one execute of the chosen configuration writes.
 *   repeats : timed executes per candidate, 1..1000 (else GE_ERR_INVALID_VALUE), each
 *            candidate after one untimed execute.
 *   best_ms : optional (may be NULL): receives the chosen configuration's mean time per
 *            execute in milliseconds, from HIP events on `stream`.
 * Candidates: for fp32 the 64x64 and 128x128 tiles; for fp16/bf16 with transposed
 * operands the 256x256 and 128x128 lockstep tiles (the latter with a 2- and a 3-stage
 * ring); otherwise the 256x256 tile (persistent, and one workgroup per tile with the
 * fragment reads interleaved into the MFMAs or issued in blocks), the 192x256 and 128x256
 * tiles (persistent) and the 128x128 tile with eight waves (2- or 3-stage ring) or four,
 * each with and without the split tail where it applies. A candidate whose
 * workspace cannot be allocated is skipped. The call synchronises `stream`, must
 * not overlap another execute of this plan, and runs on the device current at plan
 * time. On an error the plan keeps its configuration (GE_ERR_HIP if a launch or an
 * event call failed).
 */
ge_status_t gemm_epilog_autotune(ge_handle_t h, const void* A, const void* B, const void* bias, void* D, void* aux,
                                 void* bgrad, void* stream, int repeats, float* best_ms);

/* What a plan decides, as reported by gemm_epilog_plan_info. */
typedef struct {
  int tile_m, tile_n, tile_k;  /* workgroup tile and k-tile (tile_k 0: register-staged kernel) */
  int waves;                   /* waves per workgroup */
  int64_t tiles;               /* output tiles */
  int persistent_workgroups;   /* > 0: that many workgroups walk the tiles; 0: one per tile */
  int whole_tiles;             /* tiles computed whole (== tiles unless the last round is split) */
  int split_workgroups;        /* workgroups sharing the k loops of the remaining tiles */
  int split_run_ktiles;        /* k-tiles per split workgroup */
  int group_m;                 /* m-tiles per group of the tile order */
  size_t workspace_bytes;      /* device workspace the plan allocates */
  int stages;                  /* LDS stages of the operand ring (0: register-staged kernel) */
} ge_plan_info_t;

/*
 * gemm_epilog_plan_info - the configuration gemm_epilog_plan_ex would choose for this
 * problem on a gfx950 device with `compute_units` compute units, computed on the host
 * with no HIP call and no allocation (no device needed). The plan step of [P2] (body:
 * the costly choices are made once, when planning), exposed for inspection.
 *   m .. op_b      : as for gemm_epilog_plan_ex, same rules and errors.
 *   compute_units  : 1 .. 4096 (else GE_ERR_INVALID_VALUE); 256 on MI355X.
 *   info           : receives the decisions (GE_ERR_NULL_POINTER if NULL).
 * Honours the same environment switches as gemm_epilog_plan.
 */
ge_status_t gemm_epilog_plan_info(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep, ge_op_t op_a,
                                  ge_op_t op_b, int compute_units, ge_plan_info_t* info);

/*
 * gemm_epilog_lost_waits - how many split-tail waits of this plan's executes ran out
 * since the plan was made or since the last call, and reset the count.
 * A plan whose last round of tiles is split hands parts of a tile's k loop to other
 * workgroups; the workgroup that finishes the tile waits, bounded (about a second),
 * for their partial sums. A wait that runs out gives that tile NaN in D instead of
 * hanging the device, and leaves the plan's flags clean for later executes. The waits
 * end once the workgroups they wait for are scheduled, which a split plan's grid alone
 * always allows (its split workgroups fit the device at once); kernels of other streams
 * that keep compute units busy for longer than the bound (a second split plan's waiting
 * workgroups among them) can make a wait run out, so callers that run split plans
 * concurrently should check this count. This call
 * synchronises `stream` (hipStream_t, NULL = null stream), reads the count from the
 * plan's workspace and clears it; a plan without a split tail reports 0 at once.
 *   h     : the plan (GE_ERR_NULL_POINTER if NULL).
 *   count : receives the count (GE_ERR_NULL_POINTER if NULL).
 * GE_ERR_HIP if a copy or the synchronisation fails. Must not overlap an execute of h.
 */
ge_status_t gemm_epilog_lost_waits(ge_handle_t h, void* stream, uint32_t* count);

/* Bytes of the static device scratch that gemm_epilog_execute_noalloc works in. */
#define GEMM_EPILOG_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gemm_epilog_execute_noalloc - gemm_epilog_plan_ex and gemm_epilog_execute in one call
 * that allocates nothing: for callers that cannot allocate device memory, such as code
 * under HIP graph capture, tight serving loops and harnesses that forbid hipMalloc.
 * The plan's decisions are made on the host (as gemm_epilog_plan_info reports them) and
 * the kernels of gemm_epilog_execute run with their workspace (bias-gradient partial
 * sums, the unfused chains' T1 and T2, the split tail's partials and flags) in a static
 * device array of GEMM_EPILOG_NOALLOC_SCRATCH_BYTES (64 MiB) per device, which each GPU
 * the library runs on holds until the process ends. No hipMalloc, hipFree or other
 * allocating call is made; the first call on a device takes the array's address once
 * (hipGetSymbolAddress) and clears its flag words with a kernel on `stream`.
 *   m .. op_b : as for gemm_epilog_plan_ex, same rules and errors.
 *   A .. stream : as for gemm_epilog_execute, same rules and errors.
 * Returns GE_ERR_SCRATCH when the workspace does not fit the scratch even without the
 * split tail (e.g. DRELU_BGRAD with ceil(n/64) * m * 4 bytes of partial sums above
 * 64 MiB, the unfused chain with 2 m n element bytes above it, or the unfused backward
 * with m n element bytes above it); nothing is launched
 * then. A split tail that does not fit is left out (the tiles run whole).
 * Every call on a device shares that device's array, and the array keeps the last
 * call's contents: calls that overlap on one device (two streams, two threads) race and
 * give wrong results; calls on one stream are ordered and safe. A split-tail wait that
 * runs out gives its tile NaN in D, as for gemm_epilog_execute.
 */
ge_status_t gemm_epilog_execute_noalloc(int64_t m, int64_t n, int64_t k, ge_dtypes_t dt, ge_epilog_t ep,
                                        ge_op_t op_a, ge_op_t op_b, const void* A, const void* B, const void* bias,
                                        void* D, void* aux, void* bgrad, void* stream);

/* gemm_epilog_free - release a plan and its workspace. NULL is accepted (GE_OK).
 * Must not be called while an execute on this plan may still be running. */
ge_status_t gemm_epilog_free(ge_handle_t h);

/* Bytes of the ReLU mask for an (m, n) output: 4 * ceil(m/32) * n (0 if m or n < 1). */
size_t gemm_epilog_aux_bytes(int64_t m, int64_t n);

/* Bytes of device workspace held by a plan (0 for NULL). */
size_t gemm_epilog_workspace_bytes(ge_handle_t h);

/* Human-readable name of the kernel configuration a plan chose, e.g.
 * "f16 RELU_BIAS tile 256x256 waves 2x2". Valid while the plan lives; "" for NULL. */
const char* gemm_epilog_describe(ge_handle_t h);

/* Static string for a status code. */
const char* gemm_epilog_status_string(ge_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPILOG_H_ */
