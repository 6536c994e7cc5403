/*
 * lr_linear.h -- C ABI of the MI355X (gfx950) factorized linear layer.
 *
 * The operation
 * -------------
 * A linear layer Y = X.W whose weight has been replaced by two factors,
 * W ~ A.B, so that one large product becomes two thin ones that meet at the
 * rank r ("Why Smaller Is Slower? Dimensional Misalignment in Compressed
 * LLMs", section 1 and Figure 1).  The factor pair keeps the layer's
 * input/output interface: in the column-vector orientation of "LowRankArena:
 * What Happens When You Force SVD Compression Papers to Play by the Same
 * Rules" (Prerequisites, Figure A) y = Wx becomes y = A(Bx).  Here, row-major:
 *
 *     X[M x K] . A[K x r] = T[M x r],     T . B[r x N] = Y[M x N]
 *
 * r and N may take any value >= 1 (r = 107, 1637, 2867, N = 3999 ...):
 * the kernels pad the rank and mask the N edge on chip, so no shape falls
 * back to a slower kernel tier (the tiers and penalties that the
 * misalignment page measures in section 3.2 and Tables 3-4).
 *
 * Data types and layout
 * ---------------------
 * All matrices are bfloat16, row-major, dense (leading dimension = number
 * of columns).  Base pointers must be 16-byte aligned (any allocation made
 * by hipMalloc or torch is); rows may start at any 2-byte boundary.
 * Arithmetic: bf16 inputs, fp32 accumulation, bf16 output rounded to
 * nearest-even.  All pointers passed here are DEVICE pointers.
 *
 * Ownership
 * ---------
 * A and B are BORROWED by the handle: the caller keeps them alive until
 * lr_linear_destroy.  By default every call reads them where they are
 * (decode and prefill alike), so an update of A or B in place between calls
 * is seen by the next call.  X and Y are borrowed for the duration of the enqueued
 * work.  The handle OWNS a device workspace (allocated at create, sized for
 * max_M) that holds the exchange tables of the decode kernels, split-K
 * partial sums, and for M > 16 the bf16 intermediate T; and a 64-byte
 * pinned host word in which a decode kernel reports a wait that gave up
 * (see Errors).  Two modes instead keep a derived copy of the factors in
 * the workspace, made at create and not refreshed afterwards, which every
 * call of the handle reads (an in-place update of A or B is then not seen):
 * the dense fallback's W = A.B (LR_FLAG_DENSE, or automatic, see
 * lr_linear_create; decode and prefill both read W), and the decode-only
 * LR_FLAG_DECODE_SPLIT, whose kernel reads A and B from a copy in its 1 KB
 * operand block layout: 2 (ceil(r/16) ceil(K/32) + ceil(N/16) ceil(r/32))
 * x 512 bytes, about the size of A and B (27.1 MB for K = N = 4096,
 * r = 1637).
 * lr_linear_destroy frees all of it.  Because the workspace is shared by
 * every call on a handle, a handle must not be used by two streams at the
 * same time.
 *
 * Semantics
 * ---------
 * Y is fully overwritten (no alpha/beta, no accumulation), exactly on its
 * M x N extent; no byte outside it is written.  Calls are asynchronous on
 * the given stream (a hipStream_t passed as void*; NULL = default stream):
 * the status reflects argument validation and kernel launch only.  Faults
 * inside kernels surface at the caller's next synchronization.
 *
 * Errors
 * ------
 * Functions return an lr_status and never abort, print or throw across the
 * ABI.  lr_last_error() returns a thread-local detail string for the most
 * recent failure on the calling thread.  The workgroups of a decode launch
 * wait on one another's partial results, which needs every workgroup of the
 * launch resident at once.  Create checks every launch the handle can make
 * against its kernel's occupancy (UNSUPPORTED if one cannot fit), and every
 * launch is checked again before it is enqueued.  Another kernel running
 * concurrently on the same GPU can still hold compute units: a wait then
 * gives up after a bounded number of polls (seconds) instead of hanging,
 * the launch ends normally with an invalid output, and the handle's next
 * lr_linear_run / lr_group_run / lr_mlp_packed_run, or lr_linear_status,
 * returns LR_ERR_HIP (once).
 */
#ifndef LR_LINEAR_H
#define LR_LINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lr_status {
    LR_OK = 0,
    LR_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned base, overlap */
    LR_ERR_UNSUPPORTED = 2,   /* no gfx950 device, or flags not understood */
    LR_ERR_OUT_OF_MEMORY = 3, /* workspace allocation failed */
    LR_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} lr_status;

/* Opaque handle: one factorized projection (A, B) and its workspace. */
typedef struct lr_linear lr_linear;

/* Flags for lr_linear_create. */
#define LR_FLAG_NONE          0u
#define LR_FLAG_FORCE_DECODE  1u  /* use the fused decode kernel for every M (requires max_M <= 16) */
#define LR_FLAG_FORCE_PREFILL 2u  /* use the MFMA prefill kernels for every M */
#define LR_FLAG_DECODE_STREAMING 4u  /* decode with the register-streaming kernel even where the
                                        role-split or LDS-resident one applies (all compute the
                                        same result) */
#define LR_FLAG_PREFILL_TWO_WAVE 8u  /* prefill only with the two-waves-per-SIMD kernel (tiles of
                                        256 x 192 or 224) instead of the cost model's choice */
#define LR_FLAG_PREFILL_ONE_WAVE 16u /* prefill with the one-wave-per-SIMD kernel (256 x 256 tiles)
                                        wherever it applies: rows of its left operand (X, or T)
                                        16-byte aligned, i.e. K a multiple of 8 for phase 1 */
#define LR_FLAG_DENSE    32u  /* dense fallback: form W = A.B (bf16) at create and run Y = X.W */
#define LR_FLAG_FACTORED 64u  /* never take the dense fallback */
#define LR_FLAG_DECODE_SPLIT 128u  /* decode with the role-split kernel where its plan fits; it
                                      reads a copy of A and B in its operand block layout, made at
                                      create (see Ownership).  Decode-only: max_M <= 16 and not
                                      with FORCE_PREFILL, so every call on the handle reads the
                                      same copy */
#define LR_FLAG_DECODE_RESIDENT 256u  /* decode with the LDS-resident kernel where it applies, else
                                         the register-streaming one (the default's choice too) */
#define LR_FLAG_DECODE_XCD 512u  /* decode with the XCD-sliced kernel where its plan fits: it reads
                                    A and B in place, one workgroup per compute unit, each XCD
                                    owning an eighth of the rank; gate/up or q/k/v handles that all
                                    carry this flag share one launch in lr_group_run */
#define LR_FLAG_TEST_STALL (1u << 30) /* for testing the error path only: the T hand-off wait of every
                                         decode launch expects a value that is never stored and gives
                                         up after 2048 polls, so each decode call's output is invalid
                                         and the next call reports LR_ERR_HIP */

/* Largest M that the fused decode kernel takes (more rows use prefill). */
#define LR_DECODE_MAX_M 16

/*
 * lr_linear_create -- build a handle for one factor pair.
 *   out    : receives the handle (set to NULL on failure).
 *   K, r, N: X has K columns, A is K x r, B is r x N; each >= 1.
 *   A, B   : device pointers to the bf16 factors (borrowed; 16-byte aligned).
 *   max_M  : largest M that lr_linear_run will be called with (>= 0).
 *   flags  : LR_FLAG_* bits.
 * Chooses the kernels' partitioning for this shape and allocates the
 * workspace on the current HIP device.  By default decode (M <= 16) reads
 * the caller's row-major A and B in place and pads the rank on chip: the
 * LDS-resident kernel where its slabs fit in LDS (rank slices of 128
 * columns; T partials added inside an XCD, Y partials across XCDs), else
 * the register-streaming kernel (rank slices of 120 columns).  No copy of
 * the factors is made.  LR_FLAG_DECODE_STREAMING, _RESIDENT, _XCD and
 * _SPLIT select a kernel explicitly; _SPLIT is the only one that reads a
 * copy (see Ownership), and is the fastest where the extra bytes are
 * acceptable.  A flag whose plan does not fit the shape falls back to the
 * default.  Create launches no kernel, except for LR_FLAG_DECODE_SPLIT and
 * for the dense fallback:
 * when LR_FLAG_DENSE is set, or (without LR_FLAG_FACTORED) when the factors
 * hold at least 95% of the bytes of the K x N matrix they replace, i.e.
 * 100 r (K + N) >= 95 K N ("LowRankArena: What Happens When You Force SVD
 * Compression Papers to Play by the Same Rules", Q3: a dense GEMM where the
 * retained rank saves no memory bandwidth), create forms W = A.B in bf16
 * (fp32 accumulation) with the prefill GEMM on the null stream, plus W in
 * the dense decode kernel's operand layout, and waits for them.  Runs then
 * compute Y = X.W: decode with one workgroup per 16 columns and no exchange
 * between workgroups, prefill with one GEMM.  W is a snapshot: A and B are
 * not read again.  The workspace then holds W (K x N bf16) when max_M > 16
 * and its decode layout when decode applies.
 * Errors: INVALID_ARG (null/size/alignment, exclusive flags together),
 * UNSUPPORTED (no gfx950 device, unknown flags, FORCE_DECODE with
 * max_M > 16, DENSE with a W above 2 GiB, a decode launch whose workgroups
 * cannot all be resident at once), OUT_OF_MEMORY, HIP.
 */
lr_status lr_linear_create(lr_linear** out, int64_t K, int64_t r, int64_t N,
                           const void* A, const void* B, int64_t max_M, uint32_t flags);

/*
 * lr_linear_run -- Y[M x N] = (X[M x K] . A) . B on `stream`.
 *   M in [0, max_M]; M == 0 returns LR_OK and launches nothing.
 * M <= 16: one fused launch (GEMM1, T handed between workgroups inside the
 * launch, GEMM2, deterministic reductions; T is never written as a tensor
 * for a second kernel).
 * M > 16: MFMA GEMM1 into a bf16 T workspace, then MFMA GEMM2.
 * Graph capture: a run only enqueues kernels, and its launch arguments do
 * not change from call to call (the decode kernels stamp their exchanges
 * with a generation word kept in the workspace), so runs, group runs and
 * packed runs may be captured into a HIP graph on `stream` and replayed
 * ("FlashSVD v1.5: Making Low-Rank Transformers Inference Actually Fast",
 * abstract: per-layer graph replay).  Make one call per handle before
 * capturing (the first call sets kernel attributes), and do not replay a
 * graph while another call on the same handle is in flight.
 * Errors: INVALID_ARG (null handle/pointers, M out of range, misaligned
 * base, Y overlapping X/A/B), HIP (launch failure; or a wait of an earlier
 * decode launch on this handle gave up, see Errors above: nothing is
 * launched and the report is cleared).
 */
lr_status lr_linear_run(const lr_linear* h, const void* X, void* Y, int64_t M, void* stream);

/*
 * lr_mlp_packed_run -- a gate/up pair that shares its input X
 * ("FlashSVD v1.5: Making Low-Rank Transformers Inference Actually Fast",
 * abstract: packed MLP execution).  Computes
 *     Y_gate = (X.A_gate).B_gate   and   Y_up = (X.A_up).B_up
 * as lr_group_run with n = 2 and handles {gate, up}: at M > 16 the tiles of
 * both GEMM1s are dealt over the CUs in one prefill launch (each workgroup
 * loads the X tile of its own output tile); at decode the two run in one
 * launch where the kernel allows it (see lr_group_run), the layer's gate
 * and up (register-streaming kernel) on each handle's half-machine plan.
 * gate and up must be distinct handles with equal K; their r and N may
 * differ.  M must not exceed either handle's max_M.  Y_gate and Y_up must
 * not overlap each other or any input.
 * Errors: as lr_linear_run, plus INVALID_ARG for gate.K != up.K or
 * gate == up.
 */
lr_status lr_mlp_packed_run(const lr_linear* gate, const lr_linear* up, const void* X,
                            void* Y_gate, void* Y_up, int64_t M, void* stream);

/* Most projections one lr_group_run call takes. */
#define LR_GROUP_MAX 4

/*
 * lr_group_run -- n projections that share their input X, such as the
 * q, k and v projections of an attention block (the packed execution of
 * "FlashSVD v1.5: Making Low-Rank Transformers Inference Actually Fast",
 * abstract, widened from the gate/up pair to any n <= LR_GROUP_MAX).
 * Computes Ys[i][M x N_i] = (X[M x K] . A_i) . B_i for i < n.
 *   hs : n distinct handles (host array of handle pointers) with equal K;
 *        r and N may differ.  Each owns its workspace, so no handle may
 *        appear twice.  The prefill kernel flags of hs[0] govern the call.
 *   X  : device pointer, bf16 [M x K] row-major, shared by every projection.
 *   Ys : host array of n device pointers, bf16 [M x N_i] row-major; no
 *        output may overlap X, another output or any handle's factors.
 *   M  : rows, in [0, min max_M]; M == 0 returns LR_OK and launches nothing.
 * Projections that take the dense fallback's decode at this M share one
 * launch; factorized projections that take a decode kernel share decode
 * launches where their kernel allows it: the resident and streaming
 * kernels while the workgroups of all fit the device at once (two
 * streaming projections that do not, such as a layer's gate and up, on
 * the second plan each handle holds for half the compute units), the
 * XCD-sliced kernel always (each projection takes a share of every XCD's
 * compute units), the role-split kernels never (each fills the device).
 * The others share one launch per prefill GEMM, in which every output's
 * tiles are dealt over the CUs together.  Results equal n lr_linear_run
 * calls up to the order of fp32 additions (bitwise for the dense and
 * role-split decodes, whose per-output work does not depend on the
 * group).
 * Errors: INVALID_ARG (null array, handle or pointer, n outside
 * [1, LR_GROUP_MAX], repeated handle, unequal K, M out of range,
 * misaligned base, overlapping output), HIP (launch failure).
 */
lr_status lr_group_run(const lr_linear* const* hs, int n, const void* X, void* const* Ys,
                       int64_t M, void* stream);

/*
 * lr_decode_noalloc -- Y[M x N] = (X[M x K] . A[K x r]) . B[r x N] for
 * M <= 16, with no handle and without allocating anything: for callers that
 * cannot call hipMalloc (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It runs the decode kernel that
 * lr_linear_create + lr_linear_run choose by default for max_M = M
 * (LDS-resident or register-streaming, reading A and B in place), with that
 * kernel's exchange tables in a fixed 64 MiB device array inside the
 * library instead of a handle's workspace.
 *   X, A, B, Y : device pointers, bf16 row-major, as for lr_linear_run
 *                (16-byte aligned bases; Y must not overlap the inputs).
 *   M          : rows, in [0, 16]; 0 returns LR_OK and launches nothing.
 *   status     : optional device pointer (4-byte aligned) to a word the
 *                caller owns and clears: a wait of the launch that gives up
 *                (see Errors) stores 1 there.  NULL: not reported.
 *   stream     : hipStream_t as void* (NULL = default stream).
 * Each call enqueues a small clearing kernel and the decode kernel; it
 * calls no hipMalloc, hipFree or other allocating routine.  Every call on a
 * GPU uses that GPU's one array, which keeps the last call's contents:
 * calls that overlap in time on one GPU (different streams, or threads)
 * race and give wrong results; calls in stream order are safe.  The array
 * is the device's for the life of the process.
 * Errors: INVALID_ARG (null pointer, sizes, misaligned base, overlap,
 * M > 16), UNSUPPORTED (a shape whose tables exceed the 64 MiB array, or
 * whose launch cannot be resident at once), HIP (launch failure).
 */
lr_status lr_decode_noalloc(const void* X, const void* A, const void* B, void* Y, int64_t M,
                            int64_t K, int64_t r, int64_t N, uint32_t* status, void* stream);

/*
 * lr_linear_status -- LR_ERR_HIP (once, with a detail in lr_last_error) if a
 * decode launch of this handle gave up waiting for another of its
 * workgroups since the last report (see Errors), else LR_OK.  Reads a pinned
 * host word and enqueues nothing; synchronize the stream first to include
 * the launches still in flight.  INVALID_ARG for a NULL handle.
 */
lr_status lr_linear_status(const lr_linear* h);

/* lr_linear_destroy -- free the workspace and the handle.  NULL is a no-op.
 * The caller must ensure no enqueued work still uses the handle. */
void lr_linear_destroy(lr_linear* h);

/* Static, human-readable name of a status code. */
const char* lr_status_str(lr_status s);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* lr_last_error(void);

/*
 * lr_linear_describe -- write a one-line description of the handle's plan
 * (shape, padded rank, partition, workspace bytes) into buf (NUL-terminated,
 * truncated to len).  Returns LR_ERR_INVALID_ARG for a NULL handle or buffer.
 */
lr_status lr_linear_describe(const lr_linear* h, char* buf, int64_t len);

/*
 * lr_linear_workspace_bytes -- device bytes the handle owns (0 for NULL).
 */
int64_t lr_linear_workspace_bytes(const lr_linear* h);

#ifdef __cplusplus
}
#endif

#endif /* LR_LINEAR_H */
