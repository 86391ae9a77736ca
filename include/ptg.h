/*
 * ptg.h - C ABI of the pipelined tiled GEMM library for AMD Instinct MI355X (gfx950).
 *
 * The library computes the tiled matrix product of the standard Triton matmul in
 * "How We Built TLX: A Hardware-Native GPU Compiler for Production ML at Scale"
 * (section "Introducing TLX", listing 1: C = A.B with an fp32 accumulator), organised as
 * the producer / consumer / epilogue pipeline of listing 2 of the same section, and two
 * production forms of it from that page: the grouped GEMM of mixture-of-experts layers
 * (section "Case Study 3: Distributed Grouped GEMM for LLM Pretraining") and the
 * in-kernel broadcast linear compression (section "Case Study 2: In-Kernel Broadcast
 * Optimization for RecSys", subsection "TLX Provides a Building Block for the Final Stage
 * of This Optimization").
 *
 * Conventions shared by every call
 *   - Element types: every A, B, X, W operand is bfloat16 (raw 16-bit storage).  Outputs
 *     are float32 or bfloat16 (round to nearest, ties to even).  Products accumulate in
 *     float32.  Bias vectors are float32.
 *   - Layouts: matrices are row-major with a leading dimension (elements between rows).
 *     The second operand is either "KN" (K x N row-major, the plain B of C = A.B) or "NK"
 *     (N x K row-major, i.e. B transposed).
 *   - Memory: every matrix/vector pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates device memory, and never frees or retains a caller's pointer
 *     past the call's completion on the stream.  Host pointers are only the ptg_problem
 *     arrays, read during the call.  Scratch memory is supplied by the caller (see the
 *     *_workspace queries).
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *     call only enqueues work and returns; results are ready when the stream reaches them.
 *   - Alignment: device pointers must be 16-byte aligned, K and N multiples of 8 and
 *     leading dimensions multiples of 8 elements (16 bytes), else PTG_ERR_UNSUPPORTED.
 *   - Sizes: M = 0 or N = 0 is a valid no-op.  K = 0 is rejected (PTG_ERR_UNSUPPORTED).
 *     The kernels address one tile of every operand (256 rows), the output included, with
 *     31-bit byte offsets: a call whose operand or output tile would need more (for the
 *     output: ((255 * ldc + 256) * element size) >= 2^31) is rejected with
 *     PTG_ERR_UNSUPPORTED before anything runs.
 *   - Errors are returned, never thrown; ptg_last_error() holds a thread-local message for
 *     the last failing call on the calling thread.  Preconditions on device-resident data
 *     (group offsets, user indices) are not read by the host; violating them is undefined
 *     unless checked with the *_check helpers below.
 *   - Calls are reentrant and may run on several streams and threads at once.  State kept
 *     between calls: the per-thread error text, a per-device cache of device properties,
 *     the watchdog words (see ptg_watchdog), the *_check helpers' result words (one per
 *     check in flight, handed out under a lock) and the pinned host staging buffers of
 *     ptg_grouped_gemm_ptr_array (see there).
 *   - Kernel-side faults: every pipeline wait is bounded and every address range is
 *     checked on the device; a launch that trips one finishes without hanging, sets a
 *     watchdog bit and leaves its output incomplete.  The enqueueing call has already
 *     returned PTG_OK by then: ptg_watchdog() reports it, and the *_check helpers return
 *     PTG_ERR_DEVICE_CHECK while the current device's watchdog word is nonzero.
 *   - Debug switches, read from the environment at every call (set and not "0" turns one
 *     on).  PTG_LOG: each launch prints its entry point, shape and tile configuration to
 *     stderr.  PTG_CHECK: the calls whose inputs include device-resident bookkeeping
 *     (ptg_grouped_gemm, ptg_grouped_gemm_split and ptg_grouped_gemm_wgrad: group offsets;
 *     ptg_ikbo_attention: user offsets; the ptg_broadcast_gemm family: user indices) first
 *     run the matching *_check helper, which synchronises the stream, and return its error
 *     (PTG_ERR_DEVICE_CHECK) instead of launching.  Both are for debugging: PTG_CHECK makes
 *     those calls wait for the stream.
 */
#ifndef PTG_H_
#define PTG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PTG_OK = 0,
    PTG_ERR_INVALID_ARG = 1,   /* null pointer with nonzero extent, negative size, ld too small */
    PTG_ERR_UNSUPPORTED = 2,   /* alignment, K or N not a multiple of 8, size limits, bad enum */
    PTG_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace query */
    PTG_ERR_HIP = 4,           /* a HIP runtime call failed (launch error, bad stream, no device) */
    PTG_ERR_DEVICE_CHECK = 5   /* a *_check helper found invalid device-resident data */
} ptg_status;

typedef enum { PTG_BF16 = 0, PTG_F32 = 1 } ptg_dtype;               /* output element type */
typedef enum { PTG_B_KN = 0, PTG_B_NK = 1 } ptg_layout;             /* second-operand layout */
typedef enum {
    PTG_EPI_NONE = 0,       /* out = acc */
    PTG_EPI_BIAS = 1,       /* out = acc + bias[n] */
    PTG_EPI_SILU = 2,       /* out = silu(acc),         silu(v) = v / (1 + exp(-v)) */
    PTG_EPI_BIAS_SILU = 3   /* out = silu(acc + bias[n]) */
} ptg_epilogue;

/*
 * ptg_gemm - C = epi(A.B + bias), one pipelined persistent launch.
 * The operation of listing 1 ("Introducing TLX": acc = 0; for each K block acc += A.B;
 * store), with the epilogue stage of listing 2 extended by a fused bias and SiLU.
 *   M, N, K   problem size (M, N >= 0; K > 0; N, K multiples of 8)
 *   A         bf16 [M x K], row stride lda >= K
 *   B         bf16, [K x N] with row stride ldb >= N (PTG_B_KN) or [N x K] with ldb >= K (PTG_B_NK)
 *   C         [M x N] of c_dtype, row stride ldc >= N; fully overwritten, never read
 *   bias      float32 [N], required by the BIAS epilogues, ignored otherwise (may be NULL)
 */
ptg_status ptg_gemm(int64_t M, int64_t N, int64_t K,
                    const void* A, int64_t lda,
                    const void* B, int64_t ldb, ptg_layout b_layout,
                    void* C, int64_t ldc, ptg_dtype c_dtype,
                    const float* bias, ptg_epilogue epi, void* stream);

/*
 * ptg_grouped_gemm - mixture-of-experts grouped GEMM ("Case Study 3: Distributed Grouped GEMM
 * for LLM Pretraining": the grouped matrix products of the experts).  Rows of X and Y are
 * sorted by expert; expert g owns rows [offsets[g], offsets[g+1]) and multiplies W_g:
 *   Y[r] = epi(X[r] . W_g + bias[g])
 *   G             number of experts, 1 <= G <= 1024
 *   M_total, N, K X is bf16 [M_total x K] dense (ld = K); Y is [M_total x N] dense (ld = N)
 *   W             bf16, G matrices back to back: [G x K x N] (PTG_B_KN) or [G x N x K] (PTG_B_NK)
 *   group_offsets DEVICE int32 [G + 1]: offsets[0] = 0, nondecreasing, offsets[G] = M_total.
 *                 Empty groups are allowed.  Read only on the device (no host sync).
 *   bias          float32 [G x N] for the BIAS epilogues, else ignored
 * Rows of Y that belong to no group cannot exist under the precondition; every row is written.
 */
ptg_status ptg_grouped_gemm(int32_t G, int64_t M_total, int64_t N, int64_t K,
                            const void* X, const void* W, ptg_layout w_layout,
                            const int32_t* group_offsets,
                            void* Y, ptg_dtype y_dtype,
                            const float* bias, ptg_epilogue epi, void* stream);

/*
 * ptg_grouped_gemm_split - ptg_grouped_gemm with a workspace that lets the last round of tiles
 * use otherwise idle workgroups: when that round fills at most half the workgroups, each of its
 * tiles runs as two units, a full tile by columns (128 each), any other tile by reduction (each
 * unit takes half of the k-steps; the two fp32 partial sums are added in the workspace by the
 * unit that finishes second, which then runs the epilogue).  Same arguments, results and
 * errors as ptg_grouped_gemm, plus:
 *   workspace  DEVICE, 16-byte aligned, ws_bytes >= ptg_grouped_gemm_split_workspace() (for the
 *              current device: a 128-byte sync block and a 256 KB partial image per possible
 *              split tile, half the device's compute units; 32 MiB and 16 KiB on a 256-CU
 *              MI355X).  Its content on entry does not matter and needs no clearing: the sync
 *              words carry a per-call epoch.  Calls that run at the same time must not share it.
 * A tile split by reduction sums its two halves of k separately, so its elements may differ
 * from ptg_grouped_gemm's in the last bits (the same fp32 accumulation tolerance holds); the
 * result does not depend on which unit finishes first.
 * ptg_grouped_gemm_split_workspace returns 0 when no device is available.
 */
size_t ptg_grouped_gemm_split_workspace(void);
ptg_status ptg_grouped_gemm_split(int32_t G, int64_t M_total, int64_t N, int64_t K,
                                  const void* X, const void* W, ptg_layout w_layout,
                                  const int32_t* group_offsets,
                                  void* Y, ptg_dtype y_dtype,
                                  const float* bias, ptg_epilogue epi,
                                  void* workspace, size_t ws_bytes, void* stream);

/* ptg_grouped_gemm_check - validates group_offsets on the device (offsets[0] = 0,
 * nondecreasing, offsets[G] = M_total), synchronises `stream`, and returns PTG_OK, or
 * PTG_ERR_DEVICE_CHECK when the offsets break the precondition or the device's watchdog
 * word is set (a fault of an earlier launch).  Checks on different streams or threads run
 * concurrently, each with a result word of its own; up to 256 may be in flight at once
 * (beyond that PTG_ERR_UNSUPPORTED). */
ptg_status ptg_grouped_gemm_check(int32_t G, int64_t M_total, const int32_t* group_offsets,
                                  void* stream);

/*
 * ptg_grouped_gemm_wgrad - weight gradient of the grouped GEMM above, the second matrix
 * product of its backward pass (same case study; the input gradient dX_g = dY_g . W_g^T is
 * ptg_grouped_gemm with the forward's K x N weights passed as PTG_B_NK, N and K swapped):
 *   dW[g] = X_g^T . dY_g,  X_g and dY_g the rows [offsets[g], offsets[g+1]) of X and dY
 *   G             number of experts, 1 <= G <= 1024
 *   M_total, K, N X is bf16 [M_total x K] dense (ld = K); dY is bf16 [M_total x N] dense
 *                 (ld = N); K and N multiples of 8; M_total >= 0 (any value: the reduction
 *                 length of expert g is its row count, which need not be a multiple of 8)
 *   group_offsets DEVICE int32 [G + 1], same precondition as ptg_grouped_gemm
 *   dW            [G x K x N] of dw_dtype, dense; fully overwritten, never read.  An expert
 *                 without rows gets dW[g] = 0 (also when M_total = 0; X and dY may then be NULL).
 *   workspace     DEVICE, 16-byte aligned, ws_bytes >= ptg_grouped_gemm_wgrad_workspace()
 *                 (256): the queue from which the persistent workgroups take tiles.  Owned by
 *                 the caller; its content on entry does not matter (the call resets it on
 *                 `stream` first).  Calls that run at the same time must not share one.
 * Errors: as ptg_grouped_gemm (no epilogue, no bias), plus PTG_ERR_WORKSPACE.  Accumulation is
 * fp32 over the expert's rows; the result is not added to dW's previous content.
 */
size_t ptg_grouped_gemm_wgrad_workspace(void);
ptg_status ptg_grouped_gemm_wgrad(int32_t G, int64_t M_total, int64_t K, int64_t N,
                                  const void* X, const void* dY, const int32_t* group_offsets,
                                  void* dW, ptg_dtype dw_dtype, void* workspace, size_t ws_bytes,
                                  void* stream);

/*
 * ptg_ikbo_attention - the attention form of the in-kernel broadcast ("Case Study 2: In-Kernel
 * Broadcast Optimization for RecSys": for FlashAttention, the K/V reads are amortised across
 * the candidates that share one user context).  Candidates are sorted by user; user u owns
 * candidates [user_offsets[u], user_offsets[u+1]).  For candidate c of user u and head h:
 *   O[c][h] = softmax_j(scale * Q[c][h] . K[u][j][h]) . V[u][j][h]   (j = 0 .. L-1, no mask)
 *   U             users, 1 <= U <= 1024
 *   Mc            candidates (rows of Q and O), >= 0
 *   H, D          heads and head dimension; D must be 128
 *   L             keys per user context, a positive multiple of 64
 *   scale         finite score scale (1/sqrt(D) for the usual attention)
 *   Q             bf16 [Mc x H x D] dense
 *   K, V          bf16 [U x L x H x D] dense
 *   user_offsets  DEVICE int32 [U + 1]: 0 first, nondecreasing, Mc last (empty users allowed);
 *                 ptg_grouped_gemm_check(U, Mc, user_offsets, stream) validates it
 *   O             [Mc x H x D] of o_dtype, fully overwritten
 * Softmax in fp32 (running maximum and sum over 64-key blocks), products in bf16 MFMAs with
 * fp32 accumulation.  Errors as ptg_gemm; PTG_ERR_UNSUPPORTED for D != 128 or L % 64 != 0.
 */
ptg_status ptg_ikbo_attention(int64_t U, int64_t Mc, int64_t H, int64_t D, int64_t L, float scale,
                              const void* Q, const void* K, const void* V,
                              const int32_t* user_offsets, void* O, ptg_dtype o_dtype, void* stream);

/*
 * Pointer-array grouped GEMM: independent problems, each with its own pointers, shapes and
 * leading dimensions, in one persistent launch ("Case Study 3: Distributed Grouped GEMM for
 * LLM Pretraining": grouped matrix products; "Case Study 2", final stage of the linear-
 * compression kernel: short problems keep the pipeline full across problem boundaries).
 * Problem p computes C_p = epi(A_p . B_p + bias_p), B_p stored K x N (KN).
 *   ptg_grouped_gemm_ptr_array_workspace(count) - bytes of DEVICE workspace for `count`
 *       problems (0 for count <= 0): a 256-byte header, the tile prefix and 80 bytes per problem.
 *   ptg_grouped_gemm_ptr_array(count, problems, c_dtype, epi, workspace, ws_bytes, stream) -
 *       validates the HOST array `problems` (1 <= count <= 2048), writes the problem table into
 *       `workspace` with an asynchronous copy on `stream`, and launches the batch after it.
 *       `problems` may be freed or reused as soon as the call returns: the table is staged in a
 *       pinned host buffer of the library's own (a small per-device pool, allocated on first
 *       use and kept until exit; a buffer is reused once the copy that read it has completed,
 *       and the call waits on the host only if every buffer of the pool is still in flight).
 *       There is no host synchronisation of `stream`.  Each C_p must be of `c_dtype`.
 *   ptg_grouped_gemm_ptr_array_prepare / _run - the same call in two halves, so that a table
 *       written once can be launched many times: prepare validates and writes the table (it
 *       records c_dtype and epi in the table); run launches the batch recorded in `workspace`
 *       and does no host work.  run with a c_dtype, epi or count that differs from the
 *       table's is refused on the device: the kernel compares them with the table header
 *       before it touches any operand, writes nothing, and sets watchdog bit 2.
 * The table lists the problems with the longest reductions first (stable otherwise), so the
 * launch ends on its cheapest tiles; the order of execution is not observable, since every
 * problem writes only its own C_p.  Rewrite the table whenever a pointer or shape changes.
 * Calls that run at the same time must not share a workspace.
 * Errors: per problem as ptg_gemm (the failing problem's index is in ptg_last_error), plus
 * PTG_ERR_WORKSPACE; PTG_ERR_UNSUPPORTED also when a problem's output tile of 256 rows
 * cannot be addressed with 31-bit byte offsets (((255 * ldc + 256) * element size) >= 2^31).
 */
typedef struct {
    int64_t M, N, K;          /* M >= 0, N and K multiples of 8, K > 0 */
    const void* A;            /* bf16 [M x K], row stride lda */
    const void* B;            /* bf16 [K x N], row stride ldb (KN layout) */
    void* C;                  /* [M x N] of the call's c_dtype, row stride ldc */
    const float* bias;        /* float32 [N] (BIAS epilogues) or NULL */
    int64_t lda, ldb, ldc;
} ptg_problem;

size_t ptg_grouped_gemm_ptr_array_workspace(int32_t count);
ptg_status ptg_grouped_gemm_ptr_array(int32_t count, const ptg_problem* problems, ptg_dtype c_dtype,
                                      ptg_epilogue epi, void* workspace, size_t ws_bytes, void* stream);
ptg_status ptg_grouped_gemm_ptr_array_prepare(int32_t count, const ptg_problem* problems, ptg_dtype c_dtype,
                                              ptg_epilogue epi, void* workspace, size_t ws_bytes, void* stream);
ptg_status ptg_grouped_gemm_ptr_array_run(int32_t count, const void* workspace, size_t ws_bytes,
                                          ptg_dtype c_dtype, ptg_epilogue epi, void* stream);

/*
 * ptg_broadcast_gemm - in-kernel broadcast linear compression ("Case Study 2: In-Kernel
 * Broadcast Optimization for RecSys"): user features are consumed at their natural batch
 * size U, candidate features at Mc, and the broadcast happens inside the computation:
 *   Y[r] = epi([Xu[user_idx[r]] | Xc[r]] . W + bias)
 * computed by matmul decomposition: P = Xu . W[0:Ku] once per user (fp32, in `workspace`),
 * then Y = epi(Xc . W[Ku:Ku+Kc] + P[user_idx] + bias); Xu[user_idx] is never materialised.
 *   U, Mc         users and candidates (U >= 1, Mc >= 0)
 *   Ku, Kc, N     user width, candidate width, output width (multiples of 8; Ku, Kc > 0)
 *   Xu            bf16 [U x Ku] dense;  Xc bf16 [Mc x Kc] dense
 *   user_idx      DEVICE int32 [Mc], each in [0, U); any order
 *   W             bf16 [(Ku + Kc) x N] (PTG_B_KN, rows 0..Ku-1 meet the user features) or
 *                 [N x (Ku + Kc)] (PTG_B_NK, columns 0..Ku-1 meet the user features)
 *   Y             [Mc x N] of y_dtype, dense
 *   bias          float32 [N] for the BIAS epilogues
 *   workspace     DEVICE scratch of at least ptg_broadcast_gemm_workspace(U, N) bytes
 * The user product is small (U rows), so it is split along Ku into up to 32 slices that run
 * side by side; their fp32 partial products go to the workspace after P and are summed in
 * slice order (results do not depend on timing).  The workspace query returns
 * U * N * 4 * (1 + S) bytes, S the slice count for U x N (a function of U and N only, at most
 * 32; S = 1 needs no partials: U * N * 4 bytes).
 * Errors: as ptg_gemm, plus PTG_ERR_WORKSPACE; PTG_ERR_UNSUPPORTED also when U * N * 4 >= 2^31
 * (the gather addresses P with 31-bit byte offsets).
 */
size_t ptg_broadcast_gemm_workspace(int64_t U, int64_t N);
ptg_status ptg_broadcast_gemm(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N,
                              const void* Xu, const void* Xc, const int32_t* user_idx,
                              const void* W, ptg_layout w_layout,
                              void* Y, ptg_dtype y_dtype,
                              const float* bias, ptg_epilogue epi,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * ptg_broadcast_gemm_fused - ptg_broadcast_gemm as one persistent launch: the final form of the
 * linear compression in "How We Built TLX", Case Study 2, subsection "TLX Provides a Building
 * Block for the Final Stage of This Optimization", where the user and candidate products share
 * one pipeline instead of draining it between launches, with tile-level release and acquire
 * between workgroups.  Same arguments and results as ptg_broadcast_gemm (P summed over a
 * different number of slices: fp32 rounding may differ in the last bits); the workspace is
 * DEVICE scratch of at least ptg_broadcast_gemm_fused_workspace(U, N) bytes (16-byte aligned).
 * The launch runs, from one ticket counter, user units (slice s of Ku for one 256-column block,
 * each about half a candidate tile's k-steps; the fp32 partial product goes to the workspace and
 * each consumer wave then publishes this call's epoch in its arrival flag), reduction units
 * (the producer waves wait for every flag of their column block, sum the slices in order, add
 * the bias, write rows of P and count themselves into the block's ready word), then each
 * workgroup's candidate tiles in a fixed XCD-aware order (published to the consumers once their
 * column block's ready word is complete; the accumulators start from P).  Sync words carry the call's epoch (from a
 * process-wide counter), so the workspace needs no clearing between calls; calls that share
 * one workspace must not overlap.  Every wait is bounded (see ptg_watchdog).
 * Errors: as ptg_broadcast_gemm; PTG_ERR_UNSUPPORTED also unless U <= 256, Ku > 64 (two
 * 64-deep slices), N <= 130816 (the sync words' 4 KB block) and the workspace is under 2 GiB.
 * Measured on MI355X (64 users, 81,403 candidates, [2048 | 512] -> 1024, bf16): slower than
 * ptg_broadcast_gemm, because the candidates cannot start before P is complete (P is their
 * accumulators' start value).
 */
size_t ptg_broadcast_gemm_fused_workspace(int64_t U, int64_t N);
ptg_status ptg_broadcast_gemm_fused(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N,
                                    const void* Xu, const void* Xc, const int32_t* user_idx,
                                    const void* W, ptg_layout w_layout,
                                    void* Y, ptg_dtype y_dtype,
                                    const float* bias, ptg_epilogue epi,
                                    void* workspace, size_t ws_bytes, void* stream);

/*
 * ptg_broadcast_gemm_noalloc - ptg_broadcast_gemm for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and errors as ptg_broadcast_gemm, without the workspace: P and the
 * user phase's partial products live in a file-scope device array of the library, 16 MiB per
 * GPU (16,777,216 bytes), held until the process ends.  A call whose workspace query
 * ptg_broadcast_gemm_workspace(U, N) exceeds 16 MiB is refused with PTG_ERR_UNSUPPORTED.  The
 * call allocates nothing (no hipMalloc, no allocating library routine); on its first use on a
 * device it looks up that device's copy of the array.  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (every call overwrites what it reads, so
 * nothing needs clearing): calls that overlap on one GPU (on different streams, or from
 * different threads) race and must not be issued.
 */
ptg_status ptg_broadcast_gemm_noalloc(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N,
                                      const void* Xu, const void* Xc, const int32_t* user_idx,
                                      const void* W, ptg_layout w_layout,
                                      void* Y, ptg_dtype y_dtype,
                                      const float* bias, ptg_epilogue epi, void* stream);

/* ptg_broadcast_gemm_check - validates 0 <= user_idx[r] < U on the device, synchronises
 * `stream`, returns PTG_OK or PTG_ERR_DEVICE_CHECK (also when the device's watchdog word is
 * set); concurrent as ptg_grouped_gemm_check. */
ptg_status ptg_broadcast_gemm_check(int64_t U, int64_t Mc, const int32_t* user_idx, void* stream);

/* Text of a status code (static storage), and the calling thread's last error detail. */
const char* ptg_status_string(ptg_status s);
const char* ptg_last_error(void);

/* ptg_watchdog - every wait of the pipeline is bounded; a wait that gives up (which a correct
 * launch never does) sets a per-device word instead of hanging.  Reads that word of the
 * current device into *value and clears it when `clear` is nonzero.  Synchronous. */
ptg_status ptg_watchdog(uint32_t* value, int32_t clear);

/* Library version, and the tile configuration the dense path would pick for (M, N, K):
 * writes BM, BN, BK, stages, consumer waves, producer waves into cfg[0..5].  Producer waves 0
 * marks the one-role kernel, whose waves both copy and compute (either B layout, K a multiple
 * of 32, and at least 128 tiles of 256 x 256 or more tiles of 128 x 128 than the device has
 * compute units).  For tests and logging; returns
 * PTG_ERR_INVALID_ARG for a NULL cfg. */
int32_t ptg_version(void);
ptg_status ptg_describe_config(int64_t M, int64_t N, int64_t K, ptg_layout b_layout, int32_t cfg[6]);

#ifdef __cplusplus
}
#endif

#endif /* PTG_H_ */
