// ptg_launch.h - host-side launch descriptions shared by the C ABI layer and the kernels.
// Plain structs (no device code): the ABI layer fills them after validation, the launchers
// in ptg_kernels.hip pick a tile configuration and enqueue one persistent kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptg {

// One dense problem C = epi(A.B + bias [+ P[gidx[m]]]).
struct DenseLaunch {
  const void* A;
  const void* B;
  void* C;
  const float* bias;          // [N] or null
  const int32_t* gidx;        // [M] row -> row of P, or null (broadcast gather)
  const float* P;             // [p_rows x ldp] fp32, or null
  int64_t lda, ldb, ldc, ldp, p_rows;
  int64_t M, N, K;
  int b_kn;                   // 1: B is K x N; 0: B is N x K
  int epi;                    // ptg_epilogue value
  int out_f32;                // 1: float32 output; 0: bfloat16
  // Split-K (fp32 output only): split s covers k in [s * k_chunk, (s + 1) * k_chunk) and
  // writes its partial product to C + s * c_split elements.  splits = 1: the whole K.
  int32_t splits = 1;
  int64_t k_chunk = 0;
  int64_t c_split = 0;
};

struct GroupedLaunch {
  const void* X;
  const void* W;
  void* Y;
  const float* bias;          // [G x N] or null
  const int32_t* offsets;     // device [G + 1]
  int64_t M_total, N, K;
  int32_t G;
  int b_kn, epi, out_f32;
  // Optional workspace (grouped_split_workspace_bytes) for the reduction split of the last
  // round's tiles; null: no reduction split.  `epoch` is unique per launch.
  void* workspace = nullptr;
  size_t ws_bytes = 0;
  uint32_t epoch = 0;
};
// Workspace of the grouped GEMM's reduction split on a device with `cus` compute units:
// per split tile (at most cus / 2 of them) a 128-byte block of sync words and a 256 KB image
// of the partial accumulators (one 32 KB register image per consumer wave).
constexpr size_t kSplitSyncBytes = 128;
constexpr size_t kSplitImageBytes = 256 * 256 * 4;
inline size_t grouped_split_slots(int cus) { return (size_t)(cus > 1 ? cus / 2 : 1); }
inline size_t grouped_split_sync_bytes(int cus) {
  return (grouped_split_slots(cus) * kSplitSyncBytes + 4095) / 4096 * 4096;
}
inline size_t grouped_split_workspace_bytes(int cus) {
  return grouped_split_sync_bytes(cus) + grouped_split_slots(cus) * kSplitImageBytes;
}
int device_compute_units();

// Weight gradient of the grouped GEMM: dW[g] = X_g^T . dY_g over group g's rows.
struct WgradLaunch {
  const void* X;              // [M_total x K]
  const void* dY;             // [M_total x N]
  void* dW;                   // [G x K x N]
  const int32_t* offsets;     // device [G + 1]
  void* workspace;            // kWgradWorkspace bytes: the tile-queue counter
  int64_t M_total, K, N;
  int32_t G;
  int out_f32;
};
constexpr size_t kWgradWorkspace = 256;
// Device-side record of one problem of a batch (written by ptg_gemm_batch_prepare).
struct BatchProblem {
  const void* A;
  const void* B;
  void* C;
  const float* bias;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t pad;
};
static_assert(sizeof(BatchProblem) == 80, "BatchProblem layout");

// Address ranges [lo, hi) a kernel may touch, derived by the host from validated arguments
// (see the kernel's range checks).
struct Guards {
  uint64_t a_lo, a_hi, b_lo, b_hi;      // DMA sources
  uint64_t c_lo, c_hi;                  // output
  uint64_t bias_lo, bias_hi, gidx_lo, gidx_hi, p_lo, p_hi;  // epilogue operands
  uint64_t w_lo, w_hi;                  // workspace (split images, sync words, P and partials)
  uint64_t a2_lo, a2_hi;                // a second first-operand range (broadcast: Xu beside Xc)
};

// Workspace layout of a batch: [header 256 B][prefix int32 (count + 1), padded to 256 B][problems].
struct BatchHeader {
  int32_t magic;
  int32_t count;
  int32_t total_tiles;
  int32_t bm, bn;
  int32_t epi;
  int32_t out_f32;              // output element type the table was written for (C ranges)
  int32_t reserved0;
  Guards guard;                 // union of the problems' operand ranges
  int32_t reserved[24];
};
static_assert(sizeof(BatchHeader) == 256, "BatchHeader layout");
constexpr int32_t kBatchMagic = 0x50544742;  // "PTGB"

inline size_t batch_prefix_bytes(int32_t count) {
  return ((size_t)(count + 1) * 4 + 255) / 256 * 256;
}
inline size_t batch_workspace_bytes(int32_t count) {
  return sizeof(BatchHeader) + batch_prefix_bytes(count) + (size_t)count * sizeof(BatchProblem);
}

struct BatchLaunch {
  const void* workspace;
  int32_t count;
  int epi, out_f32;             // compared with the table header on the device
};

// Limits enforced by the ABI layer.
constexpr int32_t kMaxGroups = 1024;       // group offsets and tile prefix live in LDS
constexpr int32_t kMaxBatch = 2048;        // batch tile prefix lives in LDS
constexpr int64_t kMaxDim = (int64_t)1 << 30;

// Tile shape used by the batch path (the prefix written by prepare depends on it).
constexpr int kBatchBM = 128, kBatchBN = 128;

hipError_t launch_dense(const DenseLaunch& d, hipStream_t stream);

// The one-role dense kernel (every wave both copies and computes; 256 x 256 x 32 tiles, three
// LDS slots): second operand N x K, K a multiple of 32, no split, at least 128 tiles.
// launch_dense takes it whenever onerole_fits holds.
bool onerole_fits(const DenseLaunch& d);
hipError_t launch_onerole(const DenseLaunch& d, hipStream_t stream);
void onerole_describe(int32_t cfg[6]);
// out[i] = sum over s of parts[s * count + i] (s ascending), plus bias[i % n] if bias.
hipError_t launch_reduce_splits(float* out, const float* parts, int64_t count, int32_t splits,
                                const float* bias, int64_t n, hipStream_t stream);
// Split count of the broadcast path's user phase for a U x N product (a function of the
// shape only, so that the workspace query and the call agree), and the maximum over K.
int32_t broadcast_user_splits(int64_t U, int64_t N);
// The one-launch broadcast workspace: a block of sync words (4 KB of 64-bit words: the ticket
// word, one ready word per 256-column block; then the arrival flags, 8 per user-phase slice and
// column block), rounded to 4 KB, then P [U x N] fp32, then the user phase's partial products
// [S x U x N] fp32.
inline size_t broadcast_flags_offset() { return 4096; }
constexpr int32_t kBroadcastMaxSlices = 32;  // user-phase slices of the one-launch form
inline size_t broadcast_sync_bytes(int64_t N, int32_t S) {
  const int64_t n_blocks = (N + 255) / 256;
  return (broadcast_flags_offset() + (size_t)n_blocks * (size_t)(S > 1 ? S : 1) * 8 * 4 + 4095) / 4096 * 4096;
}
// The broadcast GEMM as one persistent launch (user units, reduction units and candidate
// tiles; IkboSched in ptg_kernels.hip).  Used when broadcast_single_launch_fits holds.
struct BroadcastLaunch {
  const void* Xu;
  const void* Xc;
  const int32_t* idx;
  const void* W;
  void* Y;
  const float* bias;          // [N] or null
  void* workspace;            // sync_bytes + (1 + S) U N 4 bytes
  size_t sync_bytes;          // the sync block (broadcast_sync_bytes of the workspace query)
  int64_t U, Mc, Ku, Kc, N;
  int32_t S;                  // user-phase slices
  int64_t k_chunk;            // k per slice (whole k-steps)
  int b_kn, epi, out_f32;
  uint32_t epoch;             // unique per launch
};
bool broadcast_single_launch_fits(int64_t U, int64_t N, int32_t S);
hipError_t launch_broadcast_single(const BroadcastLaunch& b, hipStream_t stream);
hipError_t launch_grouped(const GroupedLaunch& g, hipStream_t stream);
hipError_t launch_batch(const BatchLaunch& b, hipStream_t stream);
hipError_t launch_grouped_wgrad(const WgradLaunch& w, hipStream_t stream);
// IKBO attention: O[c] = softmax(scale Q[c] . K[u]^T) . V[u] per head, u the user of c.
constexpr int kAttnHeadDim = 128;
struct AttentionLaunch {
  const void* Q;              // [Mc x H x D] bf16
  const void* K;              // [U x L x H x D] bf16
  const void* V;              // [U x L x H x D] bf16
  void* O;                    // [Mc x H x D]
  const int32_t* offsets;     // device [U + 1]
  int64_t U, Mc, H, L;
  double scale;
  int out_f32;
};
hipError_t launch_attention(const AttentionLaunch& p, hipStream_t stream);
// Validation of device-resident preconditions: runs a check kernel on `stream`, waits for
// it, and sets *bad to 1 if the data violates the precondition (0 otherwise).  Each check
// takes a result word of its own from a small device array (claimed under a lock, released
// after the wait), so checks on several streams or threads do not share one; *busy is set
// when every word is in use (nothing then runs).
constexpr int kCheckWords = 256;
hipError_t check_offsets(const int32_t* offsets, int32_t G, int64_t M_total, hipStream_t stream,
                         int* bad, int* busy);
hipError_t check_index(const int32_t* idx, int64_t n, int64_t U, hipStream_t stream, int* bad,
                       int* busy);
// The dense path's tile configuration for a problem: BM, BN, BK, stages, consumers, producers.
void dense_config(int64_t M, int64_t N, int64_t K, int b_kn, int32_t cfg[6]);
// Watchdog words of the bounded waits (nonzero if a wait ever gave up): the GEMM kernels'
// word and the attention kernel's word.
hipError_t read_watchdog(uint32_t* value, int clear);
hipError_t read_onerole_watchdog(uint32_t* value, int clear);
hipError_t read_attention_watchdog(uint32_t* value, int clear);

}  // namespace ptg
