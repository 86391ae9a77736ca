// ptg_kernels.hip - tile schedulers, tile-configuration choice and kernel launches.
//
// Three schedulers feed the same pipelined kernel (ptg_device.hpp):
//   Dense   - one problem; tiles visited in an XCD-aware, M-grouped order.
//   Grouped - mixture-of-experts grouped GEMM: the expert row ranges come from int32 offsets
//             in device memory (How We Built TLX, "Case Study 3: Distributed Grouped GEMM for
//             LLM Pretraining"); the per-expert tile prefix is rebuilt in LDS by every
//             workgroup, so the host never reads the offsets.
//   Wgrad   - the weight gradient of the grouped GEMM, dW_g = X_g^T . dY_g: a full output per
//             expert, reduced over the expert's rows (the A operand is X read transposed).
//   Batch   - independent problems (pointer-array form) from a table in the caller's
//             workspace, with the tile prefix staged in LDS; the persistent workgroups run
//             across problem boundaries without draining the ring ("Case Study 2", final
//             stage of the linear-compression kernel).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>
#include <vector>

#include "ptg_device.hpp"
#include "ptg_launch.h"

namespace ptg {

// ---------------------------------------------------------------------------------------
// Dense scheduler
// ---------------------------------------------------------------------------------------
struct DenseSched {
  struct Args {
    const __bf16* A;
    const __bf16* B;
    char* C;
    const float* bias;
    const int32_t* gidx;
    const float* P;
    int64_t lda, ldb, ldc;
    int32_t ldp, p_rows;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n, group_m;
    int32_t epi, out_f32, out_bytes;
    int32_t splits;              // split-K: splits of k_chunk each, outputs c_split apart
    int64_t k_chunk, c_split;
    // units from split_from on are column halves of the last round's tiles (two per tile);
    // split_from at or past the tile count: no split (see launch_dense_cfg)
    int64_t split_from;
    Guards guard;
  };
  __device__ static Guards guards(const Args& a) { return a.guard; }
  static constexpr int LDS_BYTES = 16;
  static constexpr bool kDynamic = false;
  static constexpr int kModes = kModesNone;

  template <class C>
  __device__ static void init(const Args&, char*) {}

  template <class C>
  __device__ static bool tile(const Args& a, int j, TileSrc& t, char*) {
    int64_t L0 = (int64_t)j * gridDim.x + xcd_rank(blockIdx.x, gridDim.x);
    int part = -1;  // column half of a split tile
    if (L0 >= a.split_from) {
      part = (int)((L0 - a.split_from) & 1);
      L0 = a.split_from + (L0 - a.split_from) / 2;
    }
    const int64_t ntiles = (int64_t)a.tiles_m * a.tiles_n;
    if (L0 >= ntiles * a.splits) return false;
    const int64_t split = L0 / ntiles, L = L0 % ntiles;
    const int64_t k0 = split * a.k_chunk;
    // groups of `group_m` tile rows, walked column by column inside a group
    const int64_t per_group = (int64_t)a.group_m * a.tiles_n;
    const int64_t grp = L / per_group, in = L % per_group;
    const int first_m = (int)(grp * a.group_m);
    const int gm = min(a.tiles_m - first_m, a.group_m);
    const int tm = first_m + (int)(in % gm), tn = (int)(in / gm);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN + (part > 0 ? C::BN / 2 : 0);
    t.A = a.A + m0 * a.lda + k0;
    t.lda = a.lda;
    t.B = C::B_KN ? a.B + k0 * a.ldb + n0 : a.B + n0 * a.ldb + k0;
    t.ldb = a.ldb;
    t.info.tag = 0;  // set by the producer when it publishes the slot
    t.info.K = (int)min(a.k_chunk, (int64_t)a.K - k0);
    t.info.m_rows = (int)min((int64_t)C::BM, a.M - m0);
    t.info.n_cols = (int)min((int64_t)(part >= 0 ? C::BN / 2 : C::BN), a.N - n0);
    t.info.C = (uint64_t)(a.C + (split * a.c_split + m0 * a.ldc + n0) * a.out_bytes);
    t.info.ldc = a.ldc;
    t.info.bias = a.bias ? (uint64_t)(a.bias + n0) : 0;
    t.info.gidx = a.gidx ? (uint64_t)(a.gidx + m0) : 0;
    t.info.P = a.P ? (uint64_t)(a.P + n0) : 0;
    t.info.ldp = a.ldp;
    t.info.p_bytes = a.P ? (uint32_t)(((int64_t)a.p_rows * a.ldp - n0) * 4) : 0u;
    return true;
  }
};

// ---------------------------------------------------------------------------------------
// Exclusive prefix sum over n <= NT * IPT values held one per index, in LDS, by the whole
// workgroup.  `val(i)` gives value i; the result goes to out[0..n] (out[n] = total).
// ---------------------------------------------------------------------------------------
template <int NT, class F>
__device__ __forceinline__ void block_exclusive_scan(int n, F val, int32_t* out, int32_t* wave_sums) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWAVE = NT / 64;
  const int per = (n + NT - 1) / NT;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int32_t local = 0;
  for (int i = lo; i < hi; ++i) local += val(i);
  // inclusive scan of `local` across the wave
  int32_t inc = local;
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_sums[wave] = inc;
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int w = 0; w < NWAVE; ++w) {
      const int32_t x = wave_sums[w];
      wave_sums[w] = run;
      run += x;
    }
    wave_sums[NWAVE] = run;
  }
  __syncthreads();
  int32_t run = wave_sums[wave] + inc - local;
  for (int i = lo; i < hi; ++i) {
    out[i] = run;
    run += val(i);
  }
  if (tid == 0) out[n] = wave_sums[NWAVE];
  __syncthreads();
}

// Largest index p in [0, n) with pre[p] <= x (pre nondecreasing, pre[0] <= x < pre[n], n at most
// 64 * 64), found by the 64 lanes of a wave in two rounds of LDS reads: the lanes test 64
// evenly spaced entries, then the entries of the interval that holds x.  Much shorter than a
// serial bisection (two dependent LDS reads instead of about log2 n).
__device__ __forceinline__ int wave_upper_index(const int32_t* pre, int n, int32_t x) {
  const int lane = lane_id();
  const int step = (n + 63) >> 6;
  const int i1 = min(lane * step, n);
  const uint64_t b1 = __ballot(pre[i1] <= x);           // lane 0 always: pre[0] <= x
  const int base = (63 - __builtin_clzll(b1)) * step;
  const int i2 = min(base + lane, n);
  const uint64_t b2 = __ballot(lane < step && pre[i2] <= x);  // lane 0 always
  return base + (63 - __builtin_clzll(b2));
}

// Largest index g in [0, n) with pre[g] <= x (pre nondecreasing, pre[0] <= x < pre[n]).
__device__ __forceinline__ int upper_index(const int32_t* pre, int n, int64_t x) {
  int lo = 0, hi = n;  // invariant: pre[lo] <= x < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)pre[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------------------
// Grouped (mixture-of-experts) scheduler
// ---------------------------------------------------------------------------------------
// Each group g owns rows [off[g], off[g+1]) and is cut into BM-row tiles.  A tile with more
// than BM/2 valid rows costs a full tile; one with at most BM/2 (a group's last partial tile)
// costs about half, since the consumer waves of its empty half idle (consumer_role).  The
// full tiles of all groups come first and the half tiles after them, so the persistent
// workgroups meet the heavy work early; rounds alternate direction over the workgroups
// (snake order), so that the workgroups that took a full tile late take a half tile or
// none at the end.  Within a group, full tiles come in bands of group_m m-tiles walked column
// by column: the workgroups of one XCD, which take consecutive tiles, then share both the
// band's rows of X and a few column strips of W_g in their L2.
//
// The full tiles of a last round that leaves workgroups idle are split by columns: each
// becomes two units of BN / 2 columns on two workgroups.  A unit has half the tile's matrix
// work, and the workgroups would otherwise idle.  Half tiles stay whole: a unit of one would
// issue as many load instructions as the whole tile (its other columns are only masked) and
// load the X rows twice, and measured slower.  Every output element keeps its k-sequence, so
// results do not change.  The tile count is known only on the device, so each workgroup works
// this out from the prefix sums.
//
// With a workspace, a last round of at most half the workgroups instead runs every tile as
// two units: full tiles by columns as above, the others (a group's last, partial tile) by
// reduction, each unit taking half of the k-steps, their fp32 partial sums combined in the
// workspace by whichever unit finishes second (combine_split16).  Such a tile's sums then
// run in two parts, so its bits may differ from the unsplit tile's (same tolerance).
struct GroupedSched {
  struct Args {
    const __bf16* X;
    const __bf16* W;
    char* Y;
    const float* bias;
    const int32_t* offsets;
    char* split_sync;      // workspace of the reduction split (null: none)
    char* split_images;
    uint32_t epoch;
    int64_t M_total;
    int32_t G, N, K, tiles_n, group_m;
    int32_t epi, out_f32, out_bytes;
    Guards guard;
  };
  __device__ static Guards guards(const Args& a) { return a.guard; }
  // offsets[G + 1], full-tile prefix[G + 1], half-tile prefix[G + 1], scan scratch, then the
  // first tile of the last round, the number of its full tiles that are split by columns,
  // and whether its other tiles are split by reduction
  static constexpr int kScratchInts = 20;
  static constexpr int LDS_BYTES = 3 * (kMaxGroups + 1) * 4 + kScratchInts * 4 + 3 * 4;
  static constexpr bool kDynamic = false;
  static constexpr int kModes = kModesSplit;

  // full (more than BM/2 valid rows) and half m-tiles of a group of cnt rows
  template <class C>
  __device__ static int full_mtiles(int cnt) { return cnt / C::BM + (cnt % C::BM > C::BM / 2 ? 1 : 0); }
  template <class C>
  __device__ static int half_mtiles(int cnt) { return (cnt % C::BM > 0 && cnt % C::BM <= C::BM / 2) ? 1 : 0; }

  template <class C>
  __device__ static void init(const Args& a, char* lds) {
    int32_t* off = reinterpret_cast<int32_t*>(lds);
    int32_t* pre_full = off + kMaxGroups + 1;
    int32_t* pre_half = pre_full + kMaxGroups + 1;
    int32_t* scratch = pre_half + kMaxGroups + 1;
    // Offsets are clamped to [0, M_total]: the precondition says they already are, and the
    // clamp keeps every access inside X and Y even when a caller breaks it.
    for (int i = threadIdx.x; i <= a.G; i += C::NT) {
      const int64_t o = a.offsets[i];
      off[i] = (int32_t)(o < 0 ? 0 : (o > a.M_total ? a.M_total : o));
    }
    __syncthreads();
    const int tn = a.tiles_n;
    block_exclusive_scan<C::NT>(a.G, [&](int g) {
      const int cnt = off[g + 1] - off[g];
      return cnt > 0 ? full_mtiles<C>(cnt) * tn : 0;
    }, pre_full, scratch);
    block_exclusive_scan<C::NT>(a.G, [&](int g) {
      const int cnt = off[g + 1] - off[g];
      return cnt > 0 ? half_mtiles<C>(cnt) * tn : 0;
    }, pre_half, scratch);
    static_assert(C::NT / 64 + 1 <= kScratchInts, "scan scratch holds one sum per wave and the total");
    if (threadIdx.x == 0) {
      // pre_full[G] and pre_half[G] were written by this thread
      const int64_t n_full = pre_full[a.G];
      const int64_t T = n_full + pre_half[a.G];
      const int64_t grid = gridDim.x;
      const int64_t last = (T / grid) * grid, rem = T - last;  // the last round's tiles
      const int64_t nf = n_full > last ? min(rem, n_full - last) : 0;  // its full tiles
      const bool by_cols = a.N % C::BN == 0 && C::BN % 128 == 0;
      // every tile of the last round as two units (columns or reduction): needs the workspace,
      // at most one unit per workgroup, and at least two k-steps per tile
      const bool ksplit = a.split_sync != nullptr && rem > 0 && 2 * rem <= grid && a.K > C::BK;
      const bool split = ksplit || (nf > 0 && rem + nf <= grid && by_cols);
      scratch[kScratchInts] = (int32_t)(split ? last : T);
      scratch[kScratchInts + 1] = (int32_t)(split && by_cols ? nf : 0);
      scratch[kScratchInts + 2] = ksplit ? 1 : 0;
    }
  }

  template <class C>
  __device__ static bool tile(const Args& a, int j, TileSrc& t, char* lds) {
    const int32_t* off = reinterpret_cast<const int32_t*>(lds);
    const int32_t* pre_full = off + kMaxGroups + 1;
    const int32_t* pre_half = pre_full + kMaxGroups + 1;
    const int64_t split_from = (pre_half + kMaxGroups + 1)[kScratchInts];
    const int64_t split_nf = (pre_half + kMaxGroups + 1)[kScratchInts + 1];
    const bool ksplit = (pre_half + kMaxGroups + 1)[kScratchInts + 2] != 0;
    const int r = (int)xcd_rank(blockIdx.x, gridDim.x);
    int64_t L = (int64_t)j * gridDim.x + ((j & 1) ? (int64_t)gridDim.x - 1 - r : r);
    int part = -1;   // column half of a split tile
    int khalf = -1;  // reduction half of a split tile
    int64_t slot = 0;
    if (ksplit && L >= split_from) {
      // units 2 t and 2 t + 1 are the halves of the round's tile t: by columns for its first
      // split_nf tiles (full ones), by reduction for the others; past the last tile there is
      // no unit (below)
      const int64_t u = L - split_from;
      slot = u / 2;
      L = split_from + slot;
      if (slot < split_nf) part = (int)(u & 1);
      else khalf = (int)(u & 1);
    } else if (split_nf > 0 && L >= split_from) {
      // units 0 .. 2 nf - 1 are the halves of the round's full tiles, then its half tiles;
      // past the last tile there is no unit (below)
      const int64_t u = L - split_from;
      if (u < 2 * split_nf) {
        part = (int)(u & 1);
        L = split_from + u / 2;
      } else {
        L = split_from + split_nf + (u - 2 * split_nf);
      }
    }
    const int64_t n_full = pre_full[a.G];
    int g, mt, nt;
    if (L < n_full) {
      g = upper_index(pre_full, a.G, L);
      const int local = (int)(L - pre_full[g]);
      const int mtiles = full_mtiles<C>(off[g + 1] - off[g]);
      const int per_band = a.group_m * a.tiles_n;
      const int band = local / per_band, in = local % per_band;
      const int first_m = band * a.group_m;
      const int bm = min(mtiles - first_m, a.group_m);
      mt = first_m + in % bm;
      nt = in / bm;
    } else {
      const int64_t L2 = L - n_full;
      if (L2 >= pre_half[a.G]) return false;
      g = upper_index(pre_half, a.G, L2);
      mt = (off[g + 1] - off[g]) / C::BM;  // the group's last, partial m-tile
      nt = (int)(L2 - pre_half[g]);
    }
    const int row0 = off[g], cnt = off[g + 1] - off[g];  // cnt > 0: the group has tiles
    const int64_t m0 = (int64_t)row0 + (int64_t)mt * C::BM;
    const int64_t n0 = (int64_t)nt * C::BN + (part > 0 ? C::BN / 2 : 0);
    const int64_t wsize = (int64_t)a.K * a.N;
    // a reduction half: the first unit takes the first half of the k-steps (rounded down)
    const int64_t k_mid = (int64_t)(tile_steps<C>(a.K) / 2) * C::BK;
    const int64_t k0 = khalf > 0 ? k_mid : 0;
    const int64_t kl = khalf < 0 ? a.K : (khalf == 0 ? k_mid : a.K - k_mid);
    t.A = a.X + m0 * a.K + k0;
    t.lda = a.K;
    t.B = a.W + g * wsize + (C::B_KN ? k0 * a.N + n0 : n0 * a.K + k0);
    t.ldb = C::B_KN ? a.N : a.K;
    t.info.tag = 0;  // set by the producer when it publishes the slot
    t.info.K = (int)kl;
    if (khalf >= 0) {
      t.info.mode = (uint32_t)(khalf + 1);
      t.info.epoch = a.epoch;
      t.info.sync = (uint64_t)(a.split_sync + slot * kSplitSyncBytes);
      t.info.part = (uint64_t)(a.split_images + slot * kSplitImageBytes);
    }
    t.info.m_rows = min(C::BM, cnt - mt * C::BM);
    t.info.n_cols = (int)min((int64_t)(part >= 0 ? C::BN / 2 : C::BN), (int64_t)a.N - n0);
    t.info.C = (uint64_t)(a.Y + (m0 * a.N + n0) * a.out_bytes);
    t.info.ldc = a.N;
    t.info.bias = a.bias ? (uint64_t)(a.bias + (int64_t)g * a.N + n0) : 0;
    t.info.gidx = 0;
    t.info.P = 0;
    t.info.ldp = 0;
    t.info.p_bytes = 0;
    return true;
  }
};

// ---------------------------------------------------------------------------------------
// Grouped weight-gradient scheduler: dW_g = X_g^T . dY_g
// ---------------------------------------------------------------------------------------
// The backward counterpart of the grouped GEMM above (same case study: the expert products
// of pretraining).  Every expert owns a full K x N output, cut into BM x BN tiles; the
// reduction runs over the expert's rows, so a tile's cost is its expert's row count and
// varies from nothing (an expert without rows: one step of zeros, dW_g = 0) to most of the
// batch, while every tile writes the same BM x BN output.  A static assignment cannot balance
// such costs without knowing the row counts, which live on the device, so the workgroups take
// tiles from queues (counters in the caller's workspace, reset by a small kernel before the
// launch).
//   - One queue per XCD.  Queue x holds block x of every expert's tile grid: the m-tiles are
//     cut into pm blocks and the n-tiles into pn blocks (pm * pn = 8, chosen by the host to
//     minimise pn |X| + pm |dY|), so a slice of X_g is fetched into pn L2s and a slice of dY_g
//     into pm, instead of into whichever XCDs happen to take its tiles.  A workgroup takes
//     from its own XCD's queue, and from the others in turn once that one is drained.
//   - Within a queue, positions alternate between the heaviest and the lightest tile not yet
//     handed out (experts ordered by row count in LDS by every workgroup): the long reductions
//     start early, and the cheap, store-heavy tiles are spread over the whole run instead of
//     crowding its end, which keeps the output writes overlapped with the matrix work.
//   - Within an expert's block, tiles go down the m-tiles of one column strip, then the next.
struct WgradSched {
  struct Args {
    const __bf16* X;       // [M_total x K]
    const __bf16* dY;      // [M_total x N]
    char* dW;              // [G x K x N]
    const int32_t* offsets;
    uint32_t* queue;       // kQueues counters, kQueueStride words apart (workspace), 0 at launch
    int64_t M_total;
    int32_t G, K, N, tiles_m, tiles_n;
    int32_t pm, pn;        // blocks of m-tiles and of n-tiles, pm * pn = kQueues
    int32_t epi, out_f32, out_bytes;
    Guards guard;
  };
  __device__ static Guards guards(const Args& a) { return a.guard; }
  static constexpr bool kDynamic = true;
  static constexpr int kModes = kModesNone;
  static constexpr int kClaimSlots = 16;
  static constexpr int kQueues = 8;          // one per XCD
  static constexpr int kQueueStride = 8;     // 32 bytes between counters
  static constexpr uint32_t kNoTile = 0xFFFFFFFFu;
  // claim slots [16] (8-byte aligned first), offsets[G + 1], experts by decreasing row count [G]
  static constexpr int LDS_BYTES = kClaimSlots * 8 + (2 * kMaxGroups + 1) * 4 + 16;
  __device__ static uint64_t* claim_slots(char* lds) { return reinterpret_cast<uint64_t*>(lds); }
  __device__ static int32_t* offsets_lds(char* lds) { return reinterpret_cast<int32_t*>(lds + kClaimSlots * 8); }

  template <class C>
  __device__ static void init(const Args& a, char* lds) {
    uint64_t* slots = claim_slots(lds);
    int32_t* off = offsets_lds(lds);
    int32_t* order = off + kMaxGroups + 1;
    if (threadIdx.x < kClaimSlots) slots[threadIdx.x] = 0;  // no tag matches before a claim
    // clamped to [0, M_total] (see GroupedSched::init)
    for (int i = threadIdx.x; i <= a.G; i += C::NT) {
      const int64_t o = a.offsets[i];
      off[i] = (int32_t)(o < 0 ? 0 : (o > a.M_total ? a.M_total : o));
    }
    __syncthreads();
    // rank of expert g: experts with more rows, or as many and a smaller index, come first
    for (int g = threadIdx.x; g < a.G; g += C::NT) {
      const int cg = max(off[g + 1] - off[g], 0);
      int rank = 0;
      for (int h = 0; h < a.G; ++h) {
        const int ch = max(off[h + 1] - off[h], 0);
        rank += (ch > cg || (ch == cg && h < g)) ? 1 : 0;
      }
      order[rank] = g;
    }
    // the kernel's barrier after init publishes `order` and the cleared slots
  }

  // Block x of an expert's tile grid: m-tiles [mlo, mlo + mc), n-tiles [nlo, nlo + nc).
  __device__ static void block_of(const Args& a, int x, int& mlo, int& mc, int& nlo, int& nc) {
    const int bm = x / a.pn, bn = x % a.pn;
    mlo = bm * a.tiles_m / a.pm;
    mc = (bm + 1) * a.tiles_m / a.pm - mlo;
    nlo = bn * a.tiles_n / a.pn;
    nc = (bn + 1) * a.tiles_n / a.pn - nlo;
  }

  // A ticket for the calling workgroup's next tile: queue (4 bits) and position (28 bits), or
  // kNoTile when every queue is drained.  Called by one lane.  The XCD of a workgroup is
  // blockIdx.x mod 8 (workgroups are dealt to the XCDs round-robin).
  __device__ static uint32_t claim(const Args& a, char*) {
    const int x0 = (int)(blockIdx.x % kQueues);
    for (int d = 0; d < kQueues; ++d) {
      const int x = (x0 + d) % kQueues;
      int mlo, mc, nlo, nc;
      block_of(a, x, mlo, mc, nlo, nc);
      const uint32_t T = (uint32_t)a.G * (uint32_t)(mc * nc);
      if (T == 0) continue;
      const uint32_t pos = atomicAdd(a.queue + x * kQueueStride, 1u);
      if (pos < T) return ((uint32_t)x << 28) | pos;
    }
    return kNoTile;
  }

  // The tile of a ticket: positions of a queue alternate between the front (heaviest) and the
  // back (lightest) of its tiles ordered by cost.
  template <class C>
  __device__ static bool tile_at(const Args& a, uint32_t ticket, TileSrc& t, char* lds) {
    const int32_t* off = offsets_lds(lds);
    const int32_t* order = off + kMaxGroups + 1;
    if (ticket == kNoTile) return false;
    const int x = (int)(ticket >> 28);
    const uint32_t q = ticket & 0x0FFFFFFFu;
    int mlo, mc, nlo, nc;
    block_of(a, x, mlo, mc, nlo, nc);
    const int per = mc * nc;
    const int64_t T = (int64_t)a.G * per;
    if (per == 0 || (int64_t)q >= T) return false;
    const int64_t p = (q & 1u) ? T - 1 - (int64_t)(q >> 1) : (int64_t)(q >> 1);
    const int g = order[(int)(p / per)];
    const int local = (int)(p % per);
    const int mt = mlo + local % mc, nt = nlo + local / mc;
    const int64_t row0 = off[g];
    const int cnt = max(off[g + 1] - off[g], 0);
    const int64_t m0 = (int64_t)mt * C::BM, n0 = (int64_t)nt * C::BN;
    t.A = a.X + row0 * a.K + m0;   // X_g^T: k = row of X, m = column of X
    t.lda = a.K;
    t.B = a.dY + row0 * a.N + n0;
    t.ldb = a.N;
    t.info.tag = 0;  // set by the producer when it publishes the slot
    t.info.K = cnt;
    t.info.m_rows = (int)min((int64_t)C::BM, (int64_t)a.K - m0);
    t.info.n_cols = (int)min((int64_t)C::BN, (int64_t)a.N - n0);
    t.info.C = (uint64_t)(a.dW + (((int64_t)g * a.K + m0) * a.N + n0) * a.out_bytes);
    t.info.ldc = a.N;
    t.info.bias = 0;
    t.info.gidx = 0;
    t.info.P = 0;
    t.info.ldp = 0;
    t.info.p_bytes = 0;
    return true;
  }
};

// Resets the tile-queue counters (vector stores) ahead of the kernel that drains them.
__global__ void arm_queue_kernel(uint32_t* queue) {
  if (threadIdx.x < WgradSched::kQueues) queue[threadIdx.x * WgradSched::kQueueStride] = 0;
}

// ---------------------------------------------------------------------------------------
// Single-launch broadcast (IKBO) scheduler
// ---------------------------------------------------------------------------------------
// The in-kernel broadcast GEMM of "Case Study 2: In-Kernel Broadcast Optimization for RecSys"
// as one persistent launch (the final form its subsection "TLX Provides a Building Block for
// the Final Stage of This Optimization" describes: user and candidate GEMMs share the
// pipeline, and tiles hand results to each other with release and acquire flags).  Its work
// comes in three kinds, in this order of tickets:
//   - user units (S per column block of P): the partial product of Xu and one K-slice of
//     the user half of W, written to the workspace;
//   - reduction units (red_per_nb per column block): once every user unit of the block has
//     arrived, the sum of the partials in slice order plus the bias, rows of P;
//   - candidate tiles: Xc . W_c starting from P[idx[r]], once their block of P is ready.
// Each workgroup takes user and reduction units from a shared ticket word (its claims are in
// increasing ticket order) until none is left, then its share of the candidate tiles in the
// dense order (XCD-aware bands of m-tiles).  A unit waits only on units of smaller tickets,
// already held by running workgroups that wait on nothing later, so the launch finishes
// whether or not all its workgroups are resident at once.  The ticket, arrival and ready
// words carry the launch's epoch (epoch_add), so nothing is cleared between launches.
struct IkboSched {
  struct Args {
    const __bf16* Xu;
    const __bf16* Xc;
    const __bf16* W;
    const int32_t* idx;
    char* Y;
    const float* bias;
    float* P;              // [U x N]
    float* parts;          // [S x U x N]
    uint64_t* words;       // the ticket word, then one ready word per column block
    uint32_t* flags;       // arrival flags [n_blocks][S][NCG] (one per consumer wave)
    uint32_t epoch;
    int32_t U, Mc, Ku, Kc, N, Kt, S, k_chunk, n_blocks, red_rows, red_per_nb;
    int32_t T_user, T_dyn;
    int32_t tiles_m, tiles_n, group_m;
    int32_t epi, out_f32, out_bytes;
    Guards guard;
  };
  __device__ static Guards guards(const Args& a) { return a.guard; }
  static constexpr bool kDynamic = true;
  static constexpr int kModes = kModesBroadcast;
  static constexpr int kClaimSlots = 16;
  static constexpr uint32_t kNoTile = 0xFFFFFFFFu;
  // claim slots [16], then the workgroup's "no unit left" flag and its next candidate index
  static constexpr int LDS_BYTES = kClaimSlots * 8 + 16;
  __device__ static uint64_t* claim_slots(char* lds) { return reinterpret_cast<uint64_t*>(lds); }
  __device__ static int32_t* state(char* lds) { return reinterpret_cast<int32_t*>(lds + kClaimSlots * 8); }

  template <class C>
  __device__ static void init(const Args&, char* lds) {
    if (threadIdx.x < kClaimSlots) claim_slots(lds)[threadIdx.x] = 0;
    if (threadIdx.x < 2) state(lds)[threadIdx.x] = 0;
  }

  // The launch's arguments, read where they are used (scalar loads from the kernel-argument
  // segment, where the single argument lies at offset 0).  The empty asm hides that the
  // pointer is the same on every tile, so the compiler does not keep the thirty-odd fields in
  // scalar registers across the producer loop, where they would spill.
  typedef const __attribute__((address_space(4))) Args KArgs;
  __device__ static KArgs& fresh() {
    KArgs* p = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return *p;
  }

  // The next ticket of the calling workgroup (one lane of its first producer): user and
  // reduction units from the launch's ticket word while they last, then the workgroup's
  // candidate tiles in the dense path's XCD-aware order (tiles j grid + xcd_rank, so that tiles
  // sharing Xc rows and W columns meet in one L2).  Measured faster than per-XCD queues of
  // candidates, whose claims cost a round trip to memory per tile.
  __device__ static uint32_t claim(const Args&, char* lds) {
    KArgs& a = fresh();
    int32_t* st = state(lds);
    if (st[0] == 0) {
      const uint32_t t = epoch_add(a.words, a.epoch);
      if (t < (uint32_t)a.T_dyn) return t;
      st[0] = 1;
    }
    const int64_t L = (int64_t)(st[1]++) * gridDim.x + xcd_rank(blockIdx.x, gridDim.x);
    if (L >= (int64_t)a.tiles_m * a.tiles_n) return kNoTile;
    return (uint32_t)(a.T_dyn + L);
  }

  template <class C>
  __device__ static bool tile_at(const Args&, uint32_t ticket, TileSrc& t, char*) {
    if (ticket == kNoTile) return false;
    KArgs& a = fresh();
    const int64_t N = a.N;
    t.info.tag = 0;  // set by the producer when it publishes the slot
    t.info.epoch = a.epoch;
    if (ticket < (uint32_t)a.T_user) {
      // user unit: slice s of Ku for column block nb
      const int nb = (int)ticket / a.S, s = (int)ticket % a.S;
      const int64_t k0 = (int64_t)s * a.k_chunk, n0 = (int64_t)nb * C::BN;
      t.A = a.Xu + k0;
      t.lda = a.Ku;
      t.B = C::B_KN ? a.W + k0 * N + n0 : a.W + n0 * a.Kt + k0;
      t.ldb = C::B_KN ? N : a.Kt;
      t.info.K = (int)min((int64_t)a.k_chunk, (int64_t)a.Ku - k0);
      t.info.m_rows = a.U;
      t.info.n_cols = (int)min((int64_t)C::BN, N - n0);
      t.info.C = (uint64_t)(a.parts + (int64_t)s * a.U * N + n0);
      t.info.ldc = N;
      t.info.mode = kModeUserPartial;
      t.info.sync = (uint64_t)(a.flags + ((int64_t)nb * a.S + s) * C::NCG);
      return true;
    }
    if (ticket < (uint32_t)a.T_dyn) {
      // reduction unit q of column block nb: rows [q red_rows, +red_rows) of P
      const int r = (int)ticket - a.T_user;
      const int nb = r / a.red_per_nb, q = r % a.red_per_nb;
      const int64_t row0 = (int64_t)q * a.red_rows, n0 = (int64_t)nb * C::BN;
      t.A = nullptr;
      t.B = nullptr;
      t.info.K = 0;  // one empty k-step
      t.info.m_rows = (int)min((int64_t)a.red_rows, (int64_t)a.U - row0);
      t.info.n_cols = (int)min((int64_t)C::BN, N - n0);
      t.info.part = (uint64_t)(a.parts + row0 * N + n0);
      t.info.P = (uint64_t)(a.P + row0 * N + n0);
      t.info.ldp = (int32_t)N;
      t.info.bias = a.bias ? (uint64_t)(a.bias + n0) : 0;
      t.info.count = (uint32_t)a.S;
      t.info.stride = (uint32_t)((int64_t)a.U * N);
      t.info.mode = kModeReduce;
      t.info.sync = (uint64_t)(a.flags + (int64_t)nb * a.S * C::NCG);
      t.info.C = (uint64_t)(a.words + 1 + nb);  // the block's ready word
      {
        // the consumer waves of a user unit that own rows and columns of it (the others idle)
        const int am = min(C::WM, (a.U + C::WTM - 1) / C::WTM);
        const int an = min(C::WN, (int)((t.info.n_cols + C::WTN - 1) / C::WTN));
        uint32_t mask = 0;
        for (int m = 0; m < am; ++m)
          for (int n = 0; n < an; ++n) mask |= 1u << (m * C::WN + n);
        t.info.p_bytes = mask;
      }
      return true;
    }
    // candidate tile L (the dense order: bands of group_m m-tiles walked column by column)
    const int64_t L = (int64_t)ticket - a.T_dyn;
    const int64_t per_group = (int64_t)a.group_m * a.tiles_n;
    const int64_t grp = L / per_group, in = L % per_group;
    const int first_m = (int)(grp * a.group_m);
    const int gm = min(a.tiles_m - first_m, a.group_m);
    const int tm = first_m + (int)(in % gm), tn = (int)(in / gm);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    t.A = a.Xc + m0 * a.Kc;
    t.lda = a.Kc;
    t.B = C::B_KN ? a.W + (int64_t)a.Ku * N + n0 : a.W + n0 * a.Kt + a.Ku;
    t.ldb = C::B_KN ? N : a.Kt;
    t.info.K = a.Kc;
    t.info.m_rows = (int)min((int64_t)C::BM, (int64_t)a.Mc - m0);
    t.info.n_cols = (int)min((int64_t)C::BN, N - n0);
    t.info.C = (uint64_t)(a.Y + (m0 * N + n0) * a.out_bytes);
    t.info.ldc = N;
    t.info.gidx = (uint64_t)(a.idx + m0);
    t.info.P = (uint64_t)(a.P + n0);
    t.info.ldp = (int32_t)N;
    t.info.p_bytes = (uint32_t)(((int64_t)a.U * N - n0) * 4);
    t.info.mode = kModeCandidate;
    t.info.sync = (uint64_t)(a.words + 1 + tn);
    t.info.count = (uint32_t)(a.red_per_nb * C::NPROD);
    return true;
  }
};

// ---------------------------------------------------------------------------------------
// Batch (pointer-array) scheduler
// ---------------------------------------------------------------------------------------
struct BatchSched {
  struct Args {
    const BatchHeader* hdr;       // table header (workspace)
    const int32_t* prefix;        // [count + 1] tile prefix (workspace)
    const BatchProblem* probs;    // [count]
    int32_t count;
    int32_t epi, out_f32, out_bytes;
    const Guards* guard_ptr;
  };
  __device__ static Guards guards(const Args& a) { return *a.guard_ptr; }
  static constexpr int LDS_BYTES = (kMaxBatch + 1) * 4 + 16;
  static constexpr bool kDynamic = false;
  static constexpr int kModes = kModesNone;

  // The launch runs only the table it was asked for: a header whose magic, count, epilogue
  // or output type differs from the launch's arguments (a table written for another call)
  // gives a prefix with no tiles, so the workgroups publish the end marker at once and touch
  // no operand; watchdog bit 2 records it.
  template <class C>
  __device__ static void init(const Args& a, char* lds) {
    int32_t* pre = reinterpret_cast<int32_t*>(lds);
    const BatchHeader& h = *a.hdr;
    const bool ok = h.magic == kBatchMagic && h.count == a.count && h.epi == a.epi &&
                    h.out_f32 == a.out_f32 && h.bm == C::BM && h.bn == C::BN;
    if (ok) {
      for (int i = threadIdx.x; i <= a.count; i += C::NT) pre[i] = a.prefix[i];
    } else {
      for (int i = threadIdx.x; i <= a.count; i += C::NT) pre[i] = 0;
      if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(&g_watchdog, 2u);
    }
  }

  // The problem record is read with scalar loads (constant address space, wave-uniform index):
  // their completion is counted apart from the vector-memory counter, so the producer does not
  // wait for its own buffer-to-LDS copies in flight before it can use the record, as it would
  // after an ordinary (vector) load.
  template <class C>
  __device__ static bool tile(const Args& a, int j, TileSrc& t, char* lds) {
    typedef const __attribute__((address_space(4))) BatchProblem ConstProblem;
    const int32_t* pre = reinterpret_cast<const int32_t*>(lds);
    const int64_t L = (int64_t)j * gridDim.x + xcd_rank(blockIdx.x, gridDim.x);
    if (L >= pre[a.count]) return false;
    const int p = (int)uni((uint32_t)wave_upper_index(pre, a.count, (int32_t)L));
    const int local = (int)(L - pre[p]);
    ConstProblem& q = reinterpret_cast<ConstProblem*>(reinterpret_cast<uintptr_t>(a.probs))[p];
    const int mt = local % q.tiles_m, nt = local / q.tiles_m;
    const int64_t m0 = (int64_t)mt * C::BM, n0 = (int64_t)nt * C::BN;
    t.A = reinterpret_cast<const __bf16*>(q.A) + m0 * q.lda;
    t.lda = q.lda;
    t.B = reinterpret_cast<const __bf16*>(q.B) + n0;
    t.ldb = q.ldb;
    t.info.tag = 0;  // set by the producer when it publishes the slot
    t.info.K = q.K;
    t.info.m_rows = (int)min((int64_t)C::BM, (int64_t)q.M - m0);
    t.info.n_cols = (int)min((int64_t)C::BN, (int64_t)q.N - n0);
    t.info.C = (uint64_t)(reinterpret_cast<char*>(q.C) + (m0 * q.ldc + n0) * a.out_bytes);
    t.info.ldc = q.ldc;
    t.info.bias = q.bias ? (uint64_t)(q.bias + n0) : 0;
    t.info.gidx = 0;
    t.info.P = 0;
    t.info.ldp = 0;
    t.info.p_bytes = 0;
    return true;
  }
};

// ---------------------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------------------
// Large problems: 256 x 256 tiles, 8 consumer waves (2 x 4, 128 x 64 each) on 16x16x32
// MFMAs, 4 producers staging one k-step in registers, two 64 KB ring slots, output written as
// streaming stores of whole 128-byte row segments.  Medium/small: 128 x 128 tiles on 32x32x16
// MFMAs, two consumer groups of 4 waves (64 x 64 each) taking alternate tiles, so that one
// group's epilogue overlaps the other's matrix work, 2 producers, four 32 KB slots.  Grouped (mixture-of-experts)
// problems use the large tiles too: a group's last partial tile with at most 128 valid rows
// runs on half the consumer waves at about half the cost.
template <bool KN> using CfgLarge = Cfg<256, 256, 64, 2, 2, 4, 4, KN, 1, true, false, true>;
template <bool KN> using CfgMedium = Cfg<128, 128, 64, 4, 2, 2, 2, KN, 0, false, false, false, 2>;
template <bool KN> using CfgGrouped = CfgLarge<KN>;
// The pointer-array batch: the medium tile on 16x16x32 MFMAs with whole 128-byte row segments
// per store (the 32x32 layout stores 32-byte pieces of 32 rows).  Its short reductions leave
// it bound by the output stores: 0.2557 -> 0.2393 ms on the 1024-problem batch, same bits.
// Dense medium problems, whose work is mostly matrix work, keep the 32x32 form (4% faster
// there).
using CfgBatch = Cfg<128, 128, 64, 4, 2, 2, 2, true, 0, true, false, true, 2>;
// Weight gradient X^T . dY: the large tile with A (X^T) stored K x M and B (dY) K x N, its
// output (a full K x N per expert, the bulk of the traffic) written as streaming stores.
using CfgWgrad = Cfg<256, 256, 64, 2, 2, 4, 4, true, 1, true, true, true>;

struct DeviceInfo {
  int cus = 0;
};

static int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

int device_compute_units() { return device_cus(); }

static uint64_t addr(const void* p) { return reinterpret_cast<uint64_t>(p); }

// [p, p + bytes), or the empty range [0, 0) when p is null.
static void span(const void* p, uint64_t bytes, uint64_t& lo, uint64_t& hi) {
  lo = p ? addr(p) : 0;
  hi = p ? addr(p) + bytes : 0;
}

// Bytes of a row-major [rows x cols] matrix with row stride ld (elements of `esize` bytes).
static uint64_t mat_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  return rows > 0 ? (uint64_t)(((rows - 1) * ld + cols) * esize) : 0;
}

template <class C, class S>
static hipError_t launch_persistent(const typename S::Args& a, int64_t max_tiles, hipStream_t stream) {
  const int cus = device_cus();
  if (cus <= 0) return hipErrorNoDevice;
  const int64_t grid = max_tiles < cus ? max_tiles : cus;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ptg_kernel<C, S>), dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

template <class C>
static void describe(int32_t cfg[6]) {
  cfg[0] = C::BM; cfg[1] = C::BN; cfg[2] = C::BK; cfg[3] = C::STAGES; cfg[4] = C::NCONS; cfg[5] = C::NPROD;
}

static bool use_large(int64_t M, int64_t N) {
  // enough 256 x 256 tiles to fill the chip at least once
  const int64_t t = ((M + 255) / 256) * ((N + 255) / 256);
  return t >= 128;
}

void dense_config(int64_t M, int64_t N, int64_t K, int b_kn, int32_t cfg[6]) {
  DenseLaunch probe{};
  probe.M = M; probe.N = N; probe.K = K; probe.b_kn = b_kn;
  if (onerole_fits(probe)) {
    onerole_describe(cfg);
    return;
  }
  if (use_large(M, N)) {
    if (b_kn) describe<CfgLarge<true>>(cfg); else describe<CfgLarge<false>>(cfg);
  } else {
    if (b_kn) describe<CfgMedium<true>>(cfg); else describe<CfgMedium<false>>(cfg);
  }
}

template <class C>
static hipError_t launch_dense_cfg(const DenseLaunch& d, hipStream_t stream) {
  DenseSched::Args a;
  a.A = reinterpret_cast<const __bf16*>(d.A);
  a.B = reinterpret_cast<const __bf16*>(d.B);
  a.C = reinterpret_cast<char*>(d.C);
  a.bias = d.bias;
  a.gidx = d.gidx;
  a.P = d.P;
  a.lda = d.lda; a.ldb = d.ldb; a.ldc = d.ldc; a.ldp = (int32_t)d.ldp; a.p_rows = (int32_t)d.p_rows;
  a.M = (int32_t)d.M; a.N = (int32_t)d.N; a.K = (int32_t)d.K;
  a.tiles_m = (int32_t)((d.M + C::BM - 1) / C::BM);
  a.tiles_n = (int32_t)((d.N + C::BN - 1) / C::BN);
  a.group_m = 4;
  a.epi = d.epi; a.out_f32 = d.out_f32; a.out_bytes = d.out_f32 ? 4 : 2;
  a.splits = d.splits > 1 ? d.splits : 1;
  a.k_chunk = d.splits > 1 ? d.k_chunk : d.K;
  a.c_split = d.splits > 1 ? d.c_split : 0;
  {
    // A last round that leaves at least half the workgroups idle runs its tiles as column
    // halves on two workgroups each (every tile full width, so no half is empty).
    const int64_t total = (int64_t)a.tiles_m * a.tiles_n * a.splits;
    const int cus = device_cus();
    const int64_t grid = total < cus ? total : cus;
    const int64_t last = grid > 0 ? (total / grid) * grid : 0, rem = total - last;
    const bool split = grid > 0 && rem > 0 && 2 * rem <= grid && d.N % C::BN == 0 && C::BN % 128 == 0;
    a.split_from = split ? last : total;
  }
  Guards& g = a.guard;
  span(d.A, mat_bytes(d.M, d.K, d.lda, 2), g.a_lo, g.a_hi);
  span(d.B, d.b_kn ? mat_bytes(d.K, d.N, d.ldb, 2) : mat_bytes(d.N, d.K, d.ldb, 2), g.b_lo, g.b_hi);
  span(d.C, (uint64_t)(a.splits - 1) * a.c_split * a.out_bytes + mat_bytes(d.M, d.N, d.ldc, a.out_bytes),
       g.c_lo, g.c_hi);
  span(d.bias, (uint64_t)d.N * 4, g.bias_lo, g.bias_hi);
  span(d.gidx, (uint64_t)d.M * 4, g.gidx_lo, g.gidx_hi);
  span(d.P, mat_bytes(d.p_rows, d.ldp, d.ldp, 4), g.p_lo, g.p_hi);
  return launch_persistent<C, DenseSched>(a, (int64_t)a.tiles_m * a.tiles_n * a.splits, stream);
}

hipError_t launch_dense(const DenseLaunch& d, hipStream_t stream) {
  if (d.M == 0 || d.N == 0) return hipSuccess;
  if (onerole_fits(d)) return launch_onerole(d, stream);
  if (use_large(d.M, d.N)) {
    return d.b_kn ? launch_dense_cfg<CfgLarge<true>>(d, stream) : launch_dense_cfg<CfgLarge<false>>(d, stream);
  }
  return d.b_kn ? launch_dense_cfg<CfgMedium<true>>(d, stream) : launch_dense_cfg<CfgMedium<false>>(d, stream);
}

// ---------------------------------------------------------------------------------------
// Split-K reduction (broadcast user phase): out = sum of the partials in split order, plus
// the bias; memory-bound, 16 bytes per lane per access.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void reduce_splits_kernel(float* out, const float* parts, int64_t count,
                                                            int32_t splits, const float* bias, int64_t n) {
  typedef __attribute__((ext_vector_type(4))) float f4;
  const int64_t quads = count / 4;  // count and n are multiples of 8
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += (int64_t)gridDim.x * blockDim.x) {
    f4 acc = reinterpret_cast<const f4*>(parts)[q];
    // up to 32 partials in flight at a time (the user phase makes at most 32), added in split
    // order: one round trip to memory per quad instead of four
    constexpr int kInFlight = 32;
    for (int32_t s0 = 1; s0 < splits; s0 += kInFlight) {
      f4 v[kInFlight];
#pragma unroll
      for (int i = 0; i < kInFlight; ++i)
        v[i] = s0 + i < splits ? reinterpret_cast<const f4*>(parts + (s0 + i) * count)[q] : f4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kInFlight; ++i)
        if (s0 + i < splits) acc += v[i];
    }
    if (bias) acc += reinterpret_cast<const f4*>(bias)[(q * 4 % n) / 4];
    reinterpret_cast<f4*>(out)[q] = acc;
  }
}

hipError_t launch_reduce_splits(float* out, const float* parts, int64_t count, int32_t splits,
                                const float* bias, int64_t n, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  // 64-thread blocks: a small P still spreads over many CUs
  const int64_t quads = count / 4;
  const int64_t blocks = (quads + 63) / 64;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(64), 0, stream,
                     out, parts, count, splits, bias, n);
  return hipGetLastError();
}

// Splits of the broadcast user phase: enough to give the 256 CUs of an MI355X one tile each
// when the U x N product alone has few tiles (it is small: U users), at most 32.
int32_t broadcast_user_splits(int64_t U, int64_t N) {
  const int64_t tiles = use_large(U, N) ? ((U + 255) / 256) * ((N + 255) / 256) : ((U + 127) / 128) * ((N + 127) / 128);
  const int64_t s = 256 / (tiles > 0 ? tiles : 1);
  return (int32_t)(s < 1 ? 1 : (s > 32 ? 32 : s));
}

// The single launch needs the user rows in one large m-tile, a split user phase (at most 32
// slices, the reduction units' limit) and its sync words in their 4 KB block; the caller also
// keeps the whole workspace under 2 GiB (the reduction units address it with 31-bit offsets).
bool broadcast_single_launch_fits(int64_t U, int64_t N, int32_t S) {
  const int64_t n_blocks = (N + 255) / 256;
  return U >= 1 && U <= 256 && S >= 2 && S <= 32 && (1 + n_blocks) * 8 <= (int64_t)broadcast_flags_offset();
}

template <class C>
static hipError_t launch_broadcast_single_cfg(const BroadcastLaunch& b, hipStream_t stream) {
  IkboSched::Args a;
  a.Xu = reinterpret_cast<const __bf16*>(b.Xu);
  a.Xc = reinterpret_cast<const __bf16*>(b.Xc);
  a.W = reinterpret_cast<const __bf16*>(b.W);
  a.idx = b.idx;
  a.Y = reinterpret_cast<char*>(b.Y);
  a.bias = b.bias;
  char* ws = reinterpret_cast<char*>(b.workspace);
  a.words = reinterpret_cast<uint64_t*>(ws);
  a.flags = reinterpret_cast<uint32_t*>(ws + broadcast_flags_offset());
  a.P = reinterpret_cast<float*>(ws + b.sync_bytes);
  a.parts = a.P + b.U * b.N;
  a.epoch = b.epoch;
  a.U = (int32_t)b.U; a.Mc = (int32_t)b.Mc; a.Ku = (int32_t)b.Ku; a.Kc = (int32_t)b.Kc; a.N = (int32_t)b.N;
  a.Kt = (int32_t)(b.Ku + b.Kc);
  a.S = b.S;
  a.k_chunk = (int32_t)b.k_chunk;
  a.n_blocks = (int32_t)((b.N + C::BN - 1) / C::BN);
  a.red_rows = 2 * C::NPROD;  // two rows of P per producer wave
  a.red_per_nb = (int32_t)((b.U + a.red_rows - 1) / a.red_rows);
  a.T_user = a.n_blocks * a.S;
  a.T_dyn = a.T_user + a.n_blocks * a.red_per_nb;
  a.tiles_m = (int32_t)((b.Mc + C::BM - 1) / C::BM);
  a.tiles_n = a.n_blocks;
  a.group_m = 4;
  a.epi = b.epi; a.out_f32 = b.out_f32; a.out_bytes = b.out_f32 ? 4 : 2;
  Guards& g = a.guard;
  g = Guards{};
  const int64_t Kt = b.Ku + b.Kc;
  span(b.Xc, mat_bytes(b.Mc, b.Kc, b.Kc, 2), g.a_lo, g.a_hi);
  span(b.Xu, mat_bytes(b.U, b.Ku, b.Ku, 2), g.a2_lo, g.a2_hi);
  span(b.W, b.b_kn ? mat_bytes(Kt, b.N, b.N, 2) : mat_bytes(b.N, Kt, Kt, 2), g.b_lo, g.b_hi);
  span(b.Y, mat_bytes(b.Mc, b.N, b.N, a.out_bytes), g.c_lo, g.c_hi);
  span(b.bias, (uint64_t)b.N * 4, g.bias_lo, g.bias_hi);
  span(b.idx, (uint64_t)b.Mc * 4, g.gidx_lo, g.gidx_hi);
  span(a.P, (uint64_t)b.U * b.N * 4, g.p_lo, g.p_hi);
  span(b.workspace, b.sync_bytes + (uint64_t)(1 + b.S) * b.U * b.N * 4, g.w_lo, g.w_hi);
  return launch_persistent<C, IkboSched>(a, (int64_t)a.T_dyn + (int64_t)a.tiles_m * a.tiles_n, stream);
}

hipError_t launch_broadcast_single(const BroadcastLaunch& b, hipStream_t stream) {
  if (b.Mc == 0 || b.N == 0) return hipSuccess;
  return b.b_kn ? launch_broadcast_single_cfg<CfgLarge<true>>(b, stream)
                : launch_broadcast_single_cfg<CfgLarge<false>>(b, stream);
}

// m-tiles per band of the grouped tile order
constexpr int kGroupedBandM = 8;

template <class C>
static hipError_t launch_grouped_cfg(const GroupedLaunch& g, hipStream_t stream) {
  GroupedSched::Args a;
  a.X = reinterpret_cast<const __bf16*>(g.X);
  a.W = reinterpret_cast<const __bf16*>(g.W);
  a.Y = reinterpret_cast<char*>(g.Y);
  a.bias = g.bias;
  a.offsets = g.offsets;
  a.M_total = g.M_total;
  a.G = g.G; a.N = (int32_t)g.N; a.K = (int32_t)g.K;
  a.tiles_n = (int32_t)((g.N + C::BN - 1) / C::BN);
  a.group_m = kGroupedBandM;
  a.epi = g.epi; a.out_f32 = g.out_f32; a.out_bytes = g.out_f32 ? 4 : 2;
  a.split_sync = nullptr;
  a.split_images = nullptr;
  a.epoch = g.epoch;
  Guards& gd = a.guard;
  gd = Guards{};
  const int cus = device_cus();
  if (g.workspace && g.ws_bytes >= grouped_split_workspace_bytes(cus)) {
    a.split_sync = reinterpret_cast<char*>(g.workspace);
    a.split_images = a.split_sync + grouped_split_sync_bytes(cus);
    span(g.workspace, grouped_split_workspace_bytes(cus), gd.w_lo, gd.w_hi);
  }
  span(g.X, (uint64_t)g.M_total * g.K * 2, gd.a_lo, gd.a_hi);
  span(g.W, (uint64_t)g.G * g.K * g.N * 2, gd.b_lo, gd.b_hi);
  span(g.Y, (uint64_t)g.M_total * g.N * a.out_bytes, gd.c_lo, gd.c_hi);
  span(g.bias, (uint64_t)g.G * g.N * 4, gd.bias_lo, gd.bias_hi);
  // every group adds at most one partial m-tile
  const int64_t max_tiles = ((g.M_total + C::BM - 1) / C::BM + g.G) * a.tiles_n;
  return launch_persistent<C, GroupedSched>(a, max_tiles, stream);
}

hipError_t launch_grouped(const GroupedLaunch& g, hipStream_t stream) {
  if (g.M_total == 0 || g.N == 0) return hipSuccess;
  return g.b_kn ? launch_grouped_cfg<CfgGrouped<true>>(g, stream) : launch_grouped_cfg<CfgGrouped<false>>(g, stream);
}

hipError_t launch_grouped_wgrad(const WgradLaunch& w, hipStream_t stream) {
  using C = CfgWgrad;
  if (w.K == 0 || w.N == 0) return hipSuccess;
  WgradSched::Args a;
  a.X = reinterpret_cast<const __bf16*>(w.X);
  a.dY = reinterpret_cast<const __bf16*>(w.dY);
  a.dW = reinterpret_cast<char*>(w.dW);
  a.offsets = w.offsets;
  a.queue = reinterpret_cast<uint32_t*>(w.workspace);
  a.M_total = w.M_total;
  a.G = w.G; a.K = (int32_t)w.K; a.N = (int32_t)w.N;
  a.tiles_m = (int32_t)((w.K + C::BM - 1) / C::BM);
  a.tiles_n = (int32_t)((w.N + C::BN - 1) / C::BN);
  // XCD blocks: the split that reads X and dY into the fewest L2s (pn copies of X, pm of dY),
  // preferring splits that cut the tile grid evenly
  {
    static const int32_t splits[4][2] = {{8, 1}, {4, 2}, {2, 4}, {1, 8}};
    double best = 0;
    int bi = -1;
    for (int pass = 0; pass < 2 && bi < 0; ++pass) {
      for (int i = 0; i < 4; ++i) {
        const int32_t pm = splits[i][0], pn = splits[i][1];
        if (pass == 0 && (a.tiles_m % pm != 0 || a.tiles_n % pn != 0)) continue;
        const double cost = (double)pn * (double)w.K + (double)pm * (double)w.N;
        if (bi < 0 || cost < best) { best = cost; bi = i; }
      }
    }
    a.pm = splits[bi][0];
    a.pn = splits[bi][1];
  }
  a.epi = 0; a.out_f32 = w.out_f32; a.out_bytes = w.out_f32 ? 4 : 2;
  Guards& gd = a.guard;
  gd = Guards{};
  span(w.X, (uint64_t)w.M_total * w.K * 2, gd.a_lo, gd.a_hi);
  span(w.dY, (uint64_t)w.M_total * w.N * 2, gd.b_lo, gd.b_hi);
  span(w.dW, (uint64_t)w.G * w.K * w.N * a.out_bytes, gd.c_lo, gd.c_hi);
  hipLaunchKernelGGL(arm_queue_kernel, dim3(1), dim3(64), 0, stream, a.queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_persistent<C, WgradSched>(a, (int64_t)a.G * a.tiles_m * a.tiles_n, stream);
}

hipError_t launch_batch(const BatchLaunch& b, hipStream_t stream) {
  using C = CfgBatch;
  static_assert(C::BM == kBatchBM && C::BN == kBatchBN, "batch prefix tile shape");
  const char* ws = reinterpret_cast<const char*>(b.workspace);
  BatchSched::Args a;
  a.hdr = reinterpret_cast<const BatchHeader*>(ws);
  a.prefix = reinterpret_cast<const int32_t*>(ws + sizeof(BatchHeader));
  a.probs = reinterpret_cast<const BatchProblem*>(ws + sizeof(BatchHeader) + batch_prefix_bytes(b.count));
  a.count = b.count;
  a.epi = b.epi; a.out_f32 = b.out_f32; a.out_bytes = b.out_f32 ? 4 : 2;
  // The problems' pointers come from the host-validated table that prepare wrote, together
  // with the union of their address ranges (read by the kernel from the header).
  a.guard_ptr = reinterpret_cast<const Guards*>(ws + offsetof(BatchHeader, guard));
  // the tile count lives on the device: launch one workgroup per CU, idle ones exit at once
  return launch_persistent<C, BatchSched>(a, (int64_t)1 << 30, stream);
}

// ---------------------------------------------------------------------------------------
// Validation kernels for device-resident preconditions
// ---------------------------------------------------------------------------------------
// Result words of the check kernels (one per check in flight; no allocation).  A check claims
// a free word under a lock and releases it after its stream has been synchronised.
__device__ int32_t g_check_words[kCheckWords];

namespace {
std::mutex g_check_mu;
bool g_check_busy[kCheckWords];
std::vector<int32_t*> g_check_base;  // per device: device address of g_check_words
}  // namespace

__global__ void clear_word_kernel(int32_t* w) {
  if (threadIdx.x == 0) *w = 0;
}

__global__ void check_offsets_kernel(const int32_t* off, int32_t G, int64_t M_total, int32_t* flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i > G) return;
  bool bad = false;
  if (i == 0 && off[0] != 0) bad = true;
  if (i == G && (int64_t)off[G] != M_total) bad = true;
  if (i < G && off[i + 1] < off[i]) bad = true;
  if (bad) atomicOr(flag, 1);
}

__global__ void check_index_kernel(const int32_t* idx, int64_t n, int64_t U, int32_t* flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t v = idx[i];
  if (v < 0 || (int64_t)v >= U) atomicOr(flag, 1);
}

template <class Launch>
static hipError_t run_check(hipStream_t stream, int* bad, int* busy, Launch launch) {
  *bad = 0;
  *busy = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int slot = -1;
  int32_t* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_check_mu);
    if ((int)g_check_base.size() <= dev) g_check_base.resize(dev + 1, nullptr);
    if (!g_check_base[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check_words));
      if (e != hipSuccess) return e;
      g_check_base[dev] = static_cast<int32_t*>(p);
    }
    base = g_check_base[dev];
    for (int i = 0; i < kCheckWords; ++i) {
      if (!g_check_busy[i]) {
        g_check_busy[i] = true;
        slot = i;
        break;
      }
    }
  }
  if (slot < 0) {
    *busy = 1;
    return hipSuccess;
  }
  int32_t* flag = base + slot;
  int32_t h = 0;
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, stream, flag);
  e = hipGetLastError();
  if (e == hipSuccess) e = launch(flag);
  if (e == hipSuccess) e = hipMemcpyAsync(&h, flag, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  *bad = (e == hipSuccess && h != 0) ? 1 : 0;
  {
    std::lock_guard<std::mutex> lock(g_check_mu);
    g_check_busy[slot] = false;
  }
  return e;
}

hipError_t check_offsets(const int32_t* offsets, int32_t G, int64_t M_total, hipStream_t stream, int* bad,
                         int* busy) {
  return run_check(stream, bad, busy, [&](int32_t* flag) {
    const int64_t n = (int64_t)G + 1;
    hipLaunchKernelGGL(check_offsets_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       offsets, G, M_total, flag);
    return hipGetLastError();
  });
}

hipError_t check_index(const int32_t* idx, int64_t n, int64_t U, hipStream_t stream, int* bad, int* busy) {
  return run_check(stream, bad, busy, [&](int32_t* flag) {
    hipLaunchKernelGGL(check_index_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       idx, n, U, flag);
    return hipGetLastError();
  });
}

hipError_t read_watchdog(uint32_t* value, int clear) {
  hipError_t e = hipMemcpyFromSymbol(value, HIP_SYMBOL(g_watchdog), sizeof(uint32_t), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_watchdog), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice);
}

}  // namespace ptg

