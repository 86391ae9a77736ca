// ptg_device.hpp - gfx950 device code of the pipelined tiled GEMM.
//
// One persistent workgroup per compute unit runs a three-role software pipeline, the
// structure of listing 2 in "How We Built TLX" (section "Introducing TLX"): producer waves
// move A and B tiles into a multistage LDS ring, consumer waves run the matrix cores on
// the staged tiles, and an epilogue stage turns the fp32 accumulators into the output.
// The page's roles are re-expressed for CDNA4:
//   - Producer waves issue buffer loads that write straight into LDS (16 bytes per lane,
//     bypassing registers), the gfx950 counterpart of an asynchronous tile copy.  Each
//     producer tracks its copies with the vector-memory counter and then bumps the slot's
//     "full" counter in LDS.
//   - The ring's handoff uses monotone LDS counters instead of hardware barriers: slot
//     s = g mod STAGES holds k-step g; "full[s]" counts producer arrivals and "empty[s]"
//     counts consumer releases.  A producer never refills a slot before every consumer has
//     released it, and a consumer never reads a slot before every producer has filled it
//     (the multistage-buffer rule; the yuxiaoba.github.io reading notes on the post, section
//     "Tensor expressions with explicit handoffs").  Counters only grow, so no phase bit is
//     needed.
//   - Consumer waves read operand fragments with ds_read_b128 (K-contiguous tiles) or the
//     transposing ds_read_b64_tr_b16 (N-contiguous tiles), issue v_mfma_f32_32x32x16_bf16
//     into fp32 accumulators held in registers, release the slot as soon as the last
//     fragment of a k-step has landed in registers, and run the epilogue on their own
//     accumulators (a wave cannot hand 64 KB of accumulators to another wave on CDNA4).
//   - The producer is also the tile scheduler: it publishes each tile's epilogue metadata
//     in a small LDS ring next to the data, so the consumers never wait on global memory
//     for scheduling and the pipeline keeps running across tile (and problem) boundaries.
//
// Layouts in LDS.  A tile is BM rows of BK bf16 (K contiguous).  A B tile is BN rows of
// BK (layout NK) or BK rows of BN (layout KN).  Rows are cut in 16-byte chunks and the
// chunk index is XOR-swizzled with a function of the row, so that the fragment reads of
// one MFMA operand hit distinct LDS banks; the producer realises the swizzle by choosing
// which global chunk each lane fetches (the LDS side of a DMA load is always linear).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ptg_launch.h"

namespace ptg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
// (Vectors are reinterpreted whole: this compiler's __builtin_bit_cast of a subscripted vector
// element reads element 0 whatever the subscript.)
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

enum : int { EPI_NONE = 0, EPI_BIAS = 1, EPI_SILU = 2, EPI_BIAS_SILU = 3 };
enum : int { OUT_BF16 = 0, OUT_F32 = 1 };

// A voffset at or above 2^31 is outside every buffer descriptor built here (their record
// counts stay below 2^31), so the DMA writes zeros: used for rows, columns and k beyond
// the problem.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Upper bound on the polls of one wait: each poll is an LDS read plus a ~64-clock sleep,
// so 2^20 polls last tens of milliseconds, far beyond any wait of a working pipeline
// (microseconds).  A wait that gives up raises the workgroup's abort word, so that every
// other wait of the workgroup returns at once, and records the event in g_watchdog for the
// host; the kernel then finishes (with wrong results) instead of hanging.
constexpr uint32_t kSpinLimit = 1u << 20;

// ---------------------------------------------------------------------------------------
// Tile configuration
// ---------------------------------------------------------------------------------------
template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_, int NPROD_, bool B_KN_, int PREG_ = 0,
          bool M16_ = false, bool A_KM_ = false, bool STREAM_OUT_ = false, int CG_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  // k-steps a producer holds in registers ahead of the LDS ring (0: tiles go straight from
  // memory into LDS)
  static constexpr int PREG = PREG_;
  // Matrix instruction: v_mfma_f32_16x16x32_bf16 (true) or v_mfma_f32_32x32x16_bf16 (false).
  // Same flops per cycle; the 16x16 form moves a quarter of the accumulator registers per
  // MFMA (a third less register traffic per flop), which on random data lets the part hold a
  // higher clock under the same power.
  static constexpr bool M16 = M16_;
  static constexpr int WM = WM_, WN = WN_;             // consumer waves along M and N
  // Consumer groups ("ping-pong"): group c runs the tiles j with j mod CG = c, so that one
  // group's epilogue (conversion and output stores) overlaps the other group's matrix work.
  // Every step is released by the NCG waves of the group that runs its tile.
  static constexpr int CG = CG_;
  static constexpr int NCG = WM * WN;                   // consumer waves per group
  static constexpr int NCONS = NCG * CG, NPROD = NPROD_;
  static constexpr int NWAVES = NCONS + NPROD, NT = NWAVES * 64;
  static constexpr bool B_KN = B_KN_;
  // A stored with k as the row index (K x M, M contiguous), as X^T is in a weight gradient
  // X^T . dY: its tile is staged as BK rows of BM and read with transposing LDS reads.
  static constexpr bool A_KM = A_KM_;
  // Output written as streaming (non-temporal) stores of whole 128-byte row segments instead
  // of 64-byte halves; measured faster wherever the output is a sizeable part of the traffic
  // (weight gradient, broadcast candidates, grouped and dense GEMMs).  16x16 consumer only.
  static constexpr bool STREAM_OUT = STREAM_OUT_;
  static constexpr int WTM = BM / WM, WTN = BN / WN;    // one consumer wave's sub-tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int KSUB = BK / 16;                  // MFMA k-steps per ring slot
  static constexpr int TM16 = WTM / 16, TN16 = WTN / 16;  // 16x16 blocks per wave (M16)
  static constexpr int KS = BK / 32;                     // 32-deep k-slices per ring slot (M16)
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024, B_INSTR = B_BYTES / 1024;  // 1 KB per DMA
  static constexpr int LOADS = (A_INSTR + B_INSTR) / NPROD;  // 1 KB loads per producer per k-step
  // k-steps a producer keeps in flight before it waits for the oldest to land (bounded by
  // the ring and by the 6-bit vector-memory counter)
  static constexpr int INFLIGHT = (STAGES < 63 / LOADS) ? STAGES : 63 / LOADS;
  static constexpr int CPR_A = A_KM ? BM / 8 : BK / 8;  // 16-byte chunks per A row
  static constexpr int CPR_B = B_KN ? BN / 8 : BK / 8;  // 16-byte chunks per B row
  // rows covered by two consecutive 1 KB loads (one load covers 64 chunks)
  static constexpr int ROWS_A = 128 / CPR_A, ROWS_B = 128 / CPR_B;
  // Tile-metadata slots.  Slot j mod NINFO holds tile j's metadata from the moment the
  // producer starts fetching the tile until its epilogue is done.  The producer writes the
  // slot for tile j + NINFO while it fetches a step at most PREG + 1 steps ahead of the ring
  // slot it fills last, and it fills that slot only after the release of the step STAGES
  // earlier; with NINFO = STAGES + PREG + 3, that released step belongs to tile j + 1 or a
  // later one (every tile has at least one step), so the consumers have finished tile j,
  // epilogue included.  With two consumer groups, the group in tile j's epilogue holds back
  // the steps of its next tile, j + 2, so the ring (filled in order) cannot pass j + 2 by more
  // than STAGES steps: two more slots cover it.
  static constexpr int NINFO = STAGES + PREG + 3 + 2 * (CG - 1);
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "consumer sub-tile must be 32x32 blocks");
  static_assert(!M16 || (TM16 % 2 == 0 && TN16 % 2 == 0 && BK % 32 == 0), "16x16 path: even block counts, BK of 64");
  static_assert(BK % 16 == 0 && (BK == 32 || BK == 64), "BK must be 32 or 64");
  static_assert((A_INSTR + B_INSTR) % NPROD == 0, "DMAs must split evenly over producers");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "tiles must be whole KB");
  static_assert(LOADS <= 63, "one k-step of DMAs must fit the vector-memory counter");
  static_assert(STAGES >= 2, "the ring needs at least two slots");
  static_assert(INFLIGHT >= 1 && INFLIGHT <= STAGES, "in-flight steps are bounded by the ring");
  static_assert(PREG == 0 || PREG == 1, "0: memory to LDS; 1: one step staged in registers");
  static_assert(PREG == 0 || LOADS * 4 <= 128, "a register-staged step must fit the producer's registers");
  static_assert(NT <= 1024, "workgroup too large");
  static_assert(CG == 1 || CG == 2, "one or two consumer groups");
  static_assert(!A_KM || (M16 && PREG == 1 && (TM16 & (TM16 - 1)) == 0),
                "A stored K x M: register-staged producers and the 16x16 consumer, TM16 a power of two");
  static_assert(!STREAM_OUT || (M16 && TN16 == 4), "streaming output: 16x16 consumer, 64 columns per wave");
};

// k-steps of a tile with reduction length K.  A tile always has at least one step: an empty
// reduction (K = 0, only the weight gradient of an expert without rows has one) runs one
// step of zeros, so the ring's counting (one handoff per step) and the metadata slots'
// lifetime rule hold for every tile, and the epilogue stores zeros.
template <class C>
__host__ __device__ constexpr int tile_steps(int K) {
  return K > 0 ? (K + C::BK - 1) / C::BK : 1;
}

// Chunk swizzle for rows of BK bf16 (K contiguous), CPR chunks per row.  For 8 lanes
// reading rows r..r+7 (and for 16 lanes reading r..r+15) at one logical chunk, the
// physical chunks land in distinct 16-byte bank groups.
template <int CPR>
__host__ __device__ constexpr int swz_k(int r) {
  if constexpr (CPR == 8) {
    return ((r >> 1) ^ ((r & 1) << 2)) & 7;
  } else {
    static_assert(CPR == 4, "BK of 32 or 64");
    return ((r >> 2) ^ (r >> 1)) & 3;
  }
}

// Chunk swizzle for rows of BN bf16 (N contiguous, layout KN; also A stored K x M), CPR
// chunks per row.  A transposing read takes 4 consecutive k-rows x 32 bytes per 16 lanes; the
// XOR values of 4 consecutive rows differ in bits 1-2 and in bits 2-3 so that both 16- and
// 32-lane service groups see distinct banks.  Bit 3 of k flips bit 1 of the XOR: the 16x16
// consumer's two 16-lane groups of a 32-lane service group read the same columns of rows
// 8 apart (k-values 0-7 and 8-15 of a 32-deep slice), which then land on the other 8 chunk
// pairs of the row instead of the same banks.
template <int CPR>
__host__ __device__ constexpr int swz_n(int k) {
  if constexpr (CPR >= 16) {
    const int m = k & 3;  // 0, 6, 10, 12 for m = 0..3, then XOR 2 when bit 3 of k is set
    return ((m & 1) * 6) ^ ((m & 2) * 5) ^ (((k >> 3) & 1) << 1);
  } else {
    static_assert(CPR == 8, "BN of 64 or more");
    return (k & 3) << 1;
  }
}

// ---------------------------------------------------------------------------------------
// Tile metadata, published by the producer and read by the consumers
// ---------------------------------------------------------------------------------------
struct TileInfo {            // 16 dwords
  uint32_t tag;              // tile_tag(j) for tile j, end_tag(j) when no tile j exists
  int32_t K;                 // reduction length of this tile's problem
  int32_t m_rows, n_cols;    // valid rows / columns of the tile (<= BM, BN)
  uint64_t C;                // address of the tile's first output element
  int64_t ldc;               // output row stride in elements
  uint64_t bias;             // address of bias[n0] or 0
  uint64_t gidx;             // address of idx[m0] (broadcast gather) or 0
  uint64_t P;                // address of P[0][n0] (broadcast gather) or 0
  int32_t ldp;               // row stride of P in elements
  uint32_t p_bytes;          // bytes of P from P[0][n0] on (bounds of the gather)
  // Reduction split (grouped GEMM, last round): 0 for a whole tile; 1 or 2 for the unit that
  // reduces the first or second part of k of a tile split in two.  The two units' fp32
  // partial sums meet in the workspace (combine_split16).
  uint32_t mode;
  uint32_t epoch;            // the launch's epoch: sync words left by other launches never match
  uint64_t part;             // workspace: the tile's partial image (32 KB per consumer wave), or
                             // (reduction unit) its rows of the first partial product
  uint64_t sync;             // workspace: split tiles: per consumer wave, a 64-bit arrival word, then
                             // a 32-bit ready word; broadcast modes: the column block's arrival
                             // word, its ready word 8 bytes further
  uint32_t count;            // reduction unit: partial products to sum; candidate: ready count to await
  uint32_t stride;           // reduction unit: elements between consecutive partial products
};
static_assert(sizeof(TileInfo) == 96, "TileInfo is 24 dwords");

// Tile modes (TileInfo::mode).  0: a whole tile.  1, 2: the two units of a tile whose
// reduction is split (grouped GEMM, combine_split16).  The single-launch broadcast GEMM adds:
//   3: a user-phase partial product: fp32 output, no epilogue operation, agent-coherent stores,
//      then every consumer wave counts itself into the tile's arrival word (`sync`);
//   4: a reduction unit: no matrix work (one empty k-step); the producer waves wait until every
//      partial product of its column block has arrived, sum them in split order, add the bias,
//      write its rows of P, then count themselves into the column block's ready word;
//   5: a candidate tile: published to the consumers only once its column block's P is ready;
//      the accumulators start from P (agent-coherent loads).
constexpr uint32_t kModeUserPartial = 3, kModeReduce = 4, kModeCandidate = 5;
// The kinds of tiles a scheduler hands out (its kModes), so that a consumer compiles in only
// the code for those: whole tiles only, or also split tiles (1, 2), or also the broadcast
// modes (3-5).  The others cost its kernel no registers.
constexpr int kModesNone = 0, kModesSplit = 1, kModesBroadcast = 2;

// Tags of a metadata slot.  The consumer checks the tag of the slot it expects before it
// uses any address from it: a slot that is not exactly what the producer published stops
// the workgroup (abort word, watchdog bit 2) instead of steering stores.
__host__ __device__ constexpr uint32_t tile_tag(int j) { return 0x50544700u ^ ((uint32_t)j * 2654435761u); }
__host__ __device__ constexpr uint32_t end_tag(int j) { return 0x454e4400u ^ ((uint32_t)j * 2246822519u); }

// What the producer needs to fetch a tile (never leaves the producer's registers).
struct TileSrc {
  const __bf16* A;   // first row of the tile
  int64_t lda;
  const __bf16* B;   // first row (NK) or first column (KN) of the tile
  int64_t ldb;
  TileInfo info;
};

// Every descriptor a workgroup builds must lie inside the range (Guards, ptg_launch.h) of
// its operand; one that does not (never the case in a working pipeline) aborts the
// workgroup before any access.
__device__ __forceinline__ bool inside(uint64_t p, uint64_t bytes, uint64_t lo, uint64_t hi) {
  return p >= lo && p <= hi && bytes <= hi - p;
}

// ---------------------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------------------
// Lane index from the lane-mask counter (a function of the lane alone, so the compiler can
// recompute it where needed instead of keeping the thread index live).
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// A copy of x that the compiler cannot see through: index arithmetic derived from it is
// recomputed where it is used instead of being hoisted out of loops and kept live.
__device__ __forceinline__ int opaque(int x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// The lane index, computed afresh where it is used (nothing stays live before that point).
__device__ __forceinline__ int opaque_lane() {
  int x;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The ring counters are touched with hand-issued LDS instructions.  Compiler-issued LDS
// accesses after a DMA-to-LDS load make the compiler wait for every outstanding DMA
// (it cannot tell the counters from the ring), which would serialise the producer; the
// asm versions carry their own waits, and LDS executes one wave's accesses in order.
__device__ __forceinline__ uint32_t lds_peek(const uint32_t* p) {
  uint32_t v;
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// Ring stress build (compiled with PTG_DELAY_INJECT=1 into a separate test library, never
// into the product): every handoff, each release or fill signal and each wait, first pauses
// for a pseudo-random 0 to 8192 shader cycles (a hash of the cycle counter, the same on
// every lane of the wave), so producers and consumers meet the ring in orders a natural run
// rarely produces.  The handoff rule must hold under any timing; results stay bit-identical.
#ifndef PTG_DELAY_INJECT
#define PTG_DELAY_INJECT 0
#endif
__device__ __forceinline__ void stress_pause() {
#if PTG_DELAY_INJECT
  const uint64_t t = __builtin_amdgcn_s_memtime();
  uint32_t h = (uint32_t)t * 2654435761u ^ (uint32_t)(t >> 9);
  h ^= h >> 15;
  const uint32_t r = (h >> 8) & 15u;
  for (uint32_t i = 8; i < r + 1; ++i) __builtin_amdgcn_s_sleep(16);  // r >= 8: 1 to 8 x 1024 cycles
#endif
}

__device__ __forceinline__ void lds_bump(uint32_t* p) {
  stress_pause();
  __asm__ volatile("" ::: "memory");
  if (lane_id() == 0) {
    const uint32_t one = 1;
    __asm__ volatile("ds_add_u32 %0, %1" : : "v"(lds_addr(p)), "v"(one) : "memory");
  }
}

__device__ __forceinline__ uint64_t lds_peek64(const uint64_t* p) {
  uint64_t v;
  __asm__ volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

__device__ __forceinline__ void lds_put64(uint64_t* p, uint64_t v) {
  __asm__ volatile("" ::: "memory");
  if (lane_id() == 0) __asm__ volatile("ds_write_b64 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// One watchdog word per translation unit (each .hip file is its own code object, so the word
// has internal linkage and each file reads its own back through read_watchdog*).
static __device__ uint32_t g_watchdog = 0;

// MI300-class parts hand workgroups of one dispatch to their XCDs round-robin (8 XCDs
// on MI355X).  Renumbering so that consecutive tile indices land on one XCD lets tiles that
// share A rows or B columns meet in that XCD's L2.
__device__ __forceinline__ int64_t xcd_rank(int w, int grid) {
  return (grid % 8 == 0) ? (int64_t)(w % 8) * (grid / 8) + w / 8 : (int64_t)w;
}

// Stop the workgroup: raise its abort word (every wait returns at once) and record `why`
// in the device watchdog word (1: a wait timed out, 2: inconsistent tile metadata, 4: a DMA
// source outside its operand, 8: an epilogue access outside its operand).
__device__ __forceinline__ void raise_abort(uint32_t* abort, uint32_t why) {
  if (lane_id() == 0) {
    const uint32_t one = 1;
    __asm__ volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(abort)), "v"(one) : "memory");
    atomicOr(&g_watchdog, why);
  }
}

// Wait until a monotone LDS counter reaches `target`; bounded (see kSpinLimit).
__device__ __forceinline__ void wait_at_least(const uint32_t* p, uint32_t target, uint32_t* abort) {
  stress_pause();
  uint32_t polls = 0;
  while ((uint32_t)__builtin_amdgcn_readfirstlane(lds_peek(p)) < target) {
    __builtin_amdgcn_s_sleep(1);
    if ((++polls & 63) == 0) {
      if ((uint32_t)__builtin_amdgcn_readfirstlane(lds_peek(abort)) != 0) break;
      if (polls >= kSpinLimit) {
        raise_abort(abort, 1u);
        break;
      }
    }
  }
  __asm__ volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_lgkm0() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Wave-uniform copies of a value.  The builtin returns a signed int: it is converted to
// uint32_t before any widening, so that a low address word with bit 31 set is never
// sign-extended into the high word.
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uni64(uint64_t x) {
  return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | (uint64_t)uni((uint32_t)x);
}

// Counters shared by the workgroups of one launch live in global memory as 64-bit words:
// the launch's epoch in the high half and a count in the low half.  A word left by another
// launch counts as zero, so no launch has to clear them.  They are touched by one lane with
// agent-scope atomics (vector memory instructions, coherent across the XCDs).
// Adds one within `epoch` and returns the count before: a fetch-and-add, and when the word
// still holds another launch's epoch, a compare-and-swap that starts this epoch at one (a
// fetch-and-add that landed on the old epoch is discarded with it and retried).
__device__ __forceinline__ uint32_t epoch_add(uint64_t* w, uint32_t epoch) {
  uint64_t old = __hip_atomic_fetch_add(w, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((uint32_t)(old >> 32) != epoch) {
    uint64_t cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(cur >> 32) == epoch) {
      old = __hip_atomic_fetch_add(w, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    if (__hip_atomic_compare_exchange_strong(w, &cur, ((uint64_t)epoch << 32) | 1u, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      return 0u;
  }
  return (uint32_t)old;
}

__device__ __forceinline__ uint32_t epoch_count(const uint64_t* w, uint32_t epoch) {
  const uint64_t v = __hip_atomic_load(const_cast<uint64_t*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (uint32_t)(v >> 32) == epoch ? (uint32_t)v : 0u;
}

// Lane 0 waits (bounded, see kSpinLimit) until the word's count in `epoch` reaches `target`;
// returns false, with the workgroup aborted, when the wait gives up or the workgroup aborts.
// Polls are about a thousand clocks apart: many workgroups may poll one word, and a line
// read that often slows every other access that goes to its memory channel.
__device__ __forceinline__ bool epoch_wait(const uint64_t* w, uint32_t epoch, uint32_t target, uint32_t* abort) {
  uint32_t ok = 1;
  if (lane_id() == 0) {
    uint32_t polls = 0;
    while (epoch_count(w, epoch) < target) {
      __builtin_amdgcn_s_sleep(16);
      if ((++polls & 63) == 0 && (lds_peek(abort) != 0 || polls >= kSpinLimit)) {
        ok = 0;
        break;
      }
    }
  }
  if (uni(ok) == 0) {
    raise_abort(abort, 1u);
    return false;
  }
  return true;
}

// Buffer descriptor over [base, base + nbytes).  Base and size are wave-uniform by
// construction; reading them through readfirstlane keeps the descriptor in scalar registers
// (a descriptor the compiler believes divergent costs a loop around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t ub = uni64(reinterpret_cast<uint64_t>(base));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ub), (short)0, (int)uni(nbytes),
                                           0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ float silu(float v) {
  // e^-v as 2^(-v log2 e) on the hardware exp2; v / (1 + e^-v) is then v * sigmoid(v).
  const float e = __builtin_amdgcn_exp2f(-v * 1.4426950408889634f);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Two floats to two bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------------------
// Producer role
// ---------------------------------------------------------------------------------------
// Producer p owns DMA indices [p * LOADS, (p + 1) * LOADS) of every k-step: index i < A_INSTR
// copies 1 KB of the A tile, the rest copy the B tile.  Lane l of DMA i fills LDS bytes
// [1024 i + 16 l, +16) of the slot, i.e. physical chunk P = 64 i + l of the tile.
template <class C>
__host__ __device__ constexpr void chunk_of(int i, int lane, int& row, int& chunk) {
  if (i < C::A_INSTR) {
    const int P = i * 64 + lane;
    row = P / C::CPR_A;  // m-row (A stored M x K) or k-row (K x M)
    if constexpr (C::A_KM) chunk = (P % C::CPR_A) ^ swz_n<C::CPR_A>(row);
    else chunk = (P % C::CPR_A) ^ swz_k<C::CPR_A>(row);
  } else {
    const int P = (i - C::A_INSTR) * 64 + lane;
    row = P / C::CPR_B;  // n-row (NK) or k-row (KN)
    if constexpr (C::B_KN) chunk = (P % C::CPR_B) ^ swz_n<C::CPR_B>(row);
    else chunk = (P % C::CPR_B) ^ swz_k<C::CPR_B>(row);
  }
}

// Load q of a producer (index i0 + q) fetches, for every lane, the chunk of load q mod 2 (its
// first two loads), (q / 2) ROWS_A or ROWS_B rows further on; for an operand stored with k as
// the row index the chunk also flips bit 1 when that row offset has bit 3 set (bit 3 of the
// k-row, see swz_n; a producer's first row is a multiple of 16).  Two per-lane bases, a row
// step and a per-lane flip offset then describe all of a producer's loads.  Checked at
// compile time for each configuration that stages through registers.
template <int ROWS>
constexpr bool row_flip(int q) {
  return (((q >> 1) * ROWS) >> 3) & 1;
}

template <class C>
constexpr bool load_flip(int i, int q) {
  return (i < C::A_INSTR) ? (C::A_KM && row_flip<C::ROWS_A>(q)) : (C::B_KN && row_flip<C::ROWS_B>(q));
}

template <class C>
constexpr bool chunk_pattern_ok() {
  for (int p = 0; p < C::NPROD; ++p) {
    const int i0 = p * C::LOADS;
    for (int q = 0; q < C::LOADS; ++q) {
      const int i = i0 + q;
      const int rows = (i < C::A_INSTR) ? C::ROWS_A : C::ROWS_B;
      for (int lane = 0; lane < 64; ++lane) {
        int rb = 0, cb = 0, r = 0, c = 0;
        chunk_of<C>(i0 + (q & 1), lane, rb, cb);
        chunk_of<C>(i, lane, r, c);
        if (r != rb + (q >> 1) * rows || c != (cb ^ (load_flip<C>(i, q) ? 2 : 0))) return false;
      }
    }
  }
  return true;
}

template <class C, class S>
__device__ __forceinline__ void producer_role(const typename S::Args& args, char* ring, TileInfo* info,
                                              uint32_t* full, uint32_t* empty, uint32_t* abort, int pid,
                                              char* sched_lds, const Guards* guards) {
  static_assert(C::A_INSTR % C::LOADS == 0, "each producer copies either A or B chunks");
  static_assert(!C::A_KM, "A stored K x M is staged through registers (producer_role_regs)");
  static_assert(!S::kDynamic, "dynamic tile queues are served by producer_role_regs");
  const int lane = lane_id();
  const int i0 = pid * C::LOADS;
  const bool opA = i0 < C::A_INSTR;                 // this producer's operand
  const int lds_base = opA ? i0 * 1024 : C::A_BYTES + (i0 - C::A_INSTR) * 1024;
  uint32_t g = 0;         // k-steps issued by this workgroup so far (all tiles)
  uint32_t next_sig = 0;  // oldest k-step whose "full" has not been signalled
  for (int j = 0;; ++j) {
    TileSrc t = {};
    const bool has = S::template tile<C>(args, j, t, sched_lds);
    // Per-lane byte offset of each of this producer's chunks; rows/columns outside the
    // problem get an out-of-range offset, so the DMA writes zeros there.
    uint32_t voff[C::LOADS];
    const void* src = nullptr;
    uint32_t src_bytes = 0;
    int64_t k_stride = 2;   // bytes per unit of k along the operand (for the k-step offset)
    int nsteps = 1;
    if (has) {
      const int K = t.info.K;
      nsteps = tile_steps<C>(K);
      if (opA) {
        src = t.A;
        src_bytes = (uint32_t)((int64_t)(t.info.m_rows - 1) * t.lda * 2 + (int64_t)K * 2);
      } else {
        src = t.B;
        src_bytes = C::B_KN ? (uint32_t)((int64_t)(K - 1) * t.ldb * 2 + (int64_t)t.info.n_cols * 2)
                            : (uint32_t)((int64_t)(t.info.n_cols - 1) * t.ldb * 2 + (int64_t)K * 2);
        if (C::B_KN) k_stride = t.ldb * 2;
      }
      const uint64_t lo = uni64(opA ? guards->a_lo : guards->b_lo);
      const uint64_t hi = uni64(opA ? guards->a_hi : guards->b_hi);
      if (!inside(reinterpret_cast<uint64_t>(src), src_bytes, lo, hi)) {
        raise_abort(abort, 4u);
        src_bytes = 0;  // every copy of this tile is out of range: nothing is read
      }
#pragma unroll
      for (int q = 0; q < C::LOADS; ++q) {
        const int i = i0 + q;
        int row, c;
        chunk_of<C>(i, lane, row, c);
        bool ok;
        int64_t off;
        if (opA) {
          ok = row < t.info.m_rows;
          off = row * t.lda * 2 + c * 16;
        } else if (C::B_KN) {
          ok = c * 8 < t.info.n_cols;
          off = row * t.ldb * 2 + c * 16;
        } else {
          ok = row < t.info.n_cols;
          off = row * t.ldb * 2 + c * 16;
        }
        voff[q] = ok ? (uint32_t)off : kOutOfRange;
      }
    }
    for (int st = 0; st < nsteps; ++st, ++g) {
      const int s = g % C::STAGES;
      const uint32_t released = (uint32_t)C::NCG * (g / C::STAGES);
      if ((uint32_t)__builtin_amdgcn_readfirstlane(lds_peek(&empty[s])) < released) {
        // The slot is still in use: before sleeping on it, hand every step in flight to the
        // consumers as soon as it has landed, so that no step waits on a later issue.
        wait_vmcnt<0>();
        for (; next_sig < g; ++next_sig) lds_bump(&full[next_sig % C::STAGES]);
        wait_at_least(&empty[s], released, abort);
      }
      if (st == 0 && pid == 0 && lane == 0) {
        // publish this tile's metadata, or the end marker, in its info slot
        TileInfo ti = t.info;
        ti.tag = has ? tile_tag(j) : end_tag(j);
        info[j % C::NINFO] = ti;
      }
      if (has) {
        const int k0 = st * C::BK;
        const bool tail = k0 + C::BK > t.info.K;
        char* dst = ring + s * C::STAGE_BYTES + lds_base;
        // The k-step offset moves the descriptor's base (scalar arithmetic); the scalar
        // offset operand of the DMA stays 0: on gfx950 a nonzero one is not used with
        // buffer-to-LDS loads (it does not only move the global address).
        const int64_t kbytes = (int64_t)k0 * k_stride;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(static_cast<const char*>(src) + kbytes, src_bytes - (uint32_t)kbytes);
        const uint32_t soff = 0;
        if (!tail) {
#pragma unroll
          for (int q = 0; q < C::LOADS; ++q) dma16(rs, dst + q * 1024, voff[q], soff);
        } else {
          // the last, partial k-step: chunks past K are zero-filled
#pragma unroll
          for (int q = 0; q < C::LOADS; ++q) {
            int row, c;
            chunk_of<C>(i0 + q, lane, row, c);
            const int kpos = (!opA && C::B_KN) ? row : c * 8;
            dma16(rs, dst + q * 1024, k0 + kpos < t.info.K ? voff[q] : kOutOfRange, soff);
          }
        }
        // Steps next_sig .. g are in flight.  With INFLIGHT of them outstanding, wait until the
        // oldest has landed (the later ones may still be in flight: the vector-memory counter
        // retires loads in order) and hand it to the consumers.
        if (g + 1 - next_sig == (uint32_t)C::INFLIGHT) {
          wait_vmcnt<(C::INFLIGHT - 1) * C::LOADS>();
          lds_bump(&full[next_sig % C::STAGES]);
          ++next_sig;
        }
      } else {
        // the end marker: every step issued so far has landed, hand them all over
        wait_vmcnt<0>();
        for (; next_sig < g; ++next_sig) lds_bump(&full[next_sig % C::STAGES]);
      }
    }
    if (!has) break;
  }
  // the end marker's own step (it carries no data)
  lds_bump(&full[(g - 1) % C::STAGES]);
}

// Producer role with register staging (PREG = 1).  Each producer keeps its share of the
// next k-step in registers (buffer loads into VGPRs), ahead of the LDS ring: when a ring
// slot is released it writes the staged step into it with ds_write_b128, hands it over and
// at once issues the loads of the following step into the same registers.  A step's loads
// are thus issued one ring step earlier than a direct memory-to-LDS copy could issue them
// (that needs the slot already free), and memory latency hides behind one more step of the
// consumers' work.  The loads pick the same swizzled chunks as the DMA path, so the LDS
// image is identical.
//
// The fetch side runs one step ahead of the ring, across tile boundaries: it starts a tile
// (asks the scheduler, publishes the tile's metadata or the end marker) when it has fetched
// the previous tile's last step.

// What the fetch side keeps of the tile it fetches (every member is wave-uniform except the
// per-lane bases).
struct FetchTile {
  uint64_t src;         // operand base of the tile (A rows or B rows/columns)
  uint32_t bytes;       // bytes of the operand from src on, 0 when out of range
  uint32_t rstep;       // bytes between loads q and q + 2
  int64_t kstride;      // bytes per unit of k along the operand
  int K, nsteps;
  bool has;             // false: no tile, the end marker was published
  bool dead;            // every row of this producer's share lies past the tile's valid rows
                        // (m-rows of A, n-rows of B stored N x K): nothing to load or stage
  uint32_t vbase0, vbase1;  // per-lane offsets of this producer's loads 0 and 1
  int32_t vflip0, vflip1;   // byte offset added to load q (parity 0 or 1) when it flips (load_flip)
  int kbase0, kbase1;       // k (within a step) of loads 0 and 1; load q + 2 adds ROWS_A or
                            // ROWS_B k-rows when k is the operand's row index, else nothing
  // Narrow tile: k is the operand's row index and the tile has fewer valid columns than the
  // tile width, so loads of columns past `extent` would fetch the next tile's data; they take
  // an out-of-range offset instead.  col0 and col1 are this lane's first column in loads 0
  // and 1; a flipped load (load_flip) reads column col ^ 16.
  bool narrow;
  int extent, col0, col1;
};

// The tile a workgroup runs as its j-th.  A static scheduler derives it from j.  A dynamic one
// (S::kDynamic) hands out tickets: producer 0 takes the next one from counters in global
// memory (S::claim, vector atomics) and posts it, tagged with j + 1, in an LDS slot; the other
// producers wait for that tag.  Slot j mod kClaimSlots is rewritten for
// tile j + kClaimSlots only after every producer has fetched tile j: producers cannot drift
// further apart than the ring's depth in steps, and every tile has at least one step.
template <class C, class S>
__device__ __forceinline__ bool schedule_tile(const typename S::Args& args, int j, int pid, TileSrc& t,
                                              char* sched_lds, uint32_t* abort) {
  if constexpr (!S::kDynamic) {
    (void)pid;
    (void)abort;
    return S::template tile<C>(args, j, t, sched_lds);
  } else {
    static_assert(S::kClaimSlots >= C::NINFO + C::STAGES, "claim slots must outlive the producers' drift");
    uint64_t* slot = S::claim_slots(sched_lds) + (j % S::kClaimSlots);
    const uint32_t tag = (uint32_t)j + 1u;
    uint32_t pos;
    if (pid == 0) {
      uint32_t got = 0;
      if (lane_id() == 0) got = S::claim(args, sched_lds);
      pos = uni(got);
      lds_put64(slot, ((uint64_t)tag << 32) | pos);
    } else {
      uint32_t polls = 0;
      uint64_t v = lds_peek64(slot);
      while (uni((uint32_t)(v >> 32)) != tag) {
        __builtin_amdgcn_s_sleep(1);
        if ((++polls & 63) == 0) {
          if (uni(lds_peek(abort)) != 0) return false;
          if (polls >= kSpinLimit) {
            raise_abort(abort, 1u);
            return false;
          }
        }
        v = lds_peek64(slot);
      }
      pos = uni((uint32_t)v);
    }
    return S::template tile_at<C>(args, pos, t, sched_lds);
  }
}

// A reduction unit of the single-launch broadcast GEMM, run by the producer waves when they
// reach it (no ring data: its one k-step is empty).  Once every active consumer wave of every
// user-phase slice of its column block has published this launch's epoch in its arrival flag,
// producer p sums rows p, p + NPROD, ... of the slices' partial products in slice order (the
// order of the separate reduction kernel: the first partial, plus each following one, plus the
// bias), writes those rows of P, and counts itself into the block's ready word.  Lane l takes
// columns 4 l .. 4 l + 3.  Partials and P go through the agent-coherent path: they are written
// and read by workgroups on different XCDs within the launch.
template <class C>
__device__ __forceinline__ bool producer_reduce(const TileInfo& ti, int pid, const Guards* guards, uint32_t* abort) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  static_assert(C::BN == 256 && C::NCG <= 32, "one 256-column block: four columns per lane");
  // Flags, partials and P are addressed as offsets into one descriptor over the workspace
  // (the host keeps it under 2 GiB): its bound keeps every access inside the workspace, and
  // the unit needs few scalar registers next to the producer's own state.
  const uint64_t wlo = uni64(guards->w_lo);
  const uint32_t wsize = (uint32_t)(uni64(guards->w_hi) - wlo);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<void*>(wlo), wsize);
  const uint32_t epoch = uni(ti.epoch);
  const int parts = (int)uni(ti.count);
  const uint32_t stride = uni(ti.stride), active = uni(ti.p_bytes);
  const int rows = (int)uni((uint32_t)ti.m_rows), n_cols = (int)uni((uint32_t)ti.n_cols);
  const uint32_t ld = uni((uint32_t)ti.ldp);
  const uint32_t flags_off = (uint32_t)(uni64(ti.sync) - wlo);
  const uint32_t src_off = (uint32_t)(uni64(ti.part) - wlo), dst_off = (uint32_t)(uni64(ti.P) - wlo);
  const uint64_t span = (uint64_t)(rows - 1) * ld * 4 + (uint64_t)n_cols * 4;
  if (parts < 1 || parts * C::NCG > 256 || rows < 1 || rows > C::BM || n_cols < 1 || n_cols > C::BN ||
      uni64(ti.sync) < wlo || uni64(ti.part) < wlo || uni64(ti.P) < wlo ||
      (uint64_t)flags_off + (uint64_t)parts * C::NCG * 4 > wsize ||
      (uint64_t)src_off + (uint64_t)(parts - 1) * stride * 4 + span > wsize || (uint64_t)dst_off + span > wsize) {
    raise_abort(abort, 8u);
    return false;
  }
  const int lane = lane_id();
  // every active wave's flag of every slice: lane l checks flags l, l + 64, l + 128, l + 192
  // (polls about a thousand clocks apart, see epoch_wait)
  uint32_t polls = 0;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = lane + 64 * q;
      if (i < parts * C::NCG && ((active >> (i % C::NCG)) & 1u) &&
          __builtin_amdgcn_raw_buffer_load_b32(rw, flags_off + (uint32_t)i * 4u, 0, 16) != epoch)
        ok = false;
    }
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
    __builtin_amdgcn_s_sleep(16);
    if ((++polls & 63) == 0 && (uni(lds_peek(abort)) != 0 || polls >= kSpinLimit)) {
      raise_abort(abort, 1u);
      return false;
    }
  }
  const int col = lane * 4;
  const bool col_ok = col < n_cols;
  const uint64_t biasp = uni64(ti.bias);
  if (biasp != 0 && !inside(biasp, (uint64_t)n_cols * 4, uni64(guards->bias_lo), uni64(guards->bias_hi))) {
    raise_abort(abort, 8u);
    return false;
  }
  constexpr int kInFlight = 8;  // partial loads in flight per round
  for (int r = pid; r < rows; r += C::NPROD) {
    const uint32_t off = (uint32_t)r * ld * 4u + (uint32_t)col * 4u;
    f32x4 acc = {};
    for (int p0 = 0; p0 < parts; p0 += kInFlight) {
      // every load is issued (a slice past the last one reads zeros, touching no memory);
      // only the slices that exist are added, in order
      f32x4 v[kInFlight];
      uint32_t o = src_off + off + (uint32_t)p0 * stride * 4u;  // a running offset: few scalar registers
#pragma unroll
      for (int i = 0; i < kInFlight; ++i) {
        v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rw, (col_ok && p0 + i < parts) ? o : kOutOfRange, 0, 16));
        o += stride * 4u;
      }
#pragma unroll
      for (int i = 0; i < kInFlight; ++i) {
        const f32x4 sum = acc + v[i];
        acc = p0 + i == 0 ? v[i] : (p0 + i < parts ? sum : acc);
      }
    }
    if (biasp != 0) {
      // read per row (a short live range: the unit runs beside the producer's own state)
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(reinterpret_cast<void*>(biasp), (uint32_t)(n_cols * 4));
      acc += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, col_ok ? col * 4 : kOutOfRange, 0, 0));
    }
    if (col_ok) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), rw, dst_off + off, 0, 16);
  }
  // the rows of P have completed before the wave counts itself into the ready word
  wait_vmcnt<0>();
  if (lane == 0) epoch_add(reinterpret_cast<uint64_t*>(ti.C), epoch);
  return true;
}

template <class C, class S>
__device__ __forceinline__ FetchTile fetch_tile(const typename S::Args& args, int j, int pid, bool opA,
                                                int i0, char* sched_lds, TileInfo* info,
                                                const Guards* guards, uint32_t* abort) {
  const int lane = lane_id();
  TileSrc t = {};
  FetchTile f = {};
  // Every value is the same across the wave; saying so keeps the fetch state in scalar
  // registers (a scheduler may read LDS, whose loads the compiler treats as per-lane).
  f.has = uni(schedule_tile<C, S>(args, j, pid, t, sched_lds, abort) ? 1u : 0u) != 0;
  if constexpr (S::kModes == kModesBroadcast) {
    // the single-launch broadcast: the producers run the reduction units, and a candidate tile
    // is published only once its column block of P is ready
    const uint32_t mode = f.has ? uni(t.info.mode) : 0u;
    if (mode == kModeReduce)
      producer_reduce<C>(t.info, pid, guards, abort);
    else if (mode == kModeCandidate && pid == 0)
      epoch_wait(reinterpret_cast<const uint64_t*>(uni64(t.info.sync)), uni(t.info.epoch), uni(t.info.count), abort);
  }
  if (pid == 0 && lane == 0) {
    TileInfo ti = t.info;
    ti.tag = f.has ? tile_tag(j) : end_tag(j);
    info[j % C::NINFO] = ti;
  }
  if (!f.has) return f;
  f.K = (int)uni((uint32_t)t.info.K);
  f.nsteps = tile_steps<C>(f.K);
  const int64_t ld = (int64_t)uni64((uint64_t)(opA ? t.lda : t.ldb));
  const int extent = (int)uni((uint32_t)(opA ? t.info.m_rows : t.info.n_cols));
  f.src = uni64(reinterpret_cast<uint64_t>(opA ? (const void*)t.A : (const void*)t.B));
  const bool kmajor = opA ? C::A_KM : C::B_KN;  // k is the operand's row index
  // The share's first row (of m or n, when that is the operand's row index).  A share past
  // the valid rows feeds only output rows (A) or columns (B stored N x K) past the tile's
  // valid extent, which are never stored; on the large tile its only readers are the waves
  // that own those rows, and they idle on this tile.  Its stale LDS contents are harmless.
  f.dead = !kmajor && (i0 - (opA ? 0 : C::A_INSTR)) * 64 / (opA ? C::CPR_A : C::CPR_B) >= extent;
  if (!kmajor) {
    f.bytes = (uint32_t)((int64_t)(extent - 1) * ld * 2 + (int64_t)f.K * 2);
    f.kstride = 2;
  } else {
    f.bytes = (uint32_t)((int64_t)(f.K - 1) * ld * 2 + (int64_t)extent * 2);
    f.kstride = ld * 2;
  }
  if (f.K == 0) {
    // an empty reduction (a weight gradient of an expert without rows): its one step is
    // all zeros and touches no memory
    f.src = 0;
    f.bytes = 0;
  } else if (!inside(f.src, f.bytes, uni64(opA ? guards->a_lo : guards->b_lo), uni64(opA ? guards->a_hi : guards->b_hi)) &&
             !(opA && inside(f.src, f.bytes, uni64(guards->a2_lo), uni64(guards->a2_hi)))) {
    raise_abort(abort, 4u);
    f.bytes = 0;  // every load of this tile is out of range: nothing is read
  }
  // Rows and columns beyond the tile lie beyond the descriptor (a row past the last valid
  // one starts past its end) or in columns the epilogue never stores, so only the k tail
  // needs masking.  Two per-lane bases, a row step and a per-lane flip offset describe every
  // load's offset (chunk_pattern_ok).
  int row0 = 0, c0 = 0, row1 = 0, c1 = 0;
  chunk_of<C>(i0, lane, row0, c0);
  chunk_of<C>(i0 + 1, lane, row1, c1);
  f.vbase0 = (uint32_t)(row0 * ld * 2 + c0 * 16);
  f.vbase1 = (uint32_t)(row1 * ld * 2 + c1 * 16);
  f.vflip0 = kmajor ? ((c0 ^ 2) - c0) * 16 : 0;
  f.vflip1 = kmajor ? ((c1 ^ 2) - c1) * 16 : 0;
  f.narrow = kmajor && extent < (opA ? C::BM : C::BN);
  f.extent = extent;
  f.col0 = c0 * 8;
  f.col1 = c1 * 8;
  f.kbase0 = kmajor ? row0 : c0 * 8;  // k of the chunk's first element
  f.kbase1 = kmajor ? row1 : c1 * 8;
  f.rstep = (uint32_t)(ld * 2 * (opA ? C::ROWS_A : C::ROWS_B));
  return f;
}

// Byte offset of a producer's load q within the step (see chunk_pattern_ok); q is a
// compile-time index after unrolling, so the flip is a compile-time choice.
template <class C>
__device__ __forceinline__ uint32_t load_off(const FetchTile& f, int q, bool opA) {
  const uint32_t base = ((q & 1) ? f.vbase1 : f.vbase0) + (uint32_t)(q >> 1) * f.rstep;
  const bool flip = opA ? row_flip<C::ROWS_A>(q) : row_flip<C::ROWS_B>(q);  // vflip is 0 unless k-major
  return flip ? base + (uint32_t)((q & 1) ? f.vflip1 : f.vflip0) : base;
}

template <class C, class S>
__device__ __forceinline__ void producer_role_regs(const typename S::Args& args, char* ring, TileInfo* info,
                                                   uint32_t* full, uint32_t* empty, uint32_t* abort, int pid,
                                                   char* sched_lds, const Guards* guards) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  static_assert(C::A_INSTR % C::LOADS == 0, "each producer copies either A or B chunks");
  static_assert(C::LOADS % 2 == 0 && chunk_pattern_ok<C>(), "load offsets must follow the two-base pattern");
  const int lane = lane_id();
  const int i0 = pid * C::LOADS;
  const bool opA = i0 < C::A_INSTR;  // this producer's operand
  const int lds_base = (opA ? i0 * 1024 : C::A_BYTES + (i0 - C::A_INSTR) * 1024) + lane * 16;
  const int kq = opA ? (C::A_KM ? C::ROWS_A : 0) : (C::B_KN ? C::ROWS_B : 0);

  u32x4 R[C::LOADS];
  int fj = 0, fst = 0;  // tile and step the registers hold (or will hold)
  FetchTile f = fetch_tile<C, S>(args, 0, pid, opA, i0, sched_lds, info, guards, abort);
  for (uint32_t g = 0;; ++g) {
    // ---- fetch: issue the loads of step fst of tile fj into R (zeros past K) -----------
    if (f.has && !f.dead) {
      const int k0 = fst * C::BK;
      const int64_t kbytes = (int64_t)k0 * f.kstride;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(reinterpret_cast<const void*>(f.src + kbytes), f.bytes - (uint32_t)kbytes);
      if (k0 + C::BK <= f.K && !f.narrow) {
#pragma unroll
        for (int q = 0; q < C::LOADS; ++q)
          R[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, load_off<C>(f, q, opA), 0, 0);
      } else {
        // the last, partial k-step, or a narrow tile: k past K and columns past the tile's
        // valid ones take an out-of-range offset (zeros, no memory access)
#pragma unroll
        for (int q = 0; q < C::LOADS; ++q) {
          const int kpos = ((q & 1) ? f.kbase1 : f.kbase0) + (q >> 1) * kq;
          const bool flip = opA ? row_flip<C::ROWS_A>(q) : row_flip<C::ROWS_B>(q);
          const int col = ((q & 1) ? f.col1 : f.col0) ^ (flip ? 16 : 0);
          const bool ok = k0 + kpos < f.K && (!f.narrow || col < f.extent);
          R[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? load_off<C>(f, q, opA) : kOutOfRange, 0, 0);
        }
      }
    }
    // ---- ring: step g goes to slot s once the consumers have released it ---------------
    const int s = g % C::STAGES;
    wait_at_least(&empty[s], (uint32_t)C::NCG * (g / C::STAGES), abort);
    if (!f.has) {
      lds_bump(&full[s]);  // the end marker's step carries no data
      break;
    }
    if (!f.dead) {
      char* dst = ring + s * C::STAGE_BYTES + lds_base;
#pragma unroll
      for (int q = 0; q < C::LOADS; ++q) *reinterpret_cast<u32x4*>(dst + q * 1024) = R[q];
    }
    // LDS runs one wave's accesses in order: the writes land before the count moves
    lds_bump(&full[s]);
    // ---- advance the fetch side -------------------------------------------------------
    if (++fst == f.nsteps) {
      fst = 0;
      f = fetch_tile<C, S>(args, ++fj, pid, opA, i0, sched_lds, info, guards, abort);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Consumer role: MFMA on staged tiles, then the epilogue stage on the accumulators
// ---------------------------------------------------------------------------------------

// Start value of one consumer wave's accumulators: bias[col], or P[idx[row]][col] for a
// gathered (broadcast) launch, else zero; a gathered launch carries no bias (the host adds
// it to P).  The MFMAs then add the products on top, so the epilogue needs no loads and
// nothing extra stays live next to the accumulators (the loads land in the accumulator
// registers themselves).  Layout as in the epilogue below: register 4q + t of acc[tm][tn],
// lane l, is row 32 tm + l % 32, column 32 tn + 8q + 4 (l / 32) + t of the wave's sub-tile,
// so each lane loads runs of 4 columns.  Returns false (workgroup aborted) when the tile's
// metadata or an operand range is wrong.
template <class C>
__device__ __forceinline__ bool init_acc(f32x16 (&acc)[C::TM][C::TN], const TileInfo* ti,
                                         const Guards* guards, int epi, int wm, int wn,
                                         uint32_t* abort) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = f32x16{};
  const uint64_t biasp = uni64(ti->bias);
  const uint64_t gidxp = uni64(ti->gidx);
  const bool gather = gidxp != 0;
  const bool do_bias = (epi == EPI_BIAS || epi == EPI_BIAS_SILU) && biasp != 0 && !gather;
  if (!do_bias && !gather) return true;
  const int m_rows = (int)uni((uint32_t)ti->m_rows);
  const int n_cols = (int)uni((uint32_t)ti->n_cols);
  const uint64_t Pp = uni64(ti->P);
  const int ldp = (int)uni((uint32_t)ti->ldp);
  const uint32_t p_bytes = uni(ti->p_bytes);
  if (m_rows < 1 || m_rows > C::BM || n_cols < 1 || n_cols > C::BN) {
    raise_abort(abort, 2u);
    return false;
  }
  const Guards& gd = *guards;
  if ((do_bias && !inside(biasp, (uint64_t)n_cols * 4, uni64(gd.bias_lo), uni64(gd.bias_hi))) ||
      (gather && (!inside(gidxp, (uint64_t)m_rows * 4, uni64(gd.gidx_lo), uni64(gd.gidx_hi)) ||
                  !inside(Pp, p_bytes, uni64(gd.p_lo), uni64(gd.p_hi))))) {
    raise_abort(abort, 8u);
    return false;
  }
  const int lane = opaque_lane();
  const int half = lane >> 5;
  if (do_bias) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(reinterpret_cast<void*>(biasp), (uint32_t)(n_cols * 4));
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * C::WTN + tn * 32 + q * 8 + half * 4;
        const f32x4 b4 = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, col < n_cols ? col * 4 : kOutOfRange, 0, 0));
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[tm][tn][4 * q + t] = b4[t];
      }
    }
  } else {
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(reinterpret_cast<void*>(gidxp), (uint32_t)(m_rows * 4));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(reinterpret_cast<void*>(Pp), p_bytes);
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      const int row = wm * C::WTM + tm * 32 + (lane & 31);
      const bool row_ok = row < m_rows;
      const int prow = (int)__builtin_amdgcn_raw_buffer_load_b32(rg, row_ok ? row * 4 : kOutOfRange, 0, 0);
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * C::WTN + tn * 32 + q * 8 + half * 4;
          const uint32_t po = (row_ok && col < n_cols) ? (uint32_t)(prow * ldp + col) * 4u : kOutOfRange;
          const f32x4 p4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, po, 0, 0));
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[tm][tn][4 * q + t] = p4[t];
        }
      }
    }
  }
  return true;
}

// Epilogue stage of one consumer wave: SiLU if asked, conversion, stores.  The MFMAs run with
// B as the first operand, so acc[tm][tn] holds the transpose of its 32 x 32 block (layout
// above): each lane owns runs of 4 consecutive columns of one row.  fp32 output leaves in
// 16-byte stores; bf16 output is packed to 8-byte runs, and lanes l and l + 32 (same row)
// trade halves so that each holds 8 consecutive columns, again one 16-byte store.  N is a
// multiple of 8 and rows are 16-byte aligned, so a run is wholly inside the valid columns
// or wholly outside; rows and runs outside the tile get an out-of-range offset (the store
// is dropped).
template <class C>
__device__ __forceinline__ void epilogue(f32x16 (&acc)[C::TM][C::TN], int wm, int wn, int m_rows,
                                         int n_cols, uint64_t Cp, int ldc, bool do_silu, bool f32out) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const int lane = opaque_lane();
  const int half = lane >> 5;
  const int osz = f32out ? 4 : 2;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(reinterpret_cast<void*>(Cp), (uint32_t)(((int64_t)(m_rows - 1) * ldc + n_cols) * osz));
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
    const int row = wm * C::WTM + tm * 32 + (lane & 31);
    const bool row_ok = row < m_rows;
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      f32x16& v = acc[tm][tn];
      if (do_silu) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = silu(v[r]);
      }
      if (f32out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * C::WTN + tn * 32 + q * 8 + half * 4;
          const uint32_t vo = (row_ok && col < n_cols) ? (uint32_t)(row * ldc + col) * 4u : kOutOfRange;
          const f32x4 o = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rc, vo, 0, 0);
        }
      } else {
        // pack each run of 4 to bf16 (round to nearest even); then, for the run pairs (0, 1)
        // and (2, 3), the low lanes' second run trades places with the high lanes' first run
        uint32_t w[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q][0] = pack_bf16(v[4 * q], v[4 * q + 1]);
          w[q][1] = pack_bf16(v[4 * q + 2], v[4 * q + 3]);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const auto sw = __builtin_amdgcn_permlane32_swap(w[2 * pr][h], w[2 * pr + 1][h], false, false);
            w[2 * pr][h] = sw[0];
            w[2 * pr + 1][h] = sw[1];
          }
          // low lanes now hold columns 16 pr + 0..7 of the block, high lanes 16 pr + 8..15
          const int col = wn * C::WTN + tn * 32 + pr * 16 + half * 8;
          const uint32_t vo = (row_ok && col < n_cols) ? (uint32_t)(row * ldc + col) * 2u : kOutOfRange;
          const u32x4 d = {w[2 * pr][0], w[2 * pr][1], w[2 * pr + 1][0], w[2 * pr + 1][1]};
          __builtin_amdgcn_raw_buffer_store_b128(d, rc, vo, 0, 0);
        }
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void consumer_role(char* ring, const TileInfo* info, uint32_t* full, uint32_t* empty,
                                              uint32_t* abort, int cw, int epi, bool f32out,
                                              const Guards* guards) {
  static_assert(!C::A_KM, "A stored K x M is read by the 16x16 consumer (consumer_role16)");
  const int lane = lane_id();
  const int cgrp = cw / C::NCG;                // consumer group
  const int wm = (cw % C::NCG) / C::WN, wn = (cw % C::NCG) % C::WN;
  // A-fragment addressing: lane l holds row (l % 32) of a 32-row block and k-chunk l / 32.
  // Physical chunk = (2 kk + l/32) ^ swz(row) = (2 kk) ^ (l/32 ^ swz(row)) since bit 0 of
  // 2 kk is clear; swz(row) depends only on row % 16, the same for every block of the wave.
  const int ra = wm * C::WTM + (lane & 31);
  const int a_chunk = (lane >> 5) ^ swz_k<C::CPR_A>(ra);
  const int a_base = ra * C::BK * 2;
  int b_base = 0, b_chunk = 0;
  int b_kn0 = 0;  // KN: byte offset of the first transposing read of block 0 at sub-step 0
  if constexpr (!C::B_KN) {
    const int rb = wn * C::WTN + (lane & 31);
    b_chunk = (lane >> 5) ^ swz_k<C::CPR_B>(rb);
    b_base = rb * C::BK * 2;
  } else {
    // Transposing read: in each 16-lane block, lane i fetches 4 bf16 of k-row (i / 4) at
    // columns 4 (i % 4) .. +3; the hardware hands lane i the 4 k-values of column i.  The
    // second read of a fragment is 4 k-rows further down, and sub-step kk adds 16 k-rows:
    // both multiples of 4, so the swizzle (a function of k mod 4), hence the offset within
    // a row, is unchanged and both become immediate offsets.  Block tn sits 4 tn chunks
    // further along the row; the wave's first chunk index is a multiple of 4 TN, so that
    // is an XOR of the chunk index (TN a power of two), and the swizzle XOR commutes with
    // it: block tn reads at b_kn0 ^ (tn << 6).
    static_assert((C::TN & (C::TN - 1)) == 0, "TN must be a power of two");
    const int blk = lane >> 4, i = lane & 15;
    const int k = (blk >> 1) * 8 + (i >> 2);
    const int n = wn * C::WTN + (blk & 1) * 16 + (i & 3) * 4;
    b_kn0 = k * C::BN * 2 + (((n >> 3) ^ swz_n<C::CPR_B>(k)) << 4) + ((n >> 2) & 1) * 8;
  }

  uint32_t g = 0;
  for (int j = 0;; ++j) {
    // The first k-step of tile j carries its metadata.
    const int s0 = g % C::STAGES;
    wait_at_least(&full[s0], (uint32_t)C::NPROD * (g / C::STAGES + 1), abort);
    const TileInfo* ti = &info[j % C::NINFO];
    const uint32_t tag = uni(ti->tag);
    if (tag != tile_tag(j)) {
      // the end marker, or (never in a working pipeline) a slot that is not what was
      // published: release the step so the counters stay consistent, and stop
      if (tag != end_tag(j)) raise_abort(abort, 2u);
      lds_bump(&empty[s0]);
      break;
    }
    const int K = (int)uni((uint32_t)ti->K);
    const int nsteps = tile_steps<C>(K);
    if (C::CG > 1 && j % C::CG != cgrp) {
      // the other group's tile: only its step count matters here
      g += (uint32_t)nsteps;
      continue;
    }

    // A wave whose sub-tile lies wholly outside the tile's valid rows or columns has nothing
    // to compute or store: it only takes part in the handoff, releasing each step as it
    // arrives (a release never runs ahead of the step's arrival, so the counts stay exact).
    // On a tile with at most half its rows valid, half the consumer waves idle and each
    // SIMD's matrix core serves the other half alone.
    if (wm * C::WTM >= (int)uni((uint32_t)ti->m_rows) || wn * C::WTN >= (int)uni((uint32_t)ti->n_cols)) {
      lds_bump(&empty[s0]);
      ++g;
      for (int st = 1; st < nsteps; ++st, ++g) {
        const int s = g % C::STAGES;
        wait_at_least(&full[s], (uint32_t)C::NPROD * (g / C::STAGES + 1), abort);
        lds_bump(&empty[s]);
      }
      continue;
    }

    if (uni(ti->mode) != 0) {  // split tiles are served by the 16x16 consumer only
      raise_abort(abort, 2u);
      break;
    }
    f32x16 acc[C::TM][C::TN];
    if (!init_acc<C>(acc, ti, guards, epi, wm, wn, abort)) break;

    // Fragment loads of one 16-deep sub-step kk of a staged slot.
    auto load_a = [&](const char* slot, int kk, int tm) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(slot + a_base + (((kk * 2) ^ a_chunk) << 4) +
                                              tm * 32 * C::BK * 2);
    };
    auto load_b = [&](const char* slot, int kk, int tn) -> bf16x8 {
      const char* slotB = slot + C::A_BYTES;
      if constexpr (!C::B_KN) {
        return *reinterpret_cast<const bf16x8*>(slotB + b_base + (((kk * 2) ^ b_chunk) << 4) +
                                                tn * 32 * C::BK * 2);
      } else {
        const int off = b_kn0 ^ (tn << 6);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(slotB + off + kk * 16 * C::BN * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(slotB + off + (kk * 16 + 4) * C::BN * 2));
        typedef __attribute__((ext_vector_type(8))) short i16x8;
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };

    // Rolling prefetch: each fragment register is refilled with the next sub-step's
    // fragment right after its last MFMA of the current sub-step, so LDS latency hides
    // behind the remaining MFMAs.  MFMAs run B-column-major: b[tn] is free after TM MFMAs,
    // every a[tm] after the last column.
    bf16x8 a[C::TM], b[C::TN];
    {
      const char* slot0 = ring + s0 * C::STAGE_BYTES;
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) b[tn] = load_b(slot0, 0, tn);
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) a[tm] = load_a(slot0, 0, tm);
    }
    for (int st = 0; st < nsteps; ++st, ++g) {
      const int s = g % C::STAGES;
      const char* slot = ring + s * C::STAGE_BYTES;
      const bool more_steps = st + 1 < nsteps;
      const int sn = (g + 1) % C::STAGES;
      const char* next_slot = ring + sn * C::STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < C::KSUB; ++kk) {
        const bool last_kk = kk == C::KSUB - 1;
        const bool more = !last_kk || more_steps;     // a sub-step follows in this tile
        const char* nslot = last_kk ? next_slot : slot;
        const int nkk = last_kk ? 0 : kk + 1;
        bool ready = !last_kk;                        // the next slot's data is known present
        if (last_kk) {
          // this sub-step's fragments (the last reads of slot s) are in registers
          wait_lgkm0();
          lds_bump(&empty[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm) {
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[tn], a[tm], acc[tm][tn], 0, 0, 0);
            if (tn == C::TN - 1 && more) {
              if (!ready) {
                wait_at_least(&full[sn], (uint32_t)C::NPROD * ((g + 1) / C::STAGES + 1), abort);
                ready = true;
              }
              a[tm] = load_a(nslot, nkk, tm);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if (more) {
            if (!ready) {
              wait_at_least(&full[sn], (uint32_t)C::NPROD * ((g + 1) / C::STAGES + 1), abort);
              ready = true;
            }
            b[tn] = load_b(nslot, nkk, tn);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- epilogue stage: SiLU, convert, store ------------------------------------------
    // The metadata is read again here (it is still in place, see NINFO), so that nothing
    // of the epilogue stays live in registers across the MFMA loop.
    const int m_rows = (int)uni((uint32_t)ti->m_rows);
    const int n_cols = (int)uni((uint32_t)ti->n_cols);
    const uint64_t Cp = uni64(ti->C);
    const int ldc = (int)uni((uint32_t)ti->ldc);
    if (m_rows < 1 || m_rows > C::BM || n_cols < 1 || n_cols > C::BN || ldc < n_cols) {
      raise_abort(abort, 2u);
      break;
    }
    const uint64_t c_bytes = (uint64_t)((int64_t)(m_rows - 1) * ldc + n_cols) * (f32out ? 4u : 2u);
    if (!inside(Cp, c_bytes, uni64(guards->c_lo), uni64(guards->c_hi))) {
      raise_abort(abort, 8u);
      break;
    }
    epilogue<C>(acc, wm, wn, m_rows, n_cols, Cp, ldc, epi == EPI_SILU || epi == EPI_BIAS_SILU, f32out);
  }
}

// ---------------------------------------------------------------------------------------
// Consumer role with 16x16x32 MFMAs (Cfg::M16)
// ---------------------------------------------------------------------------------------
// Register layout (B as the first MFMA operand, so each accumulator holds the transpose of
// its 16 x 16 block): register t of acc[tm][tn], lane l, is row 16 tm + l % 16, column
// 16 tn + 4 (l / 16) + t of the wave's sub-tile.  Lanes l, l + 16, l + 32, l + 48 hold
// columns 0-3, 4-7, 8-11, 12-15 of the same row.

// Start value of the accumulators: bias[col], or P[idx[row]][col] for a gathered launch.
template <class C, int MODES>
__device__ __forceinline__ bool init_acc16(f32x4 (&acc)[C::TM16][C::TN16], const TileInfo* ti,
                                           const Guards* guards, int epi, int wm, int wn,
                                           uint32_t* abort) {
#pragma unroll
  for (int tm = 0; tm < C::TM16; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN16; ++tn) acc[tm][tn] = f32x4{};
  // the second unit of a split tile adds its partial sum to the first's, which carries the
  // start value
  if (MODES == kModesSplit && uni(ti->mode) == 2) return true;
  const uint64_t biasp = uni64(ti->bias);
  const uint64_t gidxp = uni64(ti->gidx);
  const bool gather = gidxp != 0;
  const bool do_bias = (epi == EPI_BIAS || epi == EPI_BIAS_SILU) && biasp != 0 && !gather;
  if (!do_bias && !gather) return true;
  const int m_rows = (int)uni((uint32_t)ti->m_rows);
  const int n_cols = (int)uni((uint32_t)ti->n_cols);
  const uint64_t Pp = uni64(ti->P);
  const int ldp = (int)uni((uint32_t)ti->ldp);
  const uint32_t p_bytes = uni(ti->p_bytes);
  if (m_rows < 1 || m_rows > C::BM || n_cols < 1 || n_cols > C::BN) {
    raise_abort(abort, 2u);
    return false;
  }
  const Guards& gd = *guards;
  if ((do_bias && !inside(biasp, (uint64_t)n_cols * 4, uni64(gd.bias_lo), uni64(gd.bias_hi))) ||
      (gather && (!inside(gidxp, (uint64_t)m_rows * 4, uni64(gd.gidx_lo), uni64(gd.gidx_hi)) ||
                  !inside(Pp, p_bytes, uni64(gd.p_lo), uni64(gd.p_hi))))) {
    raise_abort(abort, 8u);
    return false;
  }
  const int lane = opaque_lane();
  const int cq = (lane >> 4) * 4;  // this lane's first column within a 16-column block
  if (do_bias) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(reinterpret_cast<void*>(biasp), (uint32_t)(n_cols * 4));
#pragma unroll
    for (int tn = 0; tn < C::TN16; ++tn) {
      const int col = wn * C::WTN + tn * 16 + cq;
      const f32x4 b4 = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, col < n_cols ? col * 4 : kOutOfRange, 0, 0));
#pragma unroll
      for (int tm = 0; tm < C::TM16; ++tm) acc[tm][tn] = b4;
    }
  } else {
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(reinterpret_cast<void*>(gidxp), (uint32_t)(m_rows * 4));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(reinterpret_cast<void*>(Pp), p_bytes);
    int prow[C::TM16];
#pragma unroll
    for (int tm = 0; tm < C::TM16; ++tm) {
      const int row = wm * C::WTM + tm * 16 + (lane & 15);
      prow[tm] = (int)__builtin_amdgcn_raw_buffer_load_b32(rg, row < m_rows ? row * 4 : kOutOfRange, 0, 0);
    }
    // Candidates come in runs of one user's rows, so the wave's rows usually all gather the
    // same P row.  Then its columns are loaded once and copied into every row block (rows
    // past m_rows take them too; the epilogue never stores those rows).  Lane 0 holds the
    // wave's first row, which is valid: an idle wave does not get here.
    // (the single-launch broadcast reads P on the agent-coherent path: reduction units wrote
    // it during this launch, possibly on another XCD)
    auto load_p = [&](uint32_t off) -> f32x4 {
      return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, MODES == kModesBroadcast ? 16 : 0));
    };
    const int p0 = (int)uni((uint32_t)prow[0]);
    bool same = true;
#pragma unroll
    for (int tm = 0; tm < C::TM16; ++tm) {
      const int row = wm * C::WTM + tm * 16 + (lane & 15);
      if (row < m_rows && prow[tm] != p0) same = false;
    }
    if (__builtin_amdgcn_ballot_w64(!same) == 0) {
#pragma unroll
      for (int tn = 0; tn < C::TN16; ++tn) {
        const int col = wn * C::WTN + tn * 16 + cq;
        const uint32_t po = col < n_cols ? (uint32_t)(p0 * ldp + col) * 4u : kOutOfRange;
        const f32x4 p4 = load_p(po);
#pragma unroll
        for (int tm = 0; tm < C::TM16; ++tm) acc[tm][tn] = p4;
      }
    } else {
#pragma unroll
      for (int tm = 0; tm < C::TM16; ++tm) {
        const int row = wm * C::WTM + tm * 16 + (lane & 15);
        const bool row_ok = row < m_rows;
#pragma unroll
        for (int tn = 0; tn < C::TN16; ++tn) {
          const int col = wn * C::WTN + tn * 16 + cq;
          const uint32_t po = (row_ok && col < n_cols) ? (uint32_t)(prow[tm] * ldp + col) * 4u : kOutOfRange;
          acc[tm][tn] = load_p(po);
        }
      }
    }
  }
  return true;
}

// Streaming stores of 16 rows as whole 128-byte segments.  On entry lane (g, r) of the wave
// (16-lane group g, row r of 16) holds 16-byte runs X and Y of row r, at columns colX and colY;
// for each row the four groups' X runs are 64 contiguous bytes and their Y runs the next 64.
// Lanes r and r ^ 8 trade (a DPP rotation by 8 within each 16-lane row), so that one store
// writes rows 0-7 and the other rows 8-15, each as 128 contiguous bytes.  Rows at or past
// m_rows, and runs at or past n_cols, take an out-of-range offset (the store is dropped).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
__device__ __forceinline__ void store_rows128(u32x4_t X, u32x4_t Y, int colX, int colY, int row0, int lane,
                                              int m_rows, int n_cols, int ldc, uint32_t osz,
                                              __amdgpu_buffer_rsrc_t rc, bool coherent = false) {
  const bool lo = (lane & 8) == 0;
  u32x4_t A, B;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t xr = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)X[q], 0x128, 0xF, 0xF, false);  // row_ror:8
    const uint32_t yr = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)Y[q], 0x128, 0xF, 0xF, false);
    A[q] = lo ? X[q] : yr;
    B[q] = lo ? xr : Y[q];
  }
  const int col = lo ? colX : colY;
  const int rowA = row0 + (lane & 7), rowB = rowA + 8;
  const bool col_ok = col < n_cols;
  const uint32_t vA = (rowA < m_rows && col_ok) ? (uint32_t)(rowA * ldc + col) * osz : kOutOfRange;
  const uint32_t vB = (rowB < m_rows && col_ok) ? (uint32_t)(rowB * ldc + col) * osz : kOutOfRange;
  if (coherent) {
    // cache policy sc1: agent-coherent (read next by workgroups on other XCDs)
    __builtin_amdgcn_raw_buffer_store_b128(A, rc, vA, 0, 16);
    __builtin_amdgcn_raw_buffer_store_b128(B, rc, vB, 0, 16);
  } else {
    // cache policy 2: non-temporal
    __builtin_amdgcn_raw_buffer_store_b128(A, rc, vA, 0, 2);
    __builtin_amdgcn_raw_buffer_store_b128(B, rc, vB, 0, 2);
  }
}

// Epilogue: SiLU if asked, conversion, 16-byte stores.  fp32: one run of 4 columns per lane
// and block.  bf16: runs of 4 packed to 8 bytes; for the block pairs (tn, tn + 1),
// v_permlane16_swap trades the second 16-lane group's run of block tn against the first
// group's run of block tn + 1 (and groups 3 and 2 likewise), after which lane group g holds
// columns 8 (g / 2) .. + 7 of block tn + g % 2.
template <class C>
__device__ __forceinline__ void epilogue16(f32x4 (&acc)[C::TM16][C::TN16], int wm, int wn, int m_rows,
                                           int n_cols, uint64_t Cp, int ldc, bool do_silu, bool f32out,
                                           bool coherent = false) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const int lane = opaque_lane();
  const int grp = lane >> 4;
  const int osz = f32out ? 4 : 2;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(reinterpret_cast<void*>(Cp), (uint32_t)(((int64_t)(m_rows - 1) * ldc + n_cols) * osz));
#pragma unroll
  for (int tm = 0; tm < C::TM16; ++tm) {
    const int row = wm * C::WTM + tm * 16 + (lane & 15);
    const bool row_ok = row < m_rows;
    if constexpr (C::STREAM_OUT) {
      // fp32: blocks tn and tn + 1 of a row are 128 contiguous bytes; bf16: the two block
      // pairs after the group trade below are
      const int row0 = wm * C::WTM + tm * 16;
      u32x4 pair0 = {};
#pragma unroll
      for (int tn = 0; tn < C::TN16; tn += 2) {
        f32x4& v0 = acc[tm][tn];
        f32x4& v1 = acc[tm][tn + 1];
        if (do_silu) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v0[t] = silu(v0[t]);
            v1[t] = silu(v1[t]);
          }
        }
        if (f32out) {
          const int colX = wn * C::WTN + tn * 16 + grp * 4;
          store_rows128(__builtin_bit_cast(u32x4, v0), __builtin_bit_cast(u32x4, v1), colX, colX + 16, row0,
                        lane, m_rows, n_cols, ldc, 4u, rc, coherent);
        } else {
          const uint32_t x0 = pack_bf16(v0[0], v0[1]), x1 = pack_bf16(v0[2], v0[3]);
          const uint32_t y0 = pack_bf16(v1[0], v1[1]), y1 = pack_bf16(v1[2], v1[3]);
          const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
          const u32x4 d = {s0[0], s1[0], s0[1], s1[1]};
          if (tn == 0) {
            pair0 = d;
          } else {
            const int colX = wn * C::WTN + (grp & 1) * 16 + (grp >> 1) * 8;
            store_rows128(pair0, d, colX, colX + 32, row0, lane, m_rows, n_cols, ldc, 2u, rc, coherent);
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int tn = 0; tn < C::TN16; tn += 2) {
      f32x4& v0 = acc[tm][tn];
      f32x4& v1 = acc[tm][tn + 1];
      if (do_silu) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v0[t] = silu(v0[t]);
          v1[t] = silu(v1[t]);
        }
      }
      if (f32out) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = wn * C::WTN + (tn + h) * 16 + grp * 4;
          const uint32_t vo = (row_ok && col < n_cols) ? (uint32_t)(row * ldc + col) * 4u : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, h ? v1 : v0), rc, vo, 0, 0);
        }
      } else {
        uint32_t x0 = pack_bf16(v0[0], v0[1]), x1 = pack_bf16(v0[2], v0[3]);
        uint32_t y0 = pack_bf16(v1[0], v1[1]), y1 = pack_bf16(v1[2], v1[3]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
        const int col = wn * C::WTN + (tn + (grp & 1)) * 16 + (grp >> 1) * 8;
        const uint32_t vo = (row_ok && col < n_cols) ? (uint32_t)(row * ldc + col) * 2u : kOutOfRange;
        const u32x4 d = {s0[0], s1[0], s0[1], s1[1]};
        __builtin_amdgcn_raw_buffer_store_b128(d, rc, vo, 0, 0);
      }
    }
  }
}

// Combine of a tile whose reduction is split between two units on two workgroups (mode 1:
// the first part of k, mode 2: the rest).  Each consumer wave meets the wave with the same
// sub-tile in the other unit through its own sync words in the workspace:
//   - a 64-bit arrival word: the launch's epoch in the high half, the arrivals of this epoch
//     in the low half (a word from another launch counts as no arrival, so the workspace
//     needs no clearing between launches);
//   - a 32-bit ready word: the epoch, published by the first unit to arrive.
// The first to arrive writes its fp32 accumulators as a register image (block b of lane l at
// byte 16 (64 b + l) of its 32 KB) and publishes the epoch; the second waits for it, adds the
// image to its own accumulators and runs the epilogue.  The other unit may run on another
// XCD, behind another L2, so the image and the sync words go through the agent-coherent path
// (the sc1 cache policy, which agent-scope atomic loads and stores use): the image stores
// have completed (s_waitcnt) before the ready word is written, and the image is read only
// after the ready word has been seen.  No L2 write-back or invalidation is needed, which
// would also drop the other workgroups' cached operands on that XCD.  A sum of two terms
// does not depend on their order, so the result does not depend on which unit arrives first.
// Returns true when this wave holds the combined sub-tile (false: its part is handed over, or
// the workgroup aborted).
template <class C>
__device__ __forceinline__ bool combine_split16(f32x4 (&acc)[C::TM16][C::TN16], const TileInfo* ti, int w,
                                                const Guards* guards, uint32_t* abort) {
  constexpr int kImage = C::TM16 * C::TN16 * 64 * 16;  // bytes of one wave's register image
  static_assert(C::NCG * kImage <= (int)kSplitImageBytes && C::NCG * 12 <= (int)kSplitSyncBytes,
                "split workspace blocks");
  const uint32_t epoch = uni(ti->epoch);
  const uint64_t syncp = uni64(ti->sync), partp = uni64(ti->part);
  if (!inside(syncp, kSplitSyncBytes, uni64(guards->w_lo), uni64(guards->w_hi)) ||
      !inside(partp, kSplitImageBytes, uni64(guards->w_lo), uni64(guards->w_hi))) {
    raise_abort(abort, 8u);
    return false;
  }
  constexpr int kSc1 = 16;  // cache policy: agent-coherent
  uint64_t* arrive = reinterpret_cast<uint64_t*>(syncp) + w;
  uint32_t* ready = reinterpret_cast<uint32_t*>(syncp + 8 * C::NCG) + w;
  const __amdgpu_buffer_rsrc_t rimg = make_rsrc(reinterpret_cast<void*>(partp + (uint64_t)w * kImage), kImage);
  const int lane = opaque_lane();
  uint32_t first = 0;
  if (lane == 0) {
    uint64_t old = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
      const uint64_t nw = ((uint32_t)(old >> 32) == epoch) ? old + 1 : (((uint64_t)epoch << 32) | 1u);
      if (__hip_atomic_compare_exchange_strong(arrive, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        break;
    }
    first = ((uint32_t)(old >> 32) != epoch || (uint32_t)old == 0) ? 1u : 0u;
  }
  first = uni(first);  // lane 0's value
  if (first) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
#pragma unroll
    for (int tm = 0; tm < C::TM16; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::TN16; ++tn) {
        const f32x4 blk = acc[tm][tn];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, blk), rimg,
                                               (uint32_t)((tm * C::TN16 + tn) * 64 + lane) * 16u, 0, kSc1);
      }
    wait_vmcnt<0>();
    if (lane == 0) __hip_atomic_store(ready, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  uint32_t ok = 1;
  if (lane == 0) {
    uint32_t polls = 0;
    while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      __builtin_amdgcn_s_sleep(2);
      if ((++polls & 63) == 0) {
        if (lds_peek(abort) != 0 || polls >= kSpinLimit) {
          ok = 0;
          break;
        }
      }
    }
  }
  if (uni(ok) == 0) {
    raise_abort(abort, 1u);
    return false;
  }
#pragma unroll
  for (int tm = 0; tm < C::TM16; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN16; ++tn)
      acc[tm][tn] += __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rimg, (uint32_t)((tm * C::TN16 + tn) * 64 + lane) * 16u, 0, kSc1));
  return true;
}

// The consumer loop.  Per 32-deep k-slice: 2 halves of TM16/2 row blocks.  The first half
// runs row-major: a row block's fragment is refilled with the second half's fragment right
// after its last MFMA.  The second half runs column-major: each B fragment is refilled with
// the next slice's right after its last MFMA, and each A fragment with the next slice's
// first-half fragment after the last column.  Fragments in registers: TM16/2 of A and TN16 of
// B.  The ring slot is released as soon as the last fragment read from it has been consumed
// (after the first column of the last slice's second half).
template <class C, int MODES = kModesNone>
__device__ __forceinline__ void consumer_role16(char* ring, const TileInfo* info, uint32_t* full, uint32_t* empty,
                                                uint32_t* abort, int cw, int epi, bool f32out,
                                                const Guards* guards) {
  constexpr int HM = C::TM16 / 2;
  const int lane = lane_id();
  const int cgrp = cw / C::NCG;                // consumer group
  const int wm = (cw % C::NCG) / C::WN, wn = (cw % C::NCG) % C::WN;
  // A fragment (16x16x32): lane l holds row l % 16 of a 16-row block and 8 k-values from
  // k-chunk l / 16 of the slice.  Physical chunk = (4 ks + l/16) ^ swz(row)
  // = (4 ks) ^ (l/16 ^ swz(row)); swz depends on row % 16 only.
  // The row starts at a multiple of 128 bytes and the chunk index occupies address bits
  // 4-6, so slice ks (chunk XOR 4 ks) is the slice-0 offset XOR (ks << 6): one register,
  // the XOR redone at each use (kept per slice, the variants would cost registers).
  static_assert(C::BK == 64 || C::BK == 32, "slice offsets by XOR need rows of 64 or 32 bf16");
  int a_off = 0;
  if constexpr (!C::A_KM) {
    const int ra = wm * C::WTM + (lane & 15);
    a_off = ra * C::BK * 2 + (((lane >> 4) ^ swz_k<C::CPR_A>(ra)) << 4);
  } else {
    // A stored K x M: the transposing read of the K x N B tile below, with m for n.  Per
    // 16-lane group g, k-rows 8 g + i / 4 (and 4 further down) of the slice, m-columns
    // 4 (i % 4) .. +3 of row block tm; lane i receives column i, i.e. row i of the fragment.
    // The wave's first chunk, WTM / 8 tm-blocks of 2 chunks, is a multiple of 2 TM16 (a power
    // of two), so block tm moves the chunk index by an XOR of 2 tm, which commutes with the
    // swizzle XOR: block tm reads at a_off ^ (tm << 5).
    const int grp = lane >> 4, i = lane & 15;
    const int k = grp * 8 + (i >> 2);
    const int m = wm * C::WTM + (i & 3) * 4;
    a_off = k * C::BM * 2 + (((m >> 3) ^ swz_n<C::CPR_A>(k)) << 4) + ((m >> 2) & 1) * 8;
  }
  int b_off = 0, b_kn0 = 0;
  if constexpr (!C::B_KN) {
    const int rb = wn * C::WTN + (lane & 15);
    b_off = rb * C::BK * 2 + (((lane >> 4) ^ swz_k<C::CPR_B>(rb)) << 4);
  } else {
    // Transposing read per 16-lane group g: k-rows 8 g + i / 4 (and 4 further down) of the
    // slice, columns 4 (i % 4) .. +3 of block tn; lane i receives column i.  Block tn moves
    // the chunk index by 2 tn, which commutes with the swizzle XOR (the wave's first chunk
    // has bits 1-2 clear): block tn reads at b_kn0 ^ (tn << 5).
    static_assert(C::TN16 <= 4, "block offsets by XOR need 16 TN16 <= 64 columns per wave");
    const int grp = lane >> 4, i = lane & 15;
    const int k = grp * 8 + (i >> 2);
    const int n = wn * C::WTN + (i & 3) * 4;
    b_kn0 = k * C::BN * 2 + (((n >> 3) ^ swz_n<C::CPR_B>(k)) << 4) + ((n >> 2) & 1) * 8;
  }
  auto load_a = [&](const char* slot, int ks, int tm) -> bf16x8 {
    if constexpr (!C::A_KM) {
      return *reinterpret_cast<const bf16x8*>(slot + (opaque(a_off) ^ (ks << 6)) + tm * 16 * C::BK * 2);
    } else {
      const int off = opaque(a_off) ^ (tm << 5);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slot + off + ks * 32 * C::BM * 2));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slot + off + (ks * 32 + 4) * C::BM * 2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto load_b = [&](const char* slot, int ks, int tn) -> bf16x8 {
    const char* slotB = slot + C::A_BYTES;
    if constexpr (!C::B_KN) {
      return *reinterpret_cast<const bf16x8*>(slotB + (opaque(b_off) ^ (ks << 6)) + tn * 16 * C::BK * 2);
    } else {
      const int off = opaque(b_kn0) ^ (tn << 5);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slotB + off + ks * 32 * C::BN * 2));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slotB + off + (ks * 32 + 4) * C::BN * 2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  uint32_t g = 0;
  for (int j = 0;; ++j) {
    const int s0 = g % C::STAGES;
    wait_at_least(&full[s0], (uint32_t)C::NPROD * (g / C::STAGES + 1), abort);
    const TileInfo* ti = &info[j % C::NINFO];
    const uint32_t tag = uni(ti->tag);
    if (tag != tile_tag(j)) {
      if (tag != end_tag(j)) raise_abort(abort, 2u);
      lds_bump(&empty[s0]);
      break;
    }
    const int K = (int)uni((uint32_t)ti->K);
    const int nsteps = tile_steps<C>(K);
    if (C::CG > 1 && j % C::CG != cgrp) {
      // the other group's tile: only its step count matters here
      g += (uint32_t)nsteps;
      continue;
    }
    // idle wave: only takes part in the handoff (see consumer_role).  The extents are read
    // with hand-issued LDS reads, so that no copy of them stays live across the k-loop (the
    // epilogue reads the metadata again).
    // A reduction unit of the single-launch broadcast is the producers' work: every consumer
    // wave treats it as idle.
    if ((MODES == kModesBroadcast && uni(lds_peek(&ti->mode)) == kModeReduce) ||
        wm * C::WTM >= (int)uni(lds_peek(reinterpret_cast<const uint32_t*>(&ti->m_rows))) ||
        wn * C::WTN >= (int)uni(lds_peek(reinterpret_cast<const uint32_t*>(&ti->n_cols)))) {
      lds_bump(&empty[s0]);
      ++g;
      for (int st = 1; st < nsteps; ++st, ++g) {
        const int s = g % C::STAGES;
        wait_at_least(&full[s], (uint32_t)C::NPROD * (g / C::STAGES + 1), abort);
        lds_bump(&empty[s]);
      }
      continue;
    }

    f32x4 acc[C::TM16][C::TN16];
    if (!init_acc16<C, MODES>(acc, ti, guards, epi, wm, wn, abort)) break;

    bf16x8 a[HM], b[C::TN16];
    {
      const char* slot0 = ring + s0 * C::STAGE_BYTES;
#pragma unroll
      for (int tn = 0; tn < C::TN16; ++tn) b[tn] = load_b(slot0, 0, tn);
#pragma unroll
      for (int tm = 0; tm < HM; ++tm) a[tm] = load_a(slot0, 0, tm);
    }
    for (int st = 0; st < nsteps; ++st, ++g) {
      const int s = g % C::STAGES;
      const char* slot = ring + s * C::STAGE_BYTES;
      const bool more_steps = st + 1 < nsteps;
      const int sn = (g + 1) % C::STAGES;
      const char* next_slot = ring + sn * C::STAGE_BYTES;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bool last_ks = ks == C::KS - 1;
        const bool more = !last_ks || more_steps;   // a slice follows in this tile
        const char* nslot = last_ks ? next_slot : slot;
        const int nks = last_ks ? 0 : ks + 1;
        __builtin_amdgcn_sched_barrier(0);
        // first half: row blocks 0 .. HM-1, row-major; refill with the second half's rows
#pragma unroll
        for (int tm = 0; tm < HM; ++tm) {
#pragma unroll
          for (int tn = 0; tn < C::TN16; ++tn) {
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[tn], a[tm], acc[tm][tn], 0, 0, 0);
          }
          a[tm] = load_a(slot, ks, tm + HM);
          __builtin_amdgcn_sched_barrier(0);
        }
        // second half: row blocks HM .. TM16-1, column-major
#pragma unroll
        for (int tn = 0; tn < C::TN16; ++tn) {
#pragma unroll
          for (int tm = 0; tm < HM; ++tm) {
            acc[tm + HM][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[tn], a[tm], acc[tm + HM][tn], 0, 0, 0);
            if (tn == C::TN16 - 1 && more) a[tm] = load_a(nslot, nks, tm);
          }
          if (tn == 0 && last_ks) {
            // every read of slot s has been consumed: release it, and make sure the next
            // slot has landed before the first read from it
            wait_lgkm0();
            lds_bump(&empty[s]);
            if (more) wait_at_least(&full[sn], (uint32_t)C::NPROD * ((g + 1) / C::STAGES + 1), abort);
          }
          if (more) b[tn] = load_b(nslot, nks, tn);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    const uint32_t tmode = MODES != kModesNone ? uni(ti->mode) : 0u;
    // a split tile: the unit that arrives second finishes it
    if (MODES == kModesSplit && (tmode == 1 || tmode == 2) &&
        !combine_split16<C>(acc, ti, cw % C::NCG, guards, abort)) {
      if (uni(lds_peek(abort)) != 0) break;
      continue;
    }

    // a user-phase partial product goes to the workspace in fp32, without an epilogue
    // operation, on the agent-coherent path
    const bool partial = MODES == kModesBroadcast && tmode == kModeUserPartial;
    const bool out4 = f32out || partial;
    const int m_rows = (int)uni((uint32_t)ti->m_rows);
    const int n_cols = (int)uni((uint32_t)ti->n_cols);
    const uint64_t Cp = uni64(ti->C);
    const int ldc = (int)uni((uint32_t)ti->ldc);
    if (m_rows < 1 || m_rows > C::BM || n_cols < 1 || n_cols > C::BN || ldc < n_cols) {
      raise_abort(abort, 2u);
      break;
    }
    const uint64_t c_bytes = (uint64_t)((int64_t)(m_rows - 1) * ldc + n_cols) * (out4 ? 4u : 2u);
    if (!inside(Cp, c_bytes, uni64(partial ? guards->w_lo : guards->c_lo), uni64(partial ? guards->w_hi : guards->c_hi))) {
      raise_abort(abort, 8u);
      break;
    }
    epilogue16<C>(acc, wm, wn, m_rows, n_cols, Cp, ldc, !partial && (epi == EPI_SILU || epi == EPI_BIAS_SILU), out4,
                  partial);
    if (partial) {
      // the partial product, written on the agent-coherent path, has completed (the reduction
      // may run on another XCD) before the wave's arrival flag carries this launch's epoch
      wait_vmcnt<0>();
      if (lane_id() == 0)
        __hip_atomic_store(reinterpret_cast<uint32_t*>(uni64(ti->sync)) + (cw % C::NCG), uni(ti->epoch),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------------------
template <class C, class S>
__global__ __launch_bounds__(C::NT, 1) void ptg_kernel(typename S::Args args) {
  constexpr int kFlags = 2 * C::STAGES + 1;  // full[], empty[], abort
  __shared__ __attribute__((aligned(1024))) char smem[C::RING_BYTES + C::NINFO * sizeof(TileInfo) +
                                                    sizeof(Guards) + kFlags * sizeof(uint32_t) +
                                                    S::LDS_BYTES];
  char* ring = smem;
  TileInfo* info = reinterpret_cast<TileInfo*>(smem + C::RING_BYTES);
  Guards* guards = reinterpret_cast<Guards*>(smem + C::RING_BYTES + C::NINFO * sizeof(TileInfo));
  uint32_t* full = reinterpret_cast<uint32_t*>(guards + 1);
  uint32_t* empty = full + C::STAGES;
  uint32_t* abort = empty + C::STAGES;
  char* sched_lds = reinterpret_cast<char*>(full + kFlags);
  if (threadIdx.x < kFlags) full[threadIdx.x] = 0;
  // The operand ranges wait in LDS until a check needs them (kept in registers they would
  // occupy two dozen scalar registers for the whole kernel).
  if (threadIdx.x == 0) *guards = S::guards(args);
  S::template init<C>(args, sched_lds);  // cooperative; the barrier below publishes it
  __syncthreads();
  const int wave = (int)uni(threadIdx.x >> 6);  // the same for every lane of a wave
  if (wave < C::NCONS) {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (C::M16)
      consumer_role16<C, S::kModes>(ring, info, full, empty, abort, wave, args.epi, args.out_f32 != 0, guards);
    else
      consumer_role<C>(ring, info, full, empty, abort, wave, args.epi, args.out_f32 != 0, guards);
  } else {
    if constexpr (C::PREG == 1)
      producer_role_regs<C, S>(args, ring, info, full, empty, abort, wave - C::NCONS, sched_lds, guards);
    else
      producer_role<C, S>(args, ring, info, full, empty, abort, wave - C::NCONS, sched_lds, guards);
  }
}

}  // namespace ptg
