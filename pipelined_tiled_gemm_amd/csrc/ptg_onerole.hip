// ptg_onerole.hip - the one-role dense GEMM kernel and its watchdog word.
//
// The pipelined tiled GEMM of "Introducing TLX" (listing 1: acc = 0; for each K block load the
// A and B tiles, acc += A.B; store), with the loads run ahead of the matrix work through a ring
// of LDS slots as the warp-specialised kernels of that page and of "How We Built TLX" do.  Here
// the roles are not split over separate waves: each of the four waves issues a quarter of every
// k-step's memory-to-LDS copies and computes a 128 x 128 quarter of the 256 x 256 output tile.
// With one wave per SIMD a wave stall is a matrix-core stall, so the loop is written for an
// uninterrupted instruction stream:
//   - copies go straight from memory into LDS (buffer loads with the LDS flag) into five
//     32-deep slots of 32 KB;
//   - copies go in pairs of k-steps (2p, 2p + 1), whose two 64-byte halves make up each
//     128-byte row segment: each copy of step 2p is followed, 8 MFMAs later, by the copy of
//     the same rows of step 2p + 1, so the second half is served by the line the first
//     brought into L1 (one L2 request per line instead of two).  A pair is split by rows over two steps
//     (rows of copies 0-3 at step 2p - 4, 4-7 at step 2p - 3), so every step issues 8
//     copies per wave, one after every 8th MFMA;
//   - the k-loop is unrolled over ten steps (two turns of the ring), so every fragment read
//     is a fixed per-lane base register plus an immediate offset: no address arithmetic sits
//     between the MFMAs;
//   - the MFMAs are inline asm, which fixes the issue order of every LDS and memory access
//     between them to the source order.
// One barrier per step.  Before it, each wave waits for its own copies of step st + 1 and for
// its reads of step st's slot (its fragments were read during step st - 1).  After it, step
// st + 1 is complete in LDS, and every wave has finished step st - 1, so the slots of steps
// st - 1 and st (their fragments are in registers) take the copies issued during step st:
// steps st + 4 and st + 5 at even steps, st + 3 and st + 4 at odd steps (the same slots mod 5).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ptg_device.hpp"
#include "ptg_launch.h"

namespace ptg {

namespace {

// 256 x 256 x 32 tile, five slots; 2 x 2 waves of 128 x 128 (16 x 16 MFMA blocks); the
// producer count (4) fixes each wave's share of a step's 1 KB copies (8).  B stored N x K
// (KN false) or K x N (KN true).
template <bool KN>
using CfgOneRole = Cfg<256, 256, 32, 5, 2, 2, 4, KN, 1, true, false, false, 1>;

struct OneRoleArgs {
  const __bf16* A;
  const __bf16* B;
  char* C;
  const float* bias;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t epi;
  Guards guard;
};

// Tile L of the launch order.  Tiles are taken in blocks of 16 x 16 (row-major over block
// rows, the block columns of odd block rows in reverse, so that consecutive blocks share a
// panel of A or of B); inside a block, in strips of four tile rows taken column by column.
// A persistent launch of 256 workgroups runs tiles j * 256 + xcd_rank(w): round j is one
// block, and the 32 workgroups of one XCD (one L2) take a 4 x 8 patch of it, which reads 4
// panels of A and 8 of B.  Edge blocks and strips are smaller; the order stays a bijection.
__device__ __forceinline__ void onerole_tile(uint64_t L, uint32_t tiles_m, uint32_t tiles_n, int& tm, int& tn) {
  // unsigned throughout: every quantity is nonnegative, and 32-bit values widen by zero
  // extension
  const uint64_t row_tiles = 16ull * tiles_n;
  const uint32_t bi = (uint32_t)(L / row_tiles);
  uint64_t in = L - (uint64_t)bi * row_tiles;
  const uint32_t bm = min(16u, tiles_m - 16u * bi);
  const uint32_t nbj = (tiles_n + 15u) / 16u;
  const uint32_t last_bn = tiles_n - 16u * (nbj - 1u);
  uint32_t bj, bn;
  if ((bi & 1u) == 0) {
    bj = (uint32_t)(in / (16ull * bm));
    in -= (uint64_t)bj * 16u * bm;
    bn = min(16u, tiles_n - 16u * bj);
  } else if (in < (uint64_t)last_bn * bm) {
    // odd block row: the (possibly narrower) last block column comes first
    bj = nbj - 1u;
    bn = last_bn;
  } else {
    in -= (uint64_t)last_bn * bm;
    const uint32_t e = 1u + (uint32_t)(in / (16ull * bm));
    in -= (uint64_t)(e - 1u) * 16u * bm;
    bj = nbj - 1u - e;
    bn = 16u;
  }
  const uint32_t s = (uint32_t)(in / (4ull * bn));
  const uint32_t in3 = (uint32_t)(in - (uint64_t)s * 4u * bn);
  const uint32_t sm = min(4u, bm - 4u * s);
  tm = (int)(16u * bi + 4u * s + in3 % sm);
  tn = (int)(16u * bj + in3 / sm);
}

// One 16-byte-per-lane copy from memory into LDS (M0 + lane * 16), written as asm.  The
// compiler tracks a copy made with the builtin as an LDS write, and before an LDS read it
// cannot prove disjoint from it (the transposing reads of B stored K x N) it waits for every
// copy in flight, which serialises copies and matrix work; it does not track asm.  The kernel
// orders copies and reads itself (per-step vector-memory waits and the barrier).  The
// descriptor is built in scalar registers: base, stride 0, size, the flags make_rsrc uses.
// Nor does the compiler insert wait states before an asm instruction.  A copy to LDS right
// after a scalar write of M0 may use the old M0 (the wrong place): the s_nop inside the asm
// gives the one wait state needed.  A memory instruction reading a scalar register that a
// vector instruction wrote (v_readfirstlane) needs 5: the descriptor words are computed with
// scalar instructions only (checked on the compiled kernel), so none comes that way.
__device__ __forceinline__ void copy_lds16(uint64_t base, uint32_t nbytes, uint32_t lds, uint32_t voff) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4s;
  const u32x4s d = {uni((uint32_t)base), uni((uint32_t)(base >> 32)) & 0xffffu, uni(nbytes), 0x00020000u};
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(d), "{m0}"(uni(lds))
               : "memory");
}

// F32: fp32 output (else bf16), a template argument: the two epilogues behind one runtime
// branch make the compiler spill registers across the whole kernel
template <class C, bool F32>
__global__ __launch_bounds__(256, 1) void onerole_kernel(OneRoleArgs args) {
  __shared__ __attribute__((aligned(1024))) char ring[C::STAGES * C::STAGE_BYTES];
  constexpr int S = C::STAGES, L = C::LOADS;
  static_assert(C::BK == 32 && L == 8 && S == 5, "five 32-deep slots, 8 copies per wave");
  constexpr int TM = C::TM16, TN = C::TN16;  // 8 x 8 blocks of 16 x 16 per wave
  static_assert(TM == 8 && TN == 8, "128 x 128 per wave");
  const int w = (int)uni(threadIdx.x >> 6);
  const int lane = lane_id();
  const int wm = w >> 1, wn = w & 1;
  const int i0 = w * L;                      // this wave's copies: 1 KB chunks i0 .. i0 + 7
  const bool opA = i0 < C::A_INSTR;
  const int wave_lds = opA ? i0 * 1024 : C::A_BYTES + (i0 - C::A_INSTR) * 1024;
  const uint32_t ring_lds = uni(lds_addr(ring));   // the ring's LDS byte address

  // Fragment bases.  A (and B stored N x K): lane l reads row (l mod 16) of a 16-row block,
  // 16-byte k-chunk l / 16 (swizzled as the copies laid it out).  B stored K x N: two
  // transposing 8-byte reads per fragment, 4 k-rows apart; block t's base is the lane's base
  // XOR t * 32 bytes (the swizzle XORs chunk bits 1-3, which the wave's column offset leaves
  // clear), one register per block.  Slots 0-1 through base set 0, 2-3 through set 1, 4
  // through set 2 (a read's immediate offset holds 16 bits).  Opaque, so that they stay in
  // registers instead of being re-derived inside the loop.
  const int ra = wm * C::WTM + (lane & 15);
  int a0 = ra * C::BK * 2 + (((lane >> 4) ^ swz_k<C::CPR_A>(ra)) << 4);
  int a1 = a0 + 2 * C::STAGE_BYTES;
  int a2 = a0 + 4 * C::STAGE_BYTES;
  asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2));
  constexpr int NBB = C::B_KN ? TN : 1;      // B bases per slot group
  int bb[3][NBB];
  if constexpr (!C::B_KN) {
    const int rb = wn * C::WTN + (lane & 15);
    bb[0][0] = C::A_BYTES + rb * C::BK * 2 + (((lane >> 4) ^ swz_k<C::CPR_B>(rb)) << 4);
  } else {
    const int kr = (lane >> 4) * 8 + ((lane & 15) >> 2);
    const int n = wn * C::WTN + (lane & 3) * 4;
    const int bkn = kr * C::BN * 2 + (((n >> 3) ^ swz_n<C::CPR_B>(kr)) << 4) + ((n >> 2) & 1) * 8;
#pragma unroll
    for (int t2 = 0; t2 < NBB; ++t2) bb[0][t2] = C::A_BYTES + (bkn ^ (t2 << 5));
  }
#pragma unroll
  for (int t2 = 0; t2 < NBB; ++t2) {
    bb[1][t2] = bb[0][t2] + 2 * C::STAGE_BYTES;
    bb[2][t2] = bb[0][t2] + 4 * C::STAGE_BYTES;
#pragma unroll
    for (int g = 0; g < 3; ++g) asm volatile("" : "+v"(bb[g][t2]));
  }
  // Every lambda of the kernel is forced inline: one left out of line takes the accumulators
  // by reference through memory, and stores them right after an asm MFMA whose results the
  // compiler does not know to wait for.
  auto rd = [&](int base, int imm) __attribute__((always_inline)) -> bf16x8 { return *reinterpret_cast<const bf16x8*>(ring + base + imm); };
  auto frag_a = [&](int sl, int t) __attribute__((always_inline)) { return rd(sl < 2 ? a0 : sl < 4 ? a1 : a2, (sl & 1) * C::STAGE_BYTES + t * 16 * C::BK * 2); };
  auto frag_b = [&](int sl, int t) __attribute__((always_inline)) -> bf16x8 {
    const int g = sl < 2 ? 0 : sl < 4 ? 1 : 2;
    if constexpr (!C::B_KN) {
      return rd(bb[g][0], (sl & 1) * C::STAGE_BYTES + t * 16 * C::BK * 2);
    } else {
      const char* p = ring + bb[g][t] + (sl & 1) * C::STAGE_BYTES;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * C::BN * 2));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  const uint64_t ntiles = (uint64_t)(uint32_t)args.tiles_m * (uint32_t)args.tiles_n;
  const int K = args.K;
  const int nsteps = K / C::BK;
  const Guards& gd = args.guard;
  // sizes and leading dimensions are nonnegative: unsigned 64-bit address arithmetic
  const uint64_t lda = (uint64_t)args.lda, ldb = (uint64_t)args.ldb, ldc = (uint64_t)args.ldc;
  for (uint64_t Lt = (uint64_t)xcd_rank(blockIdx.x, gridDim.x); Lt < ntiles; Lt += gridDim.x) {
    int tm = 0, tn = 0;
    onerole_tile(Lt, (uint32_t)args.tiles_m, (uint32_t)args.tiles_n, tm, tn);
    const uint32_t m0 = (uint32_t)tm * C::BM, n0 = (uint32_t)tn * C::BN;
    const int m_rows = min(C::BM, args.M - (int)m0);
    const int n_cols = min(C::BN, args.N - (int)n0);
    // the wave's operand: A (m-rows of K), or B as n-rows of K (N x K) or k-rows of N (K x N)
    const bool kmajor = !opA && C::B_KN;
    const uint64_t ld = opA ? lda : ldb;
    const int extent = opA ? m_rows : n_cols;
    const uint64_t src = uni64(reinterpret_cast<uint64_t>(opA ? args.A + m0 * lda
                                                              : (C::B_KN ? args.B + n0 : args.B + n0 * ldb)));
    uint32_t bytes = kmajor ? (uint32_t)((uint64_t)(uint32_t)(K - 1) * ld * 2u + (uint64_t)(uint32_t)extent * 2u)
                            : (uint32_t)((uint64_t)(uint32_t)(extent - 1) * ld * 2u + (uint64_t)(uint32_t)K * 2u);
    const uint32_t kstride = kmajor ? (uint32_t)ld * 2u : 2u;   // bytes per unit of k
    if (!inside(src, bytes, uni64(opA ? gd.a_lo : gd.b_lo), uni64(opA ? gd.a_hi : gd.b_hi))) {
      if (lane == 0) atomicOr(&g_watchdog, 4u);
      bytes = 0;  // nothing is read: the tile's operand is all zeros
    }
    bytes = uni(bytes);
    // per-lane offset of each copy; rows (or, for B stored K x N, columns) past the tile take
    // an out-of-range offset (zeros)
    uint32_t voff[L];
#pragma unroll
    for (int q = 0; q < L; ++q) {
      int row, c;
      chunk_of<C>(i0 + q, lane, row, c);
      const bool ok = kmajor ? c * 8 < extent : row < extent;
      voff[q] = ok ? (uint32_t)(row * ld * 2 + c * 16) : kOutOfRange;
    }
    // step st's copy q into slot sl: the k-step moves the descriptor base; a step past K
    // gets an empty descriptor (no access, zeros)
    auto copy = [&](int st, int sl, int q) __attribute__((always_inline)) {
      const uint32_t kbytes = (uint32_t)st * C::BK * kstride;
      // bytes left from the step on (operand spans stay below 2 GiB); a signed maximum keeps it
      // in scalar instructions (an unsigned clamp is done in vector ones)
      const uint32_t rem = (uint32_t)max((int32_t)(bytes - kbytes), 0);
      if constexpr (C::B_KN) {
        copy_lds16(src + (rem ? kbytes : 0), rem, ring_lds + (uint32_t)(sl * C::STAGE_BYTES + wave_lds + q * 1024),
                   voff[q]);
      } else {
        // B stored N x K: every fragment read is a plain 16-byte load, which the compiler does
        // not make wait for the builtin's copies (checked on the compiled loop); the builtin
        // form measured 1.6% faster than the asm one here
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const void*>(src + (rem ? kbytes : 0)), rem);
        dma16(rs, ring + sl * C::STAGE_BYTES + wave_lds + q * 1024, voff[q], 0u);
      }
    };

    // accumulators start at the bias (bias epilogues) or zero; lane l holds columns
    // 4 (l / 16) .. + 3 of each 16-column block.  Without a bias nothing is loaded: the
    // compiler waits for every memory access in flight before it uses a loaded value (it does
    // not see that the asm copies issued after the loads are younger), which would hold the
    // first step until the whole prologue has landed.
    f32x4 acc[TM][TN];
    const bool do_bias = (args.epi == EPI_BIAS || args.epi == EPI_BIAS_SILU) && args.bias != nullptr;
    if (do_bias) {
      const uint64_t bp = uni64(reinterpret_cast<uint64_t>(args.bias + n0));
      const bool bias_ok = inside(bp, (uint64_t)n_cols * 4, uni64(gd.bias_lo), uni64(gd.bias_hi));
      if (!bias_ok && lane == 0) atomicOr(&g_watchdog, 8u);
      const __amdgpu_buffer_rsrc_t rbias = make_rsrc(reinterpret_cast<const void*>(bp), bias_ok ? (uint32_t)n_cols * 4u : 0u);
#pragma unroll
      for (int y = 0; y < TN; ++y) {
        const int col = wn * C::WTN + y * 16 + (lane >> 4) * 4;
        const f32x4 b4 = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, col < n_cols ? col * 4 : kOutOfRange, 0, 0));
#pragma unroll
        for (int x = 0; x < TM; ++x) acc[x][y] = b4;
      }
    } else {
#pragma unroll
      for (int y = 0; y < TN; ++y)
#pragma unroll
        for (int x = 0; x < TM; ++x) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // in accumulator registers before the first copy (else the compiler moves them into place
    // after the prologue, behind its wait for every load in flight)
#pragma unroll
    for (int x = 0; x < TM; ++x)
#pragma unroll
      for (int y = 0; y < TN; ++y) asm volatile("" : "+a"(acc[x][y]));
    auto mf = [&](int x, int y, const bf16x8& fa, const bf16x8& fb) __attribute__((always_inline)) {
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[x][y]) : "v"(fb), "v"(fa));
    };

    // prologue: steps 0 .. 3 (pairs 0-1 and 2-3) into slots 0 .. 3; step 0's fragments into
    // registers
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int q = 0; q < L; ++q) copy(st, st, q);
    wait_vmcnt<3 * L>();
    __builtin_amdgcn_s_barrier();
    bf16x8 xa[TM], xb[TN], ya[TM], yb[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) xb[t] = frag_b(0, t);
#pragma unroll
    for (int t = 0; t < TM; ++t) xa[t] = frag_a(0, t);
    // the asm MFMAs do not show the compiler that they read the accumulators just written by
    // ordinary vector instructions: wait states by hand
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

    // The stress build's pause is a small loop: a block boundary, after which the compiler may
    // move accumulators, so the MFMAs' results are waited for first
    auto pause = [&]() __attribute__((always_inline)) {
#if PTG_DELAY_INJECT
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      stress_pause();
#endif
    };
    // Step st = pass start + J (J, 0..9, known at compile time; slot J mod 5): its 64 MFMAs on
    // fa/fb; between them, 8 copies (one after every 8th MFMA) and step st + 1's 16 fragments
    // from slot (J + 1) mod 5 (one per 3 MFMAs, all done well before the step's end)
    auto body = [&](int st, auto Jc, const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN], bf16x8 (&na)[TM],
                    bf16x8 (&nb)[TN]) __attribute__((always_inline)) {
      constexpr int J = decltype(Jc)::value;
      pause();                     // the stress build skews the waves here (a no-op otherwise)
      // this wave's copies of step st + 1 have landed: after its last one came 9 younger
      // copies (st odd: the rest of its step, then one step's 8) or 16 (st even: two steps')
      if constexpr (J % 2 == 1) wait_vmcnt<L + 1>();
      else wait_vmcnt<2 * L>();
      wait_lgkm0();                // and its reads of step st's slot are done
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) {
          const int k = x * TN + y;
          mf(x, y, fa[x], fb[y]);
          // even step: pair p = st / 2 + 2, rows 0..3; odd step: p = (st + 3) / 2, rows 4..7
          if (k % 8 == 2) {
            const int i = k / 8;                    // 0..7: row group i / 2, half i % 2
            const int q = (J % 2 == 0 ? 0 : 4) + i / 2;
            const int n = (J % 2 == 0 ? st + 4 : st + 3) + (i & 1);
            const int ns = (J % 2 == 0 ? J + 4 : J + 3) + (i & 1);
            copy(n, ns % S, q);
          }
          if (k == 35) pause();          // and between the copies and reads of a step
          if (k % 3 == 0 && k / 3 < TN + TM) {
            const int r = k / 3;
            if (r < TN) nb[r] = frag_b((J + 1) % S, r);
            else na[r - TN] = frag_a((J + 1) % S, r - TN);
          }
        }
    };
    auto last = [&](const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN]) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) mf(x, y, fa[x], fb[y]);
    };
    // ten steps per pass: two turns of the ring, whole copy pairs, an even number of swaps
    constexpr int U = 2 * S;
    auto step_j = [&](int st0, auto Jc) __attribute__((always_inline)) {
      constexpr int J = decltype(Jc)::value;
      if constexpr (J % 2 == 0) body(st0 + J, std::integral_constant<int, J>{}, xa, xb, ya, yb);
      else body(st0 + J, std::integral_constant<int, J>{}, ya, yb, xa, xb);
    };
    // Where a block boundary follows an MFMA the compiler may move accumulators between
    // registers (it does at the loop exit); it does not see that the asm MFMAs write them late,
    // so 24 wait states (more than an MFMA's passes) come first
    auto settle = [&]() __attribute__((always_inline)) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); };
    int st = 0;
    for (; st + U < nsteps; st += U) {
      step_j(st, std::integral_constant<int, 0>{});
      step_j(st, std::integral_constant<int, 1>{});
      step_j(st, std::integral_constant<int, 2>{});
      step_j(st, std::integral_constant<int, 3>{});
      step_j(st, std::integral_constant<int, 4>{});
      step_j(st, std::integral_constant<int, 5>{});
      step_j(st, std::integral_constant<int, 6>{});
      step_j(st, std::integral_constant<int, 7>{});
      step_j(st, std::integral_constant<int, 8>{});
      step_j(st, std::integral_constant<int, 9>{});
      settle();
    }
    // 1 to 10 steps left, the first in slot 0 with its fragments in x
    const int left = nsteps - st;
    if (left >= 2) { step_j(st, std::integral_constant<int, 0>{}); settle(); }
    if (left >= 3) { step_j(st, std::integral_constant<int, 1>{}); settle(); }
    if (left >= 4) { step_j(st, std::integral_constant<int, 2>{}); settle(); }
    if (left >= 5) { step_j(st, std::integral_constant<int, 3>{}); settle(); }
    if (left >= 6) { step_j(st, std::integral_constant<int, 4>{}); settle(); }
    if (left >= 7) { step_j(st, std::integral_constant<int, 5>{}); settle(); }
    if (left >= 8) { step_j(st, std::integral_constant<int, 6>{}); settle(); }
    if (left >= 9) { step_j(st, std::integral_constant<int, 7>{}); settle(); }
    if (left >= 10) { step_j(st, std::integral_constant<int, 8>{}); settle(); }
    if ((left - 1) & 1) {
      wait_lgkm0();
#pragma unroll
      for (int t = 0; t < TM; ++t) xa[t] = ya[t];
#pragma unroll
      for (int t = 0; t < TN; ++t) xb[t] = yb[t];
      // the moves are vector writes of the MFMAs' source registers, which the compiler does
      // not know the asm MFMAs read: 8 wait states after them (the asm takes the moved values,
      // so the moves come before it)
      asm volatile("s_nop 7" ::"v"(xa[0]), "v"(xa[1]), "v"(xa[2]), "v"(xa[3]), "v"(xa[4]), "v"(xa[5]), "v"(xa[6]),
                   "v"(xa[7]));
      asm volatile("s_nop 7" ::"v"(xb[0]), "v"(xb[1]), "v"(xb[2]), "v"(xb[3]), "v"(xb[4]), "v"(xb[5]), "v"(xb[6]),
                   "v"(xb[7]));
    }
    last(xa, xb);
    // ... nor that the epilogue reads what they wrote: wait for the last MFMAs' results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    // the copies issued past the last step (empty descriptors) have landed and every wave is
    // done with the ring before the epilogue writes slot 4 and the next tile's prologue
    // refills slots 0-3 (the empty asm keeps the epilogue's LDS writes after the barrier)
    wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    constexpr uint32_t osz = F32 ? 4u : 2u;
    const uint64_t Cp = uni64(reinterpret_cast<uint64_t>(args.C + ((uint64_t)m0 * ldc + n0) * osz));
    const uint64_t c_bytes = ((uint64_t)(uint32_t)(m_rows - 1) * ldc + (uint32_t)n_cols) * osz;
    if (!inside(Cp, c_bytes, uni64(gd.c_lo), uni64(gd.c_hi))) {
      if (lane == 0) atomicOr(&g_watchdog, 8u);
      continue;
    }
    // epilogue: SiLU if asked, conversion, and the store through LDS.  Lane l holds columns
    // 4 (l / 16) .. + 3 of each 16-column block, row l mod 16.  Each wave writes its results
    // into its own 8 KB of slot 4, a piece at a time (32 rows of bf16, 16 rows of fp32), reads
    // them back as 16-byte chunks of whole rows and stores 256-byte (bf16) or 512-byte (fp32)
    // row segments.  A chunk sits at position chunk ^ (row mod 16) in its row, so that neither
    // the writes (16 rows at one column) nor the reads (whole rows) meet on one LDS bank.  The
    // wave's LDS accesses run in order, so a piece's reads see its writes and precede the next
    // piece's writes.  Slot 4 is next written by the copies of the next tile's step 4, issued
    // after a barrier that each wave reaches once its epilogue is done.
    const bool do_silu = args.epi == EPI_SILU || args.epi == EPI_BIAS_SILU;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(reinterpret_cast<void*>(Cp), (uint32_t)c_bytes);
    // the lane index re-read here: offsets derived from it are not hoisted out of the tile loop
    // (they would be held across the k-loop, where no register is free)
    const int elane = opaque_lane();
    char* const stg = ring + 4 * C::STAGE_BYTES + w * 8192;
    const uint32_t ldc_b = (uint32_t)args.ldc * osz;
    auto put = [&](const u32x4_t& v, int row, int col) __attribute__((always_inline)) {
      const uint32_t off = (row < m_rows && col < n_cols) ? (uint32_t)row * ldc_b + (uint32_t)col * osz : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 2);  // non-temporal
    };
    auto act = [&](f32x4 v) __attribute__((always_inline)) -> f32x4 {
      if (do_silu) {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = silu(v[t]);
      }
      return v;
    };
    const int r = elane & 15, g = elane >> 4;
    if constexpr (!F32) {
      // write: 8 bytes, columns y * 16 + 4 g .. + 3 of row 16 h + r (chunk 2 y + g / 2); read:
      // row 4 i + g, chunk r (columns 8 r .. + 7)
#pragma unroll
      for (int pc = 0; pc < TM / 2; ++pc) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int y = 0; y < TN; ++y) {
            const f32x4 v = act(acc[2 * pc + h][y]);
            const uint32_t lo = pack_bf16(v[0], v[1]), hi = pack_bf16(v[2], v[3]);
            *reinterpret_cast<uint2*>(stg + h * 4096 + r * 256 + (((2 * y + (g >> 1)) ^ r) << 4) + (g & 1) * 8) =
                uint2{lo, hi};
          }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 4 * i + g;
          const u32x4_t d = *reinterpret_cast<const u32x4_t*>(stg + row * 256 + ((r ^ (row & 15)) << 4));
          put(d, wm * C::WTM + 32 * pc + row, wn * C::WTN + 8 * r);
        }
      }
    } else {
      // write: 16 bytes, columns y * 16 + 4 g .. + 3 of row r (chunk 4 y + g); read: row
      // 2 i + l / 32, chunk l mod 32 (columns 4 (l mod 32) .. + 3)
      const int q = elane >> 5, c = elane & 31;
#pragma unroll
      for (int x = 0; x < TM; ++x) {
#pragma unroll
        for (int y = 0; y < TN; ++y)
          *reinterpret_cast<f32x4*>(stg + r * 512 + (((4 * y + g) ^ r) << 4)) = act(acc[x][y]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 2 * i + q;
          const u32x4_t d = *reinterpret_cast<const u32x4_t*>(stg + row * 512 + ((c ^ row) << 4));
          put(d, wm * C::WTM + 16 * x + row, wn * C::WTN + 4 * c);
        }
      }
    }
  }
}

// [p, p + bytes), or the empty range when p is null
void span(const void* p, uint64_t bytes, uint64_t& lo, uint64_t& hi) {
  lo = p ? reinterpret_cast<uint64_t>(p) : 0;
  hi = p ? reinterpret_cast<uint64_t>(p) + bytes : 0;
}

// bytes of a row-major [rows x cols] matrix with row stride ld (elements of esize bytes)
uint64_t mat_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  return rows > 0 ? (uint64_t)(((rows - 1) * ld + cols) * esize) : 0;
}

}  // namespace

bool onerole_fits(const DenseLaunch& d) {
  // 32-deep k-steps, no split, no gathered start; and enough 256 x 256 tiles to fill the chip
  // (at least 128), or more 128 x 128 tiles than CUs: there the medium tile needs a second,
  // partial round, while these tiles take one.  From 72 to 121 tiles of 256 x 256 (K = 512 to
  // 8192) this kernel measured 7-19% faster than the medium tile; at 64 (2048^2, 256 medium
  // tiles: one full round) the medium tile was faster.
  if (d.K % 32 != 0 || d.splits > 1 || d.gidx != nullptr || d.P != nullptr) return false;
  const int64_t large = ((d.M + 255) / 256) * ((d.N + 255) / 256);
  const int64_t medium = ((d.M + 127) / 128) * ((d.N + 127) / 128);
  const int cus = device_compute_units();
  return large >= 128 || (cus > 0 && medium > cus);
}

template <bool KN>
static hipError_t launch_onerole_cfg(const DenseLaunch& d, hipStream_t stream) {
  using C = CfgOneRole<KN>;
  OneRoleArgs a{};
  a.A = reinterpret_cast<const __bf16*>(d.A);
  a.B = reinterpret_cast<const __bf16*>(d.B);
  a.C = reinterpret_cast<char*>(d.C);
  a.bias = d.bias;
  a.lda = d.lda; a.ldb = d.ldb; a.ldc = d.ldc;
  a.M = (int32_t)d.M; a.N = (int32_t)d.N; a.K = (int32_t)d.K;
  a.tiles_m = (int32_t)((d.M + C::BM - 1) / C::BM);
  a.tiles_n = (int32_t)((d.N + C::BN - 1) / C::BN);
  a.epi = d.epi;
  Guards& g = a.guard;
  span(d.A, mat_bytes(d.M, d.K, d.lda, 2), g.a_lo, g.a_hi);
  span(d.B, KN ? mat_bytes(d.K, d.N, d.ldb, 2) : mat_bytes(d.N, d.K, d.ldb, 2), g.b_lo, g.b_hi);
  span(d.C, mat_bytes(d.M, d.N, d.ldc, d.out_f32 ? 4 : 2), g.c_lo, g.c_hi);
  span(d.bias, (uint64_t)d.N * 4, g.bias_lo, g.bias_hi);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  const int cus = device_compute_units();
  if (cus <= 0) return hipErrorNoDevice;
  const int grid = (int)(tiles < cus ? tiles : cus);
  if (d.out_f32)
    hipLaunchKernelGGL((onerole_kernel<C, true>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((onerole_kernel<C, false>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_onerole(const DenseLaunch& d, hipStream_t stream) {
  return d.b_kn ? launch_onerole_cfg<true>(d, stream) : launch_onerole_cfg<false>(d, stream);
}

void onerole_describe(int32_t cfg[6]) {
  using C = CfgOneRole<false>;  // the same tile for both layouts
  cfg[0] = C::BM; cfg[1] = C::BN; cfg[2] = C::BK;
  cfg[3] = C::STAGES; cfg[4] = 4; cfg[5] = 0;  // four waves, each copying and computing
}

hipError_t read_onerole_watchdog(uint32_t* value, int clear) {
  hipError_t e = hipMemcpyFromSymbol(value, HIP_SYMBOL(g_watchdog), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_watchdog), &zero, sizeof(uint32_t), 0, hipMemcpyHostToDevice);
}

}  // namespace ptg
