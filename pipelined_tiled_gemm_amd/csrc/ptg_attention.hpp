// ptg_attention.hpp - IKBO attention: every candidate's query attends to its user's keys and
// values (How We Built TLX, "Case Study 2: In-Kernel Broadcast Optimization for RecSys": for
// FlashAttention the co-design amortises the K/V reads across the candidates that share a
// user context, and the kernel is warp-specialised and persistent).
//
// Per user u (candidates [off[u], off[u+1]), contiguous) and head h:
//     O[c] = softmax(scale * Q[c] . K[u]^T) . V[u]
// Q, O: [Mc][H][D]; K, V: [U][L][H][D]; D = 128; L a multiple of 64.
//
// One persistent workgroup per compute unit.  A tile is (user, head, block of 128 of the user's
// candidates); every tile of a user and head reads the same K and V (L2 reuse: consecutive
// tiles are consecutive candidate blocks of one user and head, and land on one XCD).
//   - Two producer waves stage 64-key blocks of K and V (16 KB each) into a four-slot LDS ring
//     with buffer-to-LDS copies, handing each over through the monotone full/empty counters
//     of the GEMM kernel.
//   - Four consumer waves own 32 candidates each.  The whole computation runs transposed, so
//     that a lane owns one query: S^T = K . Q^T (32 keys x 32 queries per MFMA block, the
//     queries' fragments held in registers for the whole tile), then the online softmax per
//     query (a lane and its partner 32 lanes away hold the query's scores), then
//     O^T = V^T . P^T, with P handed from the S^T accumulators to the MFMA operand layout by one
//     v_permlane32_swap.  The running maximum, sum and the rescaling of O are lane-local; the
//     maximum is lazy (it moves only when a score passes it by more than 2^8 in weight), so O
//     is rescaled on few steps.
//   - The epilogue divides by the softmax sum and stores runs of 16 bytes.
// Compiled as its own translation unit (ptg_attention.hip), with its own watchdog word.
#pragma once
#include <hip/hip_runtime.h>

#include "ptg_device.hpp"
#include "ptg_launch.h"

namespace ptg {

namespace attn {

constexpr int D = kAttnHeadDim;     // head dimension
constexpr int BQ = 128;             // candidates per tile
constexpr int BKV = 64;             // keys per ring step
constexpr int STAGES = 4;
constexpr int NCONS = 4, NPROD = 2, NT = (NCONS + NPROD) * 64;
constexpr int ROW_BYTES = D * 2;                  // one key row of K or V (256 bytes)
constexpr int BLK_BYTES = BKV * ROW_BYTES;        // 16 KB
constexpr int STEP_BYTES = 2 * BLK_BYTES;         // K block, then V block
constexpr int LOADS = BLK_BYTES / 1024;           // 1 KB copies per producer per step
constexpr int INFLIGHT = (STAGES < 63 / LOADS) ? STAGES : 63 / LOADS;
static_assert(D == 128 && BLK_BYTES % 1024 == 0, "head dimension 128");
// How far (log2 units) the lazy running maximum of the softmax may trail the true one.
constexpr float kLazyMax = 8.0f;

// K rows are read by ds_read_b128 (16 lanes = 16 consecutive keys at one chunk): the chunk
// index XOR the key's low 4 bits puts them in 16 distinct 16-byte bank groups.  V rows are read
// transposed (4 keys x 32 bytes per 16 lanes) and use the K x N swizzle of the GEMM.
__host__ __device__ constexpr int swz_key(int key) { return key & 15; }

struct Args {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  char* O;
  const int32_t* offsets;       // [U + 1]
  int64_t Mc;
  int32_t U, H, L;
  int32_t out_f32;
  float scale_log2;             // scale * log2(e)
  uint64_t q_bytes, kv_bytes, o_bytes;
};

// The tile of sequence number j of this workgroup, from the per-user block prefix in LDS.
struct Tile {
  int u, h, q0, nq;             // user, head, first candidate, valid candidates (<= BQ)
};

__device__ __forceinline__ bool tile_of(const Args& a, const int32_t* off, const int32_t* pre, int j, Tile& t) {
  const int64_t L = (int64_t)j * gridDim.x + xcd_rank(blockIdx.x, gridDim.x);
  if (L >= pre[a.U]) return false;
  int lo = 0, hi = a.U;  // largest u with pre[u] <= L
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)pre[mid] <= L) lo = mid;
    else hi = mid;
  }
  const int u = lo;
  const int local = (int)(L - pre[u]);
  const int cnt = off[u + 1] - off[u];
  const int qb = (cnt + BQ - 1) / BQ;
  t.u = u;
  t.h = local / qb;
  t.q0 = off[u] + (local % qb) * BQ;
  t.nq = min(BQ, off[u + 1] - t.q0);
  return true;
}

// ---------------------------------------------------------------------------------------
// Producer: wave 0 copies the K block of each step, wave 1 the V block.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void producer(const Args& a, const int32_t* off, const int32_t* pre, char* ring,
                                         uint32_t* full, uint32_t* empty, uint32_t* abort, int pid) {
  const int lane = lane_id();
  const bool isK = pid == 0;
  const int64_t rs = (int64_t)a.H * D * 2;  // bytes between consecutive keys
  const int nsteps = a.L / BKV;
  // Per-lane offsets within a step: copy i covers keys 4 i .. 4 i + 3; lane l fills physical
  // chunk l % 16 of key 4 i + l / 16, which holds the logical chunk XOR the swizzle.
  uint32_t voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int key = 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ (isK ? swz_key(key) : swz_n<16>(key));
    voff[i] = (uint32_t)(key * rs + chunk * 16);
  }
  const char* base_all = reinterpret_cast<const char*>(isK ? a.K : a.V);
  uint32_t g = 0, next_sig = 0;
  for (int j = 0;; ++j) {
    Tile t;
    if (!tile_of(a, off, pre, j, t)) break;
    // this user's and head's rows: key k at base + k * rs
    const uint64_t base_off = ((uint64_t)t.u * a.L * a.H + (uint64_t)t.h) * D * 2;
    const uint32_t bytes = (uint32_t)((int64_t)(a.L - 1) * rs + D * 2);
    if (base_off + bytes > a.kv_bytes) {
      raise_abort(abort, 4u);
      break;
    }
    const char* src = base_all + base_off;
    for (int st = 0; st < nsteps; ++st, ++g) {
      const int s = g % STAGES;
      const uint32_t released = (uint32_t)NCONS * (g / STAGES);
      if (uni(lds_peek(&empty[s])) < released) {
        wait_vmcnt<0>();
        for (; next_sig < g; ++next_sig) lds_bump(&full[next_sig % STAGES]);
        wait_at_least(&empty[s], released, abort);
        if (uni(lds_peek(abort)) != 0) return;
      }
      char* dst = ring + s * STEP_BYTES + (isK ? 0 : BLK_BYTES);
      const int64_t kbytes = (int64_t)st * BKV * rs;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(src + kbytes, bytes - (uint32_t)kbytes);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dma16(r, dst + i * 1024, voff[i], 0);
      if (g + 1 - next_sig == (uint32_t)INFLIGHT) {
        wait_vmcnt<(INFLIGHT - 1) * LOADS>();
        lds_bump(&full[next_sig % STAGES]);
        ++next_sig;
      }
    }
  }
  wait_vmcnt<0>();
  for (; next_sig < g; ++next_sig) lds_bump(&full[next_sig % STAGES]);
}

// ---------------------------------------------------------------------------------------
// Consumer
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float partner(float v, int lane) {
  // the value of lane l ^ 32 (v_permlane32_swap of v with itself: the first result holds the
  // upper lanes' partners, the second the lower lanes')
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                  false, false);
  return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
}

// NEG: the scale is negative.
template <bool NEG>
__device__ __forceinline__ void consumer(const Args& a, const int32_t* off, const int32_t* pre, char* ring,
                                         uint32_t* full, uint32_t* empty, uint32_t* abort, int cw) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const int lane = lane_id();
  const int hi = lane >> 5;
  const int nsteps = a.L / BKV;
  const float s_log2 = a.scale_log2, s_abs = NEG ? -a.scale_log2 : a.scale_log2;
  // K fragment (MFMA A operand: key row lane % 32 of a 32-key block, d-chunk 2 kk + hi of the
  // 16-deep slice kk): physical chunk (2 kk + hi) ^ (key & 15) = (hi ^ (lane & 15)) ^ 2 kk.
  const int k_off = (lane & 31) * ROW_BYTES + ((hi ^ (lane & 15)) << 4);
  // V^T fragment (A operand: d row lane % 32 of a 32-row block, keys 8 hi .. + 7 of a 16-key
  // slice), read transposed as the GEMM's K x N B tiles: group b of 16 lanes reads keys
  // 8 (b / 2) + i / 4 (and 4 further on) at d 16 (b % 2) + 4 (i % 4) .. + 3.  The d-block db
  // (32 columns, 4 chunks) is an XOR of db << 6 on the offset (the base chunk is below 4).
  int v_off;
  {
    const int b = lane >> 4, i = lane & 15;
    const int key = (b >> 1) * 8 + (i >> 2);
    const int d = (b & 1) * 16 + (i & 3) * 4;
    v_off = key * ROW_BYTES + (((d >> 3) ^ swz_n<16>(key)) << 4) + ((d >> 2) & 1) * 8;
  }
  // the per-slice K offsets and per-d-block V offsets, kept in registers so that a fragment
  // read costs one address add (the slot) and an immediate offset (block, slice)
  int koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = k_off ^ (kk << 5);
#pragma unroll
  for (int db = 0; db < 4; ++db) voff[db] = v_off ^ (db << 6);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.Q, (uint32_t)a.q_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.O, (uint32_t)a.o_bytes);

  uint32_t g = 0;
  for (int j = 0;; ++j) {
    Tile t;
    if (!tile_of(a, off, pre, j, t)) break;
    // this wave's 32 queries; lane l holds query q = l % 32 (both halves)
    const int qrow = cw * 32 + (lane & 31);
    const bool q_ok = qrow < t.nq;
    const int64_t cand = (int64_t)t.q0 + qrow;
    // Q fragments (MFMA B operand: query lane % 32, d 8 hi .. + 7 of the 16-deep slice kk)
    bf16x8 qf[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint32_t vo = q_ok ? (uint32_t)(((cand * a.H + t.h) * D + kk * 16 + hi * 8) * 2) : kOutOfRange;
      qf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, vo, 0, 0));
    }
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    float m = -__builtin_inff(), l = 0.0f;

    // S^T = K . Q^T for the 64 keys of a staged step (two 32-key blocks).
    auto qk = [&](const char* kb_lds, f32x16 (&sc)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(kb_lds + kb * 32 * ROW_BYTES + koff[kk]);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sc[kb], 0, 0, 0);
        }
      }
    };
    // Online softmax of one step's scores (log2 domain, scale s), with a lazy running maximum:
    // m moves only when some query of the wave meets a score more than kLazyMax above it.
    // Until then the weights exp2(s x - m) stay below 2^kLazyMax and O and l keep their scale
    // (numerator and denominator share it, so the quotient is the same softmax), which saves
    // the rescaling of O on almost every step.  The maximum of s x is taken as |s| times the
    // maximum of x (of -x when s < 0): the same value, since rounding is monotone.
    auto softmax = [&](f32x16 (&sc)[2]) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, NEG ? -sc[kb][r] : sc[kb][r]);
      mx = fmaxf(mx, partner(mx, lane)) * s_abs;
      if (__builtin_amdgcn_ballot_w64(mx > m + kLazyMax) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      float rp[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four partial sums: no 32-long add chain
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], s_log2, -m));
          rp[r & 3] += sc[kb][r];
        }
      float rs = (rp[0] + rp[1]) + (rp[2] + rp[3]);
      rs += partner(rs, lane);
      l += rs;
    };
    // O^T += V^T . P^T over the step's four 16-key slices.  The P^T fragment of slice (kb, sl):
    // keys 8 hi .. + 7 for query lane % 32; register group r / 4 = gq holds keys 8 gq + 4 hi +
    // (0..3), and lanes l and l + 32 trade so that each holds 8 consecutive keys.
    auto pv = [&](const char* vb_lds, const f32x16 (&sc)[2]) {
#pragma unroll
      for (int sl4 = 0; sl4 < 4; ++sl4) {
        const int kb = sl4 >> 1, g0 = 2 * (sl4 & 1), g1 = g0 + 1;
        const uint32_t a0 = pack_bf16(sc[kb][4 * g0], sc[kb][4 * g0 + 1]);
        const uint32_t a1 = pack_bf16(sc[kb][4 * g0 + 2], sc[kb][4 * g0 + 3]);
        const uint32_t b0 = pack_bf16(sc[kb][4 * g1], sc[kb][4 * g1 + 1]);
        const uint32_t b1 = pack_bf16(sc[kb][4 * g1 + 2], sc[kb][4 * g1 + 3]);
        const auto w0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto w1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const u32x4 pw = {w0[0], w1[0], w0[1], w1[1]};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int off_v = voff[db] + sl4 * 16 * ROW_BYTES;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb_lds + off_v));
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb_lds + off_v + 4 * ROW_BYTES));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
    };

    // Software pipeline over the steps: the next step's S^T MFMAs are issued together with the
    // current step's softmax (independent work for the matrix core and the vector ALU of the
    // same wave), then the current step's O^T MFMAs.  The last step runs without a successor.
    f32x16 sc[2];
    {
      const int s = g % STAGES;
      wait_at_least(&full[s], (uint32_t)NPROD * (g / STAGES + 1), abort);
      if (uni(lds_peek(abort)) != 0) return;
      qk(ring + s * STEP_BYTES, sc);
    }
    for (int st = 0; st + 1 < nsteps; ++st, ++g) {
      const int s = g % STAGES, sn = (g + 1) % STAGES;
      wait_at_least(&full[sn], (uint32_t)NPROD * ((g + 1) / STAGES + 1), abort);
      if (uni(lds_peek(abort)) != 0) return;
      f32x16 scn[2];
      qk(ring + sn * STEP_BYTES, scn);
      softmax(sc);
      pv(ring + s * STEP_BYTES + BLK_BYTES, sc);
      // every read of slot s has landed in registers: release it
      wait_lgkm0();
      lds_bump(&empty[s]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sc[kb] = scn[kb];
    }
    {
      const int s = g % STAGES;
      softmax(sc);
      pv(ring + s * STEP_BYTES + BLK_BYTES, sc);
      wait_lgkm0();
      lds_bump(&empty[s]);
      ++g;
    }
    // ---- epilogue: O = O^T / l; register r of o[db] is d = 32 db + 8 (r / 4) + 4 hi + r % 4 -
    const float inv = 1.0f / l;
    if (a.out_f32) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = db * 32 + gq * 8 + hi * 4;
          const uint32_t vo = q_ok ? (uint32_t)(((cand * a.H + t.h) * D + d) * 4) : kOutOfRange;
          const f32x4 v = {o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                           o[db][4 * gq + 3] * inv};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, vo, 0, 0);
        }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          // groups 2p and 2p + 1: after the trade lane hi = 0 holds d 16 p + 0..7, hi = 1 holds
          // d 16 p + 8..15 (of the d-block)
          const int g0 = 2 * p, g1 = 2 * p + 1;
          const uint32_t x0 = pack_bf16(o[db][4 * g0] * inv, o[db][4 * g0 + 1] * inv);
          const uint32_t x1 = pack_bf16(o[db][4 * g0 + 2] * inv, o[db][4 * g0 + 3] * inv);
          const uint32_t y0 = pack_bf16(o[db][4 * g1] * inv, o[db][4 * g1 + 1] * inv);
          const uint32_t y1 = pack_bf16(o[db][4 * g1 + 2] * inv, o[db][4 * g1 + 3] * inv);
          const auto w0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto w1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const u32x4 v = {w0[0], w1[0], w0[1], w1[1]};
          const int d = db * 32 + p * 16 + hi * 8;
          const uint32_t vo = q_ok ? (uint32_t)(((cand * a.H + t.h) * D + d) * 2) : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(v, ro, vo, 0, 0);
        }
    }
  }
}

__global__ __launch_bounds__(NT, 1) void attention_kernel(Args a) {
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * STEP_BYTES];
  __shared__ uint32_t flags[2 * STAGES + 1];
  __shared__ int32_t off[kMaxGroups + 1];
  __shared__ int32_t pre[kMaxGroups + 1];
  __shared__ int32_t scan_tmp[NT / 64 + 1];
  uint32_t* full = flags;
  uint32_t* empty = flags + STAGES;
  uint32_t* abort = flags + 2 * STAGES;
  if (threadIdx.x < 2 * STAGES + 1) flags[threadIdx.x] = 0;
  // offsets clamped to [0, Mc] (the precondition says they are; the clamp keeps every access
  // inside Q and O even when a caller breaks it)
  for (int i = threadIdx.x; i <= a.U; i += NT) {
    const int64_t o = a.offsets[i];
    off[i] = (int32_t)(o < 0 ? 0 : (o > a.Mc ? a.Mc : o));
  }
  __syncthreads();
  // tiles of user u: heads x candidate blocks
  {
    const int tid = threadIdx.x, ln = tid & 63, wv = tid >> 6;
    const int per = (a.U + NT - 1) / NT;
    const int lo = min(a.U, tid * per), hi = min(a.U, lo + per);
    int32_t local = 0;
    for (int i = lo; i < hi; ++i) {
      const int cnt = max(off[i + 1] - off[i], 0);
      local += ((cnt + BQ - 1) / BQ) * a.H;
    }
    int32_t inc = local;
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t v = __shfl_up(inc, d, 64);
      if (ln >= d) inc += v;
    }
    if (ln == 63) scan_tmp[wv] = inc;
    __syncthreads();
    if (tid == 0) {
      int32_t run = 0;
      for (int w = 0; w < NT / 64; ++w) {
        const int32_t x = scan_tmp[w];
        scan_tmp[w] = run;
        run += x;
      }
      scan_tmp[NT / 64] = run;
    }
    __syncthreads();
    int32_t run = scan_tmp[wv] + inc - local;
    for (int i = lo; i < hi; ++i) {
      pre[i] = run;
      const int cnt = max(off[i + 1] - off[i], 0);
      run += ((cnt + BQ - 1) / BQ) * a.H;
    }
    if (tid == 0) pre[a.U] = scan_tmp[NT / 64];
    __syncthreads();
  }
  const int wave = (int)uni(threadIdx.x >> 6);
  if (wave < NCONS) {
    __builtin_amdgcn_s_setprio(1);
    if (a.scale_log2 < 0.0f) consumer<true>(a, off, pre, ring, full, empty, abort, wave);
    else consumer<false>(a, off, pre, ring, full, empty, abort, wave);
  } else {
    producer(a, off, pre, ring, full, empty, abort, wave - NCONS);
  }
}

}  // namespace attn

hipError_t launch_attention(const AttentionLaunch& p, hipStream_t stream) {
  attn::Args a;
  a.Q = reinterpret_cast<const __bf16*>(p.Q);
  a.K = reinterpret_cast<const __bf16*>(p.K);
  a.V = reinterpret_cast<const __bf16*>(p.V);
  a.O = reinterpret_cast<char*>(p.O);
  a.offsets = p.offsets;
  a.Mc = p.Mc;
  a.U = (int32_t)p.U;
  a.H = (int32_t)p.H;
  a.L = (int32_t)p.L;
  a.out_f32 = p.out_f32;
  a.scale_log2 = (float)(p.scale * 1.4426950408889634);
  a.q_bytes = (uint64_t)p.Mc * p.H * attn::D * 2;
  a.kv_bytes = (uint64_t)p.U * p.L * p.H * attn::D * 2;
  a.o_bytes = (uint64_t)p.Mc * p.H * attn::D * (p.out_f32 ? 4 : 2);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) return hipErrorNoDevice;
  // the tile count lives on the device (it depends on the offsets): one workgroup per CU,
  // idle ones exit at once
  hipLaunchKernelGGL(attn::attention_kernel, dim3((unsigned)cus), dim3(attn::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ptg
