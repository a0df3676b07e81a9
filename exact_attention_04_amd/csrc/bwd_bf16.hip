// Backward pass of exact attention (bf16 inputs, fp32 accumulation, gfx950).
//
// "Warmup Guide -- Inference Optimization at Depth", Ch.4 (backward pass): P
// is not stored; it is recomputed tile by tile from Q and K with the per-row
// statistics kept by the forward pass (here LSE = m + ln l, so P_ij =
// exp(s_ij - LSE_i)).  The gradients are those of the definition of Ch.1
// (S = scale Q K^T with the causal mask, P = softmax(S), O = P V):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),  D_i = sum_j P_ij dP_ij
//     dQ = scale dS K,   dK = scale dS^T Q,
// with D_i = rowsum(dO_i * O_i), which equals sum_j P_ij dP_ij because O = P V.
//
// Two kernels, no atomics (deterministic):
//   * bwd_dq: one workgroup per (batch, head, 256 query rows), laid out like
//     the forward kernel (eight waves in two groups one phase apart, so one
//     wave of every SIMD does matrix work while the other does vector work):
//     each wave holds 32 query rows' Q and dO as MFMA B operands, computes
//     the rows' D_i and LSE_i * log2(e) (written to the workspace for the
//     next kernel), K/V tiles of 32 keys (64 at d = 64) stream through LDS,
//     and per tile
//       S^T = K Q^T, dP^T = V dO^T            (scores transposed: lane = query)
//       dS^T = P^T * (dP^T - D)               (P^T = exp2(S^T c - LSE2))
//       dQ^T += K^T dS^T                      (K^T by LDS transpose reads);
//   * bwd_dkdv: one workgroup per (batch, KV head, 256 keys), eight waves
//     (two per SIMD, so one wave's vector work overlaps the other's matrix
//     work), each wave 32 keys: it holds their K rows as MFMA B operands and
//     reads their V rows from LDS (dK/dV accumulators leave no registers for
//     them); it walks the query tiles of every query head that reads its KV
//     head (grouped-query heads are summed here), Q/dO tiles and their D,
//     LSE2 rows streaming through LDS, and per 32-row block
//       S = Q K^T, dP = dO V^T                (lane = key)
//       dS = P * (dP - D)
//       dV^T += dO^T P, dK^T += Q^T dS        (dO^T, Q^T by LDS transpose reads).
//     All MFMAs are compiler builtins selected in the VGPR form (the vector
//     unit reads S and dP directly); the compiler parks part of the dK/dV
//     accumulators in AGPRs and tracks every matrix-core wait state itself.
#include "device_common.h"
#include "launch.h"
#include "tail_pool.h"

namespace attn {
namespace {

struct BwdKArgs {
  const uint16_t* q;     // [B][H][Sq][D]
  const uint16_t* k;     // [B][Hkv][Sk][D]
  const uint16_t* v;
  const uint16_t* o;     // [B][H][Sq][D]
  const uint16_t* dout;  // [B][H][Sq][D]
  const float* lse;      // [B][H][Sq] natural log
  float* lse2;           // workspace [B][H][Sq]: LSE * log2(e)
  float* dsum;           // workspace [B][H][Sq]: D
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, H, Hkv, Sq, Sk;
  int nqb;   // query blocks of the dQ kernel per (batch, head)
  int nkb;   // key blocks of the dK/dV kernel per (batch, KV head)
  float c2;  // scale * log2(e)
  float scale;
  // dynamic tails (null: every workgroup has a fixed block): the first
  // nstatic_* workgroups take the heavier blocks of every (batch, head), the
  // ndyn_* after them claim the nlight_* lightest blocks from the counter
  unsigned* tail_q;   // bwd_dq: query blocks
  unsigned* tail_kv;  // bwd_dkdv: key blocks
  int nlight_q, nstatic_q, ndyn_q, nlight_kv, nstatic_kv, ndyn_kv;
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

// 16-byte chunk position of a tile row in LDS (XOR swizzle) for tiles that
// are read both ways: row-wise as A operands (16 consecutive rows, one
// chunk each: the swizzle permutes the 16 chunk positions over any 16
// consecutive rows) and by transpose reads (4 consecutive rows x 4
// consecutive chunks: rows 4k..4k+3 differ in the swizzle's upper two bits).
// Both patterns then touch all 64 banks once.
template <int D>
__device__ __forceinline__ int b_swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Workgroup barrier for the tile hand-over: this wave's LDS reads have
// completed, and no instruction is scheduled across it.  Unlike
// __syncthreads() it does not wait for the HBM->LDS loads still in flight
// (a workgroup fence would, and so would drain the prefetch of the next
// tile); where a tile must have landed, vmcnt is waited for explicitly
// first.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---- dQ
// Eight waves, 256 query rows, in two groups of four (one wave of each per
// SIMD) that run one phase apart, as in the forward kernel: per K/V tile a
// wave has a matrix phase (the scores S^T, dP^T of the next tile and this
// tile's dQ^T += K^T dS^T, 24 MFMAs at d = 128) and a vector phase (dS^T of
// the next tile), and workgroup barriers between the phases keep one wave
// of every SIMD on the matrix core while the other does its vector work.
// K_j is read in two rounds (the scores of tile j, then dQ_j), so a tile
// buffer is free again only after the round after its scores; the tiles
// rotate through four LDS buffers, and the loads of round j fill the buffer
// of tile j-1 with tile j+3, which round j+2 reads first (three buffers,
// loads landing within their round, measured 1% slower; five no faster).
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;  // query rows per workgroup
constexpr int kDqStages = 4;            // LDS buffers per K and V stream
constexpr int kDqReadAhead = 4;         // MFMAs between an LDS operand read and its use

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq(BwdKArgs a) {
  constexpr int CPR = D / 8, KS = D / 16, NDB = D / 32;
  // keys per tile: 32 at d = 128, where the scores and dP of a 64-key tile
  // next to dS, the Q, dO operands and the dQ accumulators would not fit in
  // the registers; 64 at d = 64
  constexpr int BC = D == 128 ? 32 : 64;
  constexpr int NKB = BC / 32, NT = BC / 16;  // 32-key blocks, 16-key MFMA steps per tile
  constexpr int TILE = BC * D;
  constexpr int ROWS_PER_INSN = 1024 / (D * 2);
  constexpr int IPW = TILE * 2 / 1024 / kDqWaves;
  static_assert(IPW >= 1, "every wave loads part of each tile");
  // one LDS object per buffer, so the compiler can prove that loads into one
  // buffer never alias reads of another
  static_assert(kDqStages == 4, "one LDS object per buffer below");
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds3[TILE];
  auto kbuf = [&](const int I) __attribute__((always_inline)) {
    return I == 0 ? k_lds0 : I == 1 ? k_lds1 : I == 2 ? k_lds2 : k_lds3;
  };
  auto vbuf = [&](const int I) __attribute__((always_inline)) {
    return I == 0 ? v_lds0 : I == 1 ? v_lds1 : I == 2 ? v_lds2 : v_lds3;
  };
  typedef const __attribute__((address_space(3))) char lds_cchar;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // waves w and w + 4 share a SIMD; w < 4 leads, w >= 4 trails by one
  // phase; their row blocks interleave so both groups reach the same last key
  const bool lead = wave < 4;
  const int rb = 2 * (wave & 3) + (lead ? 0 : 1);
  // heaviest query blocks first, each XCD a contiguous range of heads; with a
  // dynamic tail the lightest quarter of every head's blocks goes last,
  // claimed at run time by whichever XCD gets there first (tail_pool.h)
  int bh, qblk;
  if (CAUSAL && a.tail_q != nullptr) {
    const int nh = a.nqb - a.nlight_q, nbh = a.nstatic_q / nh;
    if ((int)blockIdx.x < a.nstatic_q) {
      const int blk = xcd_grouped_block(blockIdx.x, a.nstatic_q);
      bh = blk / nh;
      qblk = a.nqb - 1 - (blk - bh * nh);
    } else {
      const int c = claim_tail_block(a.tail_q, a.ndyn_q);
      if (c >= nbh * a.nlight_q) return;  // nothing left (uniform over the workgroup)
      bh = c % nbh;
      qblk = a.nlight_q - 1 - c / nbh;
    }
  } else {
    const int blk = xcd_grouped_block(blockIdx.x, gridDim.x);
    bh = blk / a.nqb;
    qblk = blk - bh * a.nqb;
    if (CAUSAL) qblk = a.nqb - 1 - qblk;
  }
  const int b = bh / a.H, hq = bh - b * a.H, g = hq / (a.H / a.Hkv);
  const int q0 = qblk * kDqRows, wq0 = q0 + 32 * rb, shift = a.Sk - a.Sq;
  const int row = wq0 + n;
  const bool row_ok = row < a.Sq;
  const size_t rbase = (size_t)(b * a.H + hq) * a.Sq;
  const uint16_t* Q = a.q + rbase * D;
  const uint16_t* dO = a.dout + rbase * D;
  const uint16_t* K = uniform_ptr(a.k + (size_t)(b * a.Hkv + g) * a.Sk * D);
  const uint16_t* V = uniform_ptr(a.v + (size_t)(b * a.Hkv + g) * a.Sk * D);

  // tiles the workgroup visits (every wave runs all of them: the phases are
  // workgroup-wide); tiles [0, nfull) need no mask for this wave's rows, and
  // tiles from nneed on hold no key any of its rows sees (causal diagonal):
  // the wave skips their matrix and vector work but takes part in the loads
  // and barriers
  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, min(q0 + kDqRows, a.Sq) + shift);
  kend = max(kend, 0);
  const int nkt = (kend + BC - 1) / BC;
  int nfull = a.Sk / BC;
  if (CAUSAL) nfull = min(nfull, max(wq0 + shift + 1, 0) / BC);
  int nneed = nkt;
  if (CAUSAL) nneed = min(nkt, (max(min(wq0 + 31, a.Sq - 1) + shift + 1, 0) + BC - 1) / BC);

  // Q^T and dO^T B operands (column = this lane's row; the two halves of
  // the wave hold alternate 8-value groups of the head dims), and the row
  // statistics: D = rowsum(dO * O) from the same dO values and the matching
  // O values, LSE2 = LSE * log2(e).  They are published for the dK/dV
  // kernel, which runs next; rows that see nothing get no gradient.
  u32x4 qf[KS], df[KS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = row_ok ? load16(Q + (size_t)row * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
    df[ks] = row_ok ? load16(dO + (size_t)row * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
    const u32x4 of = row_ok ? load16(a.o + (rbase + row) * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dpart = fmaf(bf16_lo(of[i]), bf16_lo(df[ks][i]), dpart);
      dpart = fmaf(bf16_hi(of[i]), bf16_hi(df[ks][i]), dpart);
    }
  }
  const float dsum = sum_halves(dpart);
  const float lse2 = row_ok ? a.lse[rbase + row] * kLog2e : -INFINITY;  // -inf stays -inf
  if (row_ok && h == 0) {
    a.dsum[rbase + row] = dsum;
    a.lse2[rbase + row] = lse2;
  }
  const bool live = lse2 != -INFINITY;
  const float lse_use = live ? lse2 : 0.f;

  // HBM -> LDS loads (both tiles in the b_swz layout); the descriptors end
  // at the workgroup's last key, so keys past it, and tiles past the last,
  // read as zeros
  // Load i of this wave covers tile rows (wave IPW + i) ROWS_PER_INSN +
  // lane / CPR; their swizzle differs from load 0's only in the bits i sets
  // (the row's bits 2-3 at d = 128, bit 2 at d = 64), so the lane's offset
  // is voff0 ^ 16 i plus i whole loads of rows.
  static_assert(D == 128 ? IPW <= 4 : IPW <= 2, "the swizzle of load i differs from load 0's by i");
  uint32_t voff0;
  {
    const int r = wave * IPW * ROWS_PER_INSN + lane / CPR;
    voff0 = (r * D + (((lane % CPR) ^ b_swz<D>(r)) * 8)) * 2;
  }
  auto issue_tile = [&](int t, const int BUF) __attribute__((always_inline)) {
    const int j0 = t * BC;
    const int bytes = max(kend - j0, 0) * D * 2;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + (size_t)j0 * D), (short)0, bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + (size_t)j0 * D), (short)0, bytes, kBufferWord3);
    uint16_t* kd = kbuf(BUF);
    uint16_t* vd = vbuf(BUF);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t vo = (voff0 ^ (16 * i)) + i * 1024;
      buffer_load_lds16(kr, kd + (wave * IPW + i) * 512, vo);
      buffer_load_lds16(vr, vd + (wave * IPW + i) * 512, vo);
    }
  };
  // the loads of round j (P = j % S): tile j+S-1 into the buffers of tile
  // j-1, which round j-1 read for the last time; round j+1 reads tile j+2,
  // so at the end of round j each wave may leave the loads of its latest
  // S-3 rounds in flight
  auto issue = [&](int j, const int P) __attribute__((always_inline)) {
    issue_tile(j + kDqStages - 1, (P + kDqStages - 1) % kDqStages);
  };
  constexpr int kInFlight = (kDqStages - 3) * 2 * IPW;

  // LDS byte offsets of the operand reads, one register each: row-major A
  // reads of step ks (row n of a 32-key block) at a_off0 ^ 32 ks, K^T
  // transpose reads of head-dim block db (rows 16t + 4h + r4 and
  // 16t + 8 + 4h + r4, d columns 32db + 16(gq&1) + 4c4 .. +3) at
  // tr_lo0 / tr_hi0 ^ 64 db: the swizzle only permutes chunk bits that the
  // row term never sets.  An opaque redefinition per round keeps the
  // compiler from hoisting the XORs into registers of their own.
  const int gq = lane >> 4, r4 = (lane >> 2) & 3, c4 = lane & 3;
  uint32_t a_off0 = (n * D + ((h ^ b_swz<D>(n)) * 8)) * 2;
  uint32_t tr_lo0, tr_hi0;
  {
    const int dcol = 16 * (gq & 1) + 4 * c4;
    const int rl = 4 * h + r4, rh = 8 + 4 * h + r4;
    tr_lo0 = (rl * D + (((dcol >> 3) ^ b_swz<D>(rl)) * 8) + (dcol & 7)) * 2;
    tr_hi0 = (rh * D + (((dcol >> 3) ^ b_swz<D>(rh)) * 8) + (dcol & 7)) * 2;
  }
  auto refresh_offsets = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(a_off0), "+v"(tr_lo0), "+v"(tr_hi0));
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  f32x16 s[NKB], dp[NKB];  // S^T and dP^T of the next tile (register r of block kb: key 32kb + 8(r/4) + 4h + r%4)
  u32x4 dst[NT];           // dS^T of the current tile, bf16, as MFMA B operands (16-key steps)

  // S^T = K Q^T and dP^T = V dO^T of the tile in buffer BUF (one LDS read
  // per MFMA; the four accumulation chains alternate)
  auto scores = [&](const int BUF) __attribute__((always_inline)) {
    lds_cchar* kb_ = (lds_cchar*)kbuf(BUF);
    lds_cchar* vb_ = (lds_cchar*)vbuf(BUF);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t ao = a_off0 ^ (32 * ks);
        const u32x4 kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kb_ + ao + kb * 32 * D * 2);
        s[kb] = mfma_32x32x16_bf16(kf, qf[ks], s[kb]);
        const u32x4 vf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(vb_ + ao + kb * 32 * D * 2);
        dp[kb] = mfma_32x32x16_bf16(vf, df[ks], dp[kb]);
      }
    }
  };
  // dQ^T += K^T dS^T over the tile's 16-key steps (two transpose reads per
  // MFMA)
  auto dq_update = [&](const int BUF) __attribute__((always_inline)) {
    lds_cchar* kb_ = (lds_cchar*)kbuf(BUF);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb_ + (tr_lo0 ^ (64 * db)) + 16 * t * D * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb_ + (tr_hi0 ^ (64 * db)) + 16 * t * D * 2));
        u32x4 af;
        af[0] = __builtin_bit_cast(u32x2, lo)[0];
        af[1] = __builtin_bit_cast(u32x2, lo)[1];
        af[2] = __builtin_bit_cast(u32x2, hi)[0];
        af[3] = __builtin_bit_cast(u32x2, hi)[1];
        acc[db] = mfma_32x32x16_bf16(af, dst[t], acc[db]);
      }
    }
  };
  // dS^T = P^T * (dP^T - D) of tile jt from the score registers, with
  // P^T = exp2(S^T c - LSE2); MASKED hides keys past the row's last visible
  // key (causal diagonal, ragged tail)
  auto dsoft = [&](int jt, const bool MASKED) __attribute__((always_inline)) {
    const int lim = (CAUSAL ? min(a.Sk - 1, row + shift) : a.Sk - 1) - jt * BC - 4 * h;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int kb = t >> 1, base = (t & 1) * 8;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = base + 2 * w + e;
          float p = live ? fast_exp2(fmaf(s[kb][r], a.c2, -lse_use)) : 0.f;
          if (MASKED && kb * 32 + 8 * (r / 4) + (r % 4) > lim) p = 0.f;
          ds2[e] = p * (dp[kb][r] - dsum);
        }
        dst[t][w] = pack_bf16x2(ds2[0], ds2[1]);
      }
    }
  };
  auto matrix_schedule = [&]() __attribute__((always_inline)) {
    matrix_pipeline<0, 2 * NKB * KS, NT * NDB, kDqReadAhead, true>();
  };

  // Round j (P = j % S, a literal at every call).  Matrix phase: dQ_j from
  // buffer P, then S, dP of tile j+1 from buffer (P+1) % S (unless j is the
  // last tile; this order keeps dS_j and the new scores from being live
  // together).  Vector phase: dS of tile j+1.  The leading group runs
  //   issue(j) | matrix | barrier | vector | wait | barrier
  // and the trailing group, whose phases sit one barrier later,
  //   matrix | wait | barrier | issue(j+1) | vector | barrier;
  // both groups issue round j's loads after the barrier that ends round
  // j-1's matrix phase in both (the buffers of tile j-1 are then free), and
  // before the barrier that precedes round j+1's matrix phase each wave
  // waits for its loads of tile j+2 (those of earlier rounds).
  auto round = [&](int j, const int P, const bool MASKED, const bool LEAD) __attribute__((always_inline)) {
    const bool more = !MASKED || j + 1 < nkt;  // rounds of the plain loop always have a next tile
    const bool next = more && (!MASKED || j + 1 < nneed);
    if (LEAD) issue(j, P);
    refresh_offsets();
    if (!MASKED || j < nneed) dq_update(P);
    if (next) scores((P + 1) % kDqStages);
    if (!MASKED) matrix_schedule();
    if (!LEAD) wait_vmem_at_most<kInFlight>();
    lds_sync();
    if (!LEAD) issue(j + 1, (P + 1) % kDqStages);
    if (next) {
      if (MASKED && j + 1 >= nfull)
        dsoft(j + 1, true);
      else
        dsoft(j + 1, false);
    }
    if (LEAD) wait_vmem_at_most<kInFlight>();
    lds_sync();
  };

  // the whole tile loop of one group (LEAD a literal: each group gets its
  // own straight-line code, so the compiler sees which LDS buffer every read
  // and every HBM->LDS load touches)
  auto run = [&](const bool LEAD) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t + 1 < kDqStages; ++t) issue_tile(t, t);
    wait_vmem_all();
    lds_sync();
    if (nneed > 0) {
      scores(0);
      if (LEAD) {
        if (0 >= nfull)
          dsoft(0, true);
        else
          dsoft(0, false);
      }
    }
    lds_sync();
    if (!LEAD) {
      issue(0, 0);
      if (nneed > 0) {
        if (0 >= nfull)
          dsoft(0, true);
        else
          dsoft(0, false);
      }
      lds_sync();
    }
    // rounds j < nplain produce an S_{j+1} that needs no mask for this
    // wave; they run in a loop without masking code, the others (causal
    // diagonal, ragged tail) in a second loop; unrolling by the stage count
    // keeps buffer indices literal
    const int nplain = max(min(nfull, nkt) - 1, 0);
    int j = 0;
    for (; j + kDqStages <= nplain; j += kDqStages) {
#pragma unroll
      for (int u = 0; u < kDqStages; ++u) round(j + u, u, false, LEAD);
    }
    for (; j < nkt; j += kDqStages) {
      round(j, 0, true, LEAD);
#pragma unroll
      for (int u = 1; u < kDqStages; ++u)
        if (j + u < nkt) round(j + u, u, true, LEAD);
    }
    if (LEAD) lds_sync();  // the trailing group's last barrier
    wait_vmem_all();       // the zero-filling loads past the end
  };

  if (nkt > 0) {
    if (lead)
      run(true);
    else
      run(false);
  }

  // the output address from an opaque copy of the row, so that it is not
  // computed before the tile loop and held through it
  int row_e = row;
  asm volatile("" : "+v"(row_e));
  if (row_ok) {
    uint16_t* out = a.dq + (rbase + row_e) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t w0 = pack_bf16x2(acc[db][4 * rg + 0] * a.scale, acc[db][4 * rg + 1] * a.scale);
        const uint32_t w1 = pack_bf16x2(acc[db][4 * rg + 2] * a.scale, acc[db][4 * rg + 3] * a.scale);
        *reinterpret_cast<u32x2*>(out + 32 * db + 8 * rg + 4 * h) = u32x2{w0, w1};
      }
  }
}

// ---- dK, dV
// Eight waves, two per SIMD, 32 keys each; the V rows of the workgroup's
// keys sit in LDS (the dK/dV accumulators leave no registers for them).
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvKeys = 32 * kKvWaves;  // keys per workgroup

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv(BwdKArgs a) {
  constexpr int CPR = D / 8, KS = D / 16, NDB = D / 32;
  constexpr int BR = 64;  // query rows per tile
  constexpr int TILE = BR * D;
  constexpr int ROWS_PER_INSN = 1024 / (D * 2);
  constexpr int IPW = TILE * 2 / 1024 / kKvWaves;
  static_assert(IPW >= 1, "every wave loads part of each tile");
  constexpr int VIPW = kKvKeys * D * 2 / 1024 / kKvWaves;  // V rows of the workgroup into LDS
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t d_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t d_lds1[TILE];
  __shared__ __attribute__((aligned(256))) float st_lds0[2][BR];  // LSE2, D of the tile's rows
  __shared__ __attribute__((aligned(256))) float st_lds1[2][BR];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[kKvKeys * D];  // V rows k0 ..
  typedef const __attribute__((address_space(3))) char lds_cchar;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // key block 0 (seen by every query) first; with a dynamic tail the last
  // quarter of the key blocks (seen by the fewest queries) goes last,
  // claimed at run time
  int bg, kblk;
  if (CAUSAL && a.tail_kv != nullptr) {
    const int nh = a.nkb - a.nlight_kv, nbg = a.nstatic_kv / nh;
    if ((int)blockIdx.x < a.nstatic_kv) {
      const int blk = xcd_grouped_block(blockIdx.x, a.nstatic_kv);
      bg = blk / nh;
      kblk = blk - bg * nh;
    } else {
      const int c = claim_tail_block(a.tail_kv, a.ndyn_kv);
      if (c >= nbg * a.nlight_kv) return;  // nothing left (uniform over the workgroup)
      bg = c % nbg;
      kblk = nh + c / nbg;
    }
  } else {
    const int blk = xcd_grouped_block(blockIdx.x, gridDim.x);
    bg = blk / a.nkb;
    kblk = blk - bg * a.nkb;
  }
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int G = a.H / a.Hkv;
  const int k0 = kblk * kKvKeys, wk0 = k0 + 32 * wave, shift = a.Sk - a.Sq;
  const int key = wk0 + n;  // this lane's key
  const bool key_ok = key < a.Sk;
  const uint16_t* Kg = a.k + (size_t)(b * a.Hkv + g) * a.Sk * D;
  const uint16_t* Vg = a.v + (size_t)(b * a.Hkv + g) * a.Sk * D;

  // K^T B operands of this lane's key; the V rows of the workgroup's keys
  // go to LDS (rows past Sk read as zeros) and V^T is read from there
  u32x4 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kf[ks] = key_ok ? load16(Kg + (size_t)key * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
  {
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vg + (size_t)k0 * D), (short)0, max(a.Sk - k0, 0) * D * 2, kBufferWord3);
#pragma unroll
    for (int i = 0; i < VIPW; ++i) {
      const int r = (wave * VIPW + i) * ROWS_PER_INSN + lane / CPR;
      buffer_load_lds16(vr, v_lds + (wave * VIPW + i) * 512, (r * D + (((lane % CPR) ^ b_swz<D>(r)) * 8)) * 2);
    }
  }

  // query tiles that see any of the workgroup's keys: rows i with
  // i + shift >= k0, i.e. from k0 - shift on (causal); all rows otherwise
  const int qstart = CAUSAL ? max(k0 - shift, 0) : 0;
  const int t_first = min(qstart, a.Sq) / BR;
  const int ntq = (a.Sq + BR - 1) / BR - t_first;  // tiles per query head
  const int ntot = a.Sk > k0 ? ntq * G : 0;
  // tiles that need no mask for this wave's keys: every row sees every key
  // of the wave (row >= wk0 + 31 - shift) and rows and keys are in range
  const int row_full = CAUSAL ? wk0 + 31 - shift : 0;

  uint32_t voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * ROWS_PER_INSN + lane / CPR;
    voff[i] = (r * D + (((lane % CPR) ^ b_swz<D>(r)) * 8)) * 2;
  }
  // tile t (0 .. ntot-1): query head g*G + t / ntq, rows (t_first + t % ntq) * BR ..
  auto tile_head = [&](int t) __attribute__((always_inline)) { return g * G + t / ntq; };
  auto tile_row0 = [&](int t) __attribute__((always_inline)) { return (t_first + t % ntq) * BR; };
  auto issue = [&](int t, const int BUF) __attribute__((always_inline)) {
    const int hq = tile_head(t), r0 = tile_row0(t);
    const size_t rb = (size_t)(b * a.H + hq) * a.Sq + r0;
    const int bytes = max(a.Sq - r0, 0) * D * 2;
    const __amdgpu_buffer_rsrc_t qr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + rb * D), (short)0, bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t dr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.dout + rb * D), (short)0, bytes, kBufferWord3);
    uint16_t* qd = BUF ? q_lds1 : q_lds0;
    uint16_t* dd = BUF ? d_lds1 : d_lds0;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      buffer_load_lds16(qr, qd + (wave * IPW + i) * 512, voff[i]);
      buffer_load_lds16(dr, dd + (wave * IPW + i) * 512, voff[i]);
    }
    // LSE2 and D of the 64 rows (one dword per lane; rows past Sq read 0 and
    // are masked)
    if (wave < 2) {
      const float* src = (wave == 0 ? a.lse2 : a.dsum) + rb;
      const __amdgpu_buffer_rsrc_t sr =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, max(a.Sq - r0, 0) * 4, kBufferWord3);
      float* sd = BUF ? st_lds1[wave] : st_lds0[wave];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)sd, 4, lane * 4, 0, 0, 0);
    }
  };
  constexpr int kLoads = 2 * IPW;  // per wave per tile, plus one statistics load for waves 0 and 1

  const int gq = lane >> 4, r4 = (lane >> 2) & 3, c4 = lane & 3;
  // LDS byte offsets of the operand reads, one register each: the offset of
  // step ks (row-wise reads) is a_off0 ^ 32 ks, that of head-dim block db
  // (transpose reads) tr_lo0 / tr_hi0 ^ 64 db, because the swizzle only
  // permutes chunk bits that the row term never sets.  Recomputing them at
  // each use (one XOR) instead of holding 16 offsets keeps the kernel within
  // its 256 registers: a spilled value is reloaded with a vector-memory load,
  // and waiting for that reload would also wait for the next tile's loads.
  uint32_t a_off0 = (n * D + ((h ^ b_swz<D>(n)) * 8)) * 2;
  uint32_t tr_lo0, tr_hi0;
  {
    const int dcol = 16 * (gq & 1) + 4 * c4;
    const int rl = 4 * h + r4, rh = 8 + 4 * h + r4;
    tr_lo0 = (rl * D + (((dcol >> 3) ^ b_swz<D>(rl)) * 8) + (dcol & 7)) * 2;
    tr_hi0 = (rh * D + (((dcol >> 3) ^ b_swz<D>(rh)) * 8) + (dcol & 7)) * 2;
  }
  // an opaque redefinition per block keeps the compiler from hoisting the
  // sixteen XORs back out of the loop
  auto refresh_offsets = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(a_off0), "+v"(tr_lo0), "+v"(tr_hi0));
  };

  f32x16 dk[NDB], dv[NDB];  // dK^T, dV^T (rows: head dims; column: this lane's key)
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // P and dS of one 32-row block as bf16 B operands (step st holds rows
  // 8(r/4).. for r/4 in {2st, 2st+1}); only this part differs between masked
  // and unmasked tiles
  auto scores = [&](lds_cchar* qb_, lds_cchar* db_, const float* st_l, const float* st_d, int r0, int blk32,
                    u32x4 (&pp)[2], u32x4 (&dsp)[2], const bool MASKED) __attribute__((always_inline)) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t ao = a_off0 ^ (32 * ks);
      const u32x4 qa = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(qb_ + ao + blk32 * 32 * D * 2);
      const u32x4 da = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(db_ + ao + blk32 * 32 * D * 2);
      s = mfma_32x32x16_bf16(qa, kf[ks], s);
      // row 32 wave + n of the V rows: its swizzle is that of n
      const u32x4 vt = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          (lds_cchar*)v_lds + 32 * wave * D * 2 + ao);
      dp = mfma_32x32x16_bf16(da, vt, dp);
      // two waves per SIMD hide the LDS latency; keep the operands of one
      // step live at a time
      __builtin_amdgcn_sched_barrier(0);
    }
    // register r: query row r0 + 32 blk32 + 8(r/4) + 4h + r%4; this lane's key
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int rr = 32 * blk32 + 8 * rg + 4 * h;  // first of four consecutive rows
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(st_l + rr);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(st_d + rr);
      float pv[4], dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rg + e;
        float p = fast_exp2(fmaf(s[r], a.c2, -l4[e]));
        if (MASKED) {
          const int qrow = r0 + rr + e;
          const bool vis = qrow < a.Sq && key_ok && (!CAUSAL || key <= qrow + shift);
          p = vis ? p : 0.f;
        }
        pv[e] = p;
        dsv[e] = p * (dp[r] - d4[e]);
      }
      pp[rg >> 1][(rg & 1) * 2 + 0] = pack_bf16x2(pv[0], pv[1]);
      pp[rg >> 1][(rg & 1) * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
      dsp[rg >> 1][(rg & 1) * 2 + 0] = pack_bf16x2(dsv[0], dsv[1]);
      dsp[rg >> 1][(rg & 1) * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
    }
  };

  auto tile = [&](int t, const int BUF, const bool masked) __attribute__((always_inline)) {
    lds_cchar* qb_ = (lds_cchar*)(BUF ? q_lds1 : q_lds0);
    lds_cchar* db_ = (lds_cchar*)(BUF ? d_lds1 : d_lds0);
    const float* st_l = BUF ? st_lds1[0] : st_lds0[0];
    const float* st_d = BUF ? st_lds1[1] : st_lds0[1];
    const int r0 = tile_row0(t);
#pragma unroll
    for (int blk32 = 0; blk32 < BR / 32; ++blk32) {
      refresh_offsets();
      u32x4 pp[2], dsp[2];
      if (masked)
        scores(qb_, db_, st_l, st_d, r0, blk32, pp, dsp, true);
      else
        scores(qb_, db_, st_l, st_d, r0, blk32, pp, dsp, false);
      // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-row steps
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int roff = (32 * blk32 + 16 * st) * D * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint32_t tl = tr_lo0 ^ (64 * db), th = tr_hi0 ^ (64 * db);
          const i16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(db_ + tl + roff));
          const i16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(db_ + th + roff));
          const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qb_ + tl + roff));
          const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qb_ + th + roff));
          u32x4 da, qa;
          da[0] = __builtin_bit_cast(u32x2, dlo)[0];
          da[1] = __builtin_bit_cast(u32x2, dlo)[1];
          da[2] = __builtin_bit_cast(u32x2, dhi)[0];
          da[3] = __builtin_bit_cast(u32x2, dhi)[1];
          qa[0] = __builtin_bit_cast(u32x2, qlo)[0];
          qa[1] = __builtin_bit_cast(u32x2, qlo)[1];
          qa[2] = __builtin_bit_cast(u32x2, qhi)[0];
          qa[3] = __builtin_bit_cast(u32x2, qhi)[1];
          dv[db] = mfma_32x32x16_bf16(da, pp[st], dv[db]);
          dk[db] = mfma_32x32x16_bf16(qa, dsp[st], dk[db]);
          // no scheduling fence here: the compiler issues the transpose
          // reads of later steps ahead within the registers left (2% faster
          // than one step at a time; the score steps above keep theirs, since
          // without it every read is hoisted and 195 registers spill)
        }
      }
    }
  };

  if (ntot > 0) {
    issue(0, 0);
    for (int t = 0; t < ntot; t += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tt = t + u;
        if (tt < ntot) {
          if (tt + 1 < ntot) {
            issue(tt + 1, u ^ 1);
            if (wave < 2)
              wait_vmem_at_most<kLoads + 1>();
            else
              wait_vmem_at_most<kLoads>();
          } else {
            wait_vmem_all();
          }
          lds_sync();
          const int r0 = tile_row0(tt);
          const bool full = r0 >= row_full && r0 + BR <= a.Sq && wk0 + 32 <= a.Sk;
          tile(tt, u, !full);
          lds_sync();
        }
      }
    }
  }

  wait_vmem_all();  // nothing may still be landing in LDS when the workgroup ends

  if (key_ok) {
    const size_t ko = ((size_t)(b * a.Hkv + g) * a.Sk + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c = 32 * db + 8 * rg + 4 * h;
        const uint32_t k0w = pack_bf16x2(dk[db][4 * rg + 0] * a.scale, dk[db][4 * rg + 1] * a.scale);
        const uint32_t k1w = pack_bf16x2(dk[db][4 * rg + 2] * a.scale, dk[db][4 * rg + 3] * a.scale);
        *reinterpret_cast<u32x2*>(a.dk + ko + c) = u32x2{k0w, k1w};
        const uint32_t v0w = pack_bf16x2(dv[db][4 * rg + 0], dv[db][4 * rg + 1]);
        const uint32_t v1w = pack_bf16x2(dv[db][4 * rg + 2], dv[db][4 * rg + 3]);
        *reinterpret_cast<u32x2*>(a.dv + ko + c) = u32x2{v0w, v1w};
      }
  }
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// The dynamic tails' counters (tail_pool.h): two per slot, the dQ kernel's
// at the slot's start and the dK/dV kernel's 32 entries later.
static __device__ __align__(256) unsigned bwd_tail[kTailSlots * kTailStride];
TailPoolState g_bwd_tail[kTailMaxDevices];

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& p, hipStream_t s) {
  BwdKArgs a{};  // every field zero/null until set
  const size_t rows = (size_t)p.B * p.H * p.Sq;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<const uint16_t*>(p.o);
  a.dout = static_cast<const uint16_t*>(p.dout);
  a.lse = p.lse;
  a.lse2 = static_cast<float*>(p.workspace);
  a.dsum = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + align_up(rows * 4));
  a.dq = static_cast<uint16_t*>(p.dq);
  a.dk = static_cast<uint16_t*>(p.dk);
  a.dv = static_cast<uint16_t*>(p.dv);
  a.B = p.B;
  a.H = p.H;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.nqb = (p.Sq + kDqRows - 1) / kDqRows;
  a.nkb = (p.Sk + kKvKeys - 1) / kKvKeys;
  a.c2 = p.scale * kLog2e;
  a.scale = p.scale;
  a.tail_q = a.tail_kv = nullptr;
  a.nlight_q = a.nstatic_q = a.ndyn_q = a.nlight_kv = a.nstatic_kv = a.ndyn_kv = 0;
  // dynamic tails: the lightest quarter of the blocks, where each XCD's
  // fixed range of heads still holds whole heads
  const long long nbh = (long long)p.B * p.H, nbg = (long long)p.B * p.Hkv;
  const bool tail_q = CAUSAL && a.nqb >= 32 && a.nqb % 4 == 0 && nbh % 8 == 0 && nbh * a.nqb < (1LL << 30);
  const bool tail_kv = CAUSAL && a.nkb >= 16 && a.nkb % 4 == 0 && nbg % 8 == 0 && nbg * a.nkb < (1LL << 30);
  auto run = [&](unsigned* counters) {
    size_t grid_q = (size_t)p.B * p.H * a.nqb, grid_kv = (size_t)p.B * p.Hkv * a.nkb;
    if (counters != nullptr && tail_q) {
      a.tail_q = counters;
      a.nlight_q = a.nqb / 4;
      a.nstatic_q = (int)(nbh * (a.nqb - a.nlight_q));
      const int n = (int)(nbh * a.nlight_q);
      a.ndyn_q = n + n / 4;  // a quarter more claimers than blocks: faster XCDs may take more
      grid_q = (size_t)a.nstatic_q + a.ndyn_q;
    }
    if (counters != nullptr && tail_kv) {
      a.tail_kv = counters + 32;
      a.nlight_kv = a.nkb / 4;
      a.nstatic_kv = (int)(nbg * (a.nkb - a.nlight_kv));
      const int n = (int)(nbg * a.nlight_kv);
      a.ndyn_kv = n + n / 4;
      grid_kv = (size_t)a.nstatic_kv + a.ndyn_kv;
    }
    if (rows > 0) {
      hipLaunchKernelGGL((bwd_dq<D, CAUSAL>), dim3((unsigned)grid_q), dim3(kDqThreads), 0, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if ((size_t)p.B * p.Hkv * p.Sk > 0) {
      hipLaunchKernelGGL((bwd_dkdv<D, CAUSAL>), dim3((unsigned)grid_kv), dim3(kKvThreads), 0, s, a);
      return hipGetLastError();
    }
    return hipSuccess;
  };
  if (!tail_q && !tail_kv) return run(nullptr);
  return with_tail_slot(
      g_bwd_tail, [](void** ptr) { return hipGetSymbolAddress(ptr, HIP_SYMBOL(bwd_tail)); }, s, run);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Sq) {
  const size_t rows = (size_t)B * H * Sq;
  return align_up(rows * 4) * 2;
}

hipError_t launch_bwd_bf16(const BwdArgs& p, hipStream_t s) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return p.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace attn
