// FlashAttention-style forward pass, bf16 inputs, fp32 accumulation, gfx950.
//
// Algorithm: "Warmup Guide -- Inference Optimization at Depth", Ch.4 (a Q
// block is loaded once, K/V blocks stream through on-chip memory, causal
// blocks above the diagonal are skipped and the diagonal block is masked) with
// Ch.3's online softmax (running max m, running denominator l, the
// un-normalised accumulator rescaled by exp(m_old - m_new), one division by l
// at the end).  "FlashAttention, speculative decoding, quantisation and
// parallelism", Mechanics / FlashAttention gives the same loop.
//
// Mapping onto CDNA4:
//   * one workgroup = 8 waves = 256 query rows of one (batch, head), 32 rows
//     per wave; K/V tiles of 64 keys (128 at d = 64) are shared by all eight
//     waves through LDS, two buffers each, filled by direct HBM->LDS loads
//     (buffer_load ... lds) issued one tile ahead, so no registers
//     hold staged data;
//   * every tile is handled in two phases per wave: a matrix phase (scores of
//     the next tile, S_{j+1}^T = K_{j+1} Q^T, and this tile's output update,
//     O^T += V_j^T P_j^T, 32 MFMAs) and a vector phase (P_{j+1} from
//     S_{j+1}: exponentials, sums, bf16 packing).  The waves form two groups
//     of four, one wave of each group per SIMD, and the second group runs one
//     phase behind the first: workgroup barriers separate the phases, so on
//     every SIMD one wave keeps the matrix core busy while the other does its
//     vector work, and the LDS reads of a tile come from one group at a time;
//   * scores are computed transposed on the 32x32x16 bf16 MFMA, so each lane
//     holds one query column and 32 of the tile's 64 keys; the output is
//     accumulated transposed too: P^T is the B operand straight from the score
//     registers (rounded to bf16), the V^T A operand comes from row-major V
//     with the LDS transpose read (ds_read_b64_tr_b16), and the rescale
//     factor of a query is a per-lane scalar;
//   * the softmax works in base 2 with scale*log2(e) folded into one FMA,
//     against a per-row reference value m_ref instead of the exact running
//     max: the final O/l and LSE do not depend on the reference (Ch.3's
//     rescaling identity), only overflow does.  A tile is exponentiated
//     against the current m_ref without computing its max; only when a
//     lane's tile sum exceeds 2^32 (some score is > m_ref + 27 in log2
//     units) or a row has no reference yet does the wave take a slow path
//     that computes the tile max, raises m_ref, rescales the accumulator and
//     exponentiates again.  Probabilities stay below 2^32, far from fp32 and
//     bf16 overflow, and most tiles need neither a max nor a rescale;
//   * with 32 or more query blocks per head (a multiple of 8, over a
//     multiple of 16 heads), the lightest quarter of every head's blocks is
//     handed out at run time (tail_pool.h): each XCD gets a fixed eighth
//     of the heavier blocks, and the workgroups launched after those claim
//     the light blocks from a counter, so XCDs that run faster (their clocks
//     differ by up to 7% under load) take more of them and all finish
//     together; which workgroup computes a block does not change its
//     arithmetic, so the output is the same bit for bit;
//   * the output of a wave's 32 rows is staged in LDS (the tile buffers are
//     free by then) and written back as whole rows, so every store
//     instruction covers 1 KB of consecutive memory rather than 8 bytes of
//     32 rows;
//   * two denominators are kept: the fp32 sum of the probabilities (for LSE)
//     and the sum of the same probabilities rounded to bf16, i.e. of exactly
//     the weights the P.V product used (one v_dot2 per pair).  O is divided by
//     the latter, so O is a convex combination of V rows whose weights sum to
//     one; the bf16 rounding of a dominant weight then cancels instead of
//     showing up as an error of |v| * 2^-9.
#include "device_common.h"
#include "launch.h"
#include "tail_pool.h"

namespace attn {
namespace {

// Two LDS buffers per K/V tile stream; each LDS operand read of a matrix
// phase is issued kReadAhead MFMAs before the MFMA that consumes it.  (A
// third buffer, deeper read-ahead, wave priorities and matrix-core row sums
// were each measured and gave nothing.)
constexpr int kStages = 2;
constexpr int kReadAhead = 4;
constexpr int kWaves = 8;               // two groups of four, one wave of each per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;        // query rows per workgroup
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kTileSumLimit = 0x1p32f;  // fast-path bound on a lane's tile sum

struct FwdKernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int H, Hkv, Sq, Sk;
  int nqb;   // query blocks per (batch, head)
  float c2;  // scale * log2(e)
  // dynamic tail (null pool: every workgroup has a fixed block): the first
  // nstatic workgroups take the heavier nqb - nlight blocks of every head in
  // a fixed order; the ndyn workgroups after them claim the nlight lightest
  // blocks of every head, heaviest first, from the counter *pool
  unsigned* pool;
  int nlight, nstatic, ndyn;
};

// Workgroup barrier for the phase hand-over: this wave's LDS reads have
// completed and no instruction is scheduled across it (a matrix
// instruction that slipped into the vector phase would compete with the
// other wave's), but HBM->LDS loads still in flight are not waited for (a
// fence would wait for them too: they write LDS); where a tile must have
// landed, vmcnt is waited for explicitly first.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdKernelArgs a) {
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int KS = D / 16;   // MFMA steps over the head dim for S^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T (head dim)
  // Keys per K/V tile: 64 at d = 128; 128 at d = 64, where a tile's scores
  // and probabilities still fit the registers and each phase between two
  // barriers carries twice the work (3.6% faster at S = 32768; at d = 128
  // the larger tile spills)
  constexpr int kBc = D == 64 ? 128 : 64;
  constexpr int kNkb = kBc / 32;  // 32-key blocks per tile
  constexpr int kNt = kBc / 16;   // 16-key MFMA steps per tile
  constexpr int TILE = kBc * D;  // elements per K or V tile
  constexpr int ROWS_PER_INSN = 1024 / (D * 2);  // rows one wave-wide 1 KB load covers
  constexpr int INSN_PER_WAVE = TILE * 2 / 1024 / kWaves;
  static_assert(INSN_PER_WAVE >= 1, "every wave loads part of each tile");

  // two buffers each for K and V tiles, one LDS object per buffer, so the
  // compiler can prove that loads into one buffer never alias reads of
  // another
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];
  auto kbuf = [&](const int I) __attribute__((always_inline)) { return I == 0 ? k_lds0 : k_lds1; };
  auto vbuf = [&](const int I) __attribute__((always_inline)) { return I == 0 ? v_lds0 : v_lds1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int n = lane & 31;  // query column within the wave's 32 rows
  const int h = lane >> 5;  // wave half
  // Waves w and w + 4 share a SIMD; w < 4 leads, w >= 4 trails by one phase.
  // A SIMD's two waves take row blocks s and 7 - s: on the causal diagonal,
  // where a wave skips the tiles none of its rows see, every SIMD then keeps
  // some of the remaining work (adjacent blocks on one SIMD left the SIMD
  // with the last rows to set the pace; 0.8-1.1% at S = 32768, unchanged at
  // S = 8192 and 2048)
  const bool lead = wave < 4;
  const int rb = lead ? (wave & 3) : 7 - (wave & 3);

  // Workgroup order (XCDs, shader engines and the causal tail): with fewer
  // query blocks per head than an XCD has CUs (short sequences) all of an
  // XCD's heads are interleaved, heaviest blocks first, which balances the
  // causal tail and gives every four consecutive ids the same cost; with a
  // pool, causal_block_order's head pairs over the heavier blocks, then the
  // light blocks claimed from the pool (all heads' blocks of one size next
  // to each other, heaviest first); otherwise the head pairs over all blocks.
  int bh, qblk;
  {
    constexpr int kXcds = 8, kCusPerXcd = 32;
    if (CAUSAL && a.pool != nullptr) {
      const int nh = a.nqb - a.nlight;
      const int nbh = a.nstatic / nh;
      if ((int)blockIdx.x < a.nstatic) {
        const int blk = causal_block_order(blockIdx.x, a.nstatic, nh, true);
        bh = blk / nh;
        qblk = a.nqb - 1 - (blk - bh * nh);
      } else {
        const int c = claim_tail_block(a.pool, a.ndyn);
        if (c >= nbh * a.nlight) return;  // the pool is empty (uniform over the workgroup)
        bh = c % nbh;
        qblk = a.nlight - 1 - c / nbh;
      }
    } else if (CAUSAL && a.nqb < kCusPerXcd && (gridDim.x / a.nqb) % kXcds == 0) {
      const int nbh = gridDim.x / a.nqb;
      const int x = blockIdx.x % kXcds, i = blockIdx.x / kXcds, hx = nbh / kXcds;
      bh = x * hx + i % hx;
      qblk = a.nqb - 1 - i / hx;
    } else {
      const int blk = causal_block_order(blockIdx.x, gridDim.x, a.nqb, CAUSAL);
      bh = blk / a.nqb;
      qblk = blk - bh * a.nqb;
      if (CAUSAL) qblk = a.nqb - 1 - qblk;  // heaviest query blocks of a head first
    }
  }
  const int b = bh / a.H;
  const int hq = bh - b * a.H;
  const int g = hq / (a.H / a.Hkv);

  const int q0 = qblk * kBr;
  const int wq0 = q0 + 32 * rb;   // first query row of this wave
  const int shift = a.Sk - a.Sq;  // bottom-right causal alignment

  const uint16_t* Q = a.q + (size_t)(b * a.H + hq) * a.Sq * D;
  const uint16_t* K = uniform_ptr(a.k + (size_t)(b * a.Hkv + g) * a.Sk * D);
  const uint16_t* V = uniform_ptr(a.v + (size_t)(b * a.Hkv + g) * a.Sk * D);

  // tiles the workgroup visits (every wave runs all of them: the phases are
  // workgroup-wide); tiles [0, nfull) need no mask for this wave's rows
  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, min(q0 + kBr, a.Sq) + shift);
  kend = max(kend, 0);
  const int nkt = (kend + kBc - 1) / kBc;
  int nfull = a.Sk / kBc;
  if (CAUSAL) nfull = min(nfull, max(wq0 + shift + 1, 0) / kBc);
  // tiles [0, nneed) hold keys some row of this wave sees; the workgroup's
  // later tiles (causal diagonal) are hidden from all of its rows, so the
  // wave skips their matrix and vector work (it still takes part in the
  // loads and barriers)
  int nneed = nkt;
  if (CAUSAL) nneed = min(nkt, (max(min(wq0 + 31, a.Sq - 1) + shift + 1, 0) + kBc - 1) / kBc);

  // ---- direct HBM -> LDS tile loads.  Wave-wide instruction i of this wave
  // fills LDS bytes [1024*(wave*INSN_PER_WAVE+i), +1024); lane l's 16 bytes
  // land at offset 16*l, i.e. tile row r = first row + l / CPR, chunk position
  // l % CPR, which holds global chunk (position ^ swizzle(r)).  The buffer
  // descriptor of a tile starts at its first key and ends at key Sk, so rows
  // past Sk read as zeros.
  uint32_t k_voff[INSN_PER_WAVE], v_voff[INSN_PER_WAVE];
#pragma unroll
  for (int i = 0; i < INSN_PER_WAVE; ++i) {
    const int row = (wave * INSN_PER_WAVE + i) * ROWS_PER_INSN + lane / CPR;
    const int pos = lane % CPR;
    k_voff[i] = (row * D + ((pos ^ k_swz<D>(row)) * 8)) * 2;
    v_voff[i] = (row * D + ((pos ^ v_swz<D>(row)) * 8)) * 2;
  }
  // Q^T as the B operand: column n = query wq0 + n, eight head-dim values per
  // step.
  u32x4 qf[KS];
  {
    const int qrow = wq0 + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (qrow < a.Sq) ? load16(Q + (size_t)qrow * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max, base-2 domain (scaled logits * log2 e)
  float l_run = 0.f;        // running denominator, this lane's keys only
  float l_rnd = 0.f;        // same, of the bf16-rounded probabilities

  // Per-lane LDS byte offsets, fixed for the whole kernel (buffer and tile
  // offsets are immediates).  K A-operand of block kb, step ks: row
  // kb*32 + n, chunk (2ks + h) ^ swizzle(row); the swizzle of row kb*32 + n
  // is that of n.  V transpose read for d-block db, step t, half e: row
  // 16t + 8e + 4h + r4, column chunk (32db + 16(gq&1) + 4c4) / 8, swizzled by
  // the row's (r4-only) swizzle.
  const int gq = lane >> 4, r4 = (lane >> 2) & 3, c4 = lane & 3;
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = (n * D + (((ks * 2 + h) ^ k_swz<D>(n)) * 8)) * 2;
  uint32_t v_off[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dcol = 32 * db + 16 * (gq & 1) + 4 * c4;
    const int row = 4 * h + r4;
    v_off[db] = (row * D + (((dcol >> 3) ^ v_swz<D>(row)) * 8) + (dcol & 7)) * 2;
  }
  typedef const __attribute__((address_space(3))) char lds_cchar;

  f32x16 s[kNkb];  // scores of the next tile (fp32)
  u32x4 pt[kNt];   // probabilities of the current tile, bf16, as MFMA B operands

  // S^T of a tile from kbuf[KBUF]; the two 32-key blocks alternate so that
  // consecutive MFMAs never depend on each other
  auto scores = [&](const int KBUF) __attribute__((always_inline)) {
    lds_cchar* k_base = (lds_cchar*)kbuf(KBUF);
#pragma unroll
    for (int kb = 0; kb < kNkb; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb) {
        const u32x4 kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            k_base + k_off[ks] + kb * 32 * D * 2);
        s[kb] = mfma_32x32x16_bf16(kf, qf[ks], s[kb]);
      }
    }
  };

  // hide keys past a row's last visible key (causal diagonal, ragged tail)
  auto mask = [&](int j0) __attribute__((always_inline)) {
    const int qrow = wq0 + n;
    const int lim = (CAUSAL ? min(a.Sk - 1, qrow + shift) : a.Sk - 1) - j0 - 4 * h;
#pragma unroll
    for (int kb = 0; kb < kNkb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kb * 32 + 8 * (r / 4) + (r % 4) > lim) s[kb][r] = -INFINITY;
      }
  };

  // slow path: raise the reference to the tile max where it exceeds it by
  // more than the slack (or where there was none), rescaling what was
  // accumulated
  auto raise_ref = [&]() __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kNkb; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_halves(mx) * a.c2;
    const bool raise = mx > m_ref + kRescaleSlack || (m_ref == -INFINITY && mx > -INFINITY);
    const float alpha = raise ? fast_exp2(m_ref - mx) : 1.f;  // 0 when m_ref = -inf
    m_ref = raise ? mx : m_ref;
    l_run *= alpha;
    l_rnd *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
  };

  // One pass over the score tile (left intact): probabilities against the
  // reference, their fp32 sum ts, the bf16-rounded values packed as the B
  // operands of the P.V product, and the sum tr of the rounded values.
  // Partial sums run in several chains so the adds do not serialise.
  auto softmax = [&](float& ts, float& tr) __attribute__((always_inline)) {
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;  // nothing visible yet
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
    float r2[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
      const int kb = t >> 1, base = (t & 1) * 8;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = fast_exp2(fmaf(s[kb][base + 2 * w], a.c2, -m_use));
        const float p1 = fast_exp2(fmaf(s[kb][base + 2 * w + 1], a.c2, -m_use));
        a4[(2 * w) & 3] += p0;
        a4[(2 * w + 1) & 3] += p1;
        pt[t][w] = pack_bf16x2(p0, p1);
        r2[w & 1] = sum_bf16x2(pt[t][w], r2[w & 1]);
      }
    }
    ts = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    tr = r2[0] + r2[1];
  };
  // P of the score tile, with the slow path when the fast one may overflow
  // or a row has no reference yet; then the tile's sums join the running ones
  auto probabilities = [&]() __attribute__((always_inline)) {
    float ts, tr;
    softmax(ts, tr);
    const bool bad = !(ts <= kTileSumLimit) || m_ref == -INFINITY;
    if (__builtin_expect(__any(bad), 0)) {
      asm volatile("");
      raise_ref();
      softmax(ts, tr);
    }
    l_run += ts;
    l_rnd += tr;
  };

  // O^T += V^T P^T over the tile's 16-key steps
  auto accumulate = [&](const int VBUF) __attribute__((always_inline)) {
    lds_cchar* v_base = (lds_cchar*)vbuf(VBUF);
#pragma unroll
    for (int t = 0; t < kNt; ++t) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // items 0..3: keys 16t + 4h + r4; items 4..7: keys 16t + 8 + 4h + r4
        lds_cchar* vb = v_base + v_off[db] + 16 * t * D * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vb);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + 8 * D * 2));
        u32x4 vf;
        vf[0] = __builtin_bit_cast(u32x2, lo)[0];
        vf[1] = __builtin_bit_cast(u32x2, lo)[1];
        vf[2] = __builtin_bit_cast(u32x2, hi)[0];
        vf[3] = __builtin_bit_cast(u32x2, hi)[1];
        acc_o[db] = mfma_32x32x16_bf16(vf, pt[t], acc_o[db]);
      }
    }
  };

  // this wave's share of K tile t into kbuf[BUF] / V tile t into vbuf[BUF];
  // a tile at or past Sk has an empty descriptor (every lane reads zeros),
  // so a round always issues the same number of loads
  auto issue_k = [&](int t, const int BUF) __attribute__((always_inline)) {
    const int j0 = t * kBc;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(K + (size_t)j0 * D), (short)0, max(a.Sk - j0, 0) * D * 2, kBufferWord3);
    uint16_t* kd = kbuf(BUF);
#pragma unroll
    for (int i = 0; i < INSN_PER_WAVE; ++i) buffer_load_lds16(kr, kd + (wave * INSN_PER_WAVE + i) * 512, k_voff[i]);
  };
  auto issue_v = [&](int t, const int BUF) __attribute__((always_inline)) {
    const int j0 = t * kBc;
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(V + (size_t)j0 * D), (short)0, max(a.Sk - j0, 0) * D * 2, kBufferWord3);
    uint16_t* vd = vbuf(BUF);
#pragma unroll
    for (int i = 0; i < INSN_PER_WAVE; ++i) buffer_load_lds16(vr, vd + (wave * INSN_PER_WAVE + i) * 512, v_voff[i]);
  };
  // Loads of round j (S = kStages): K_{j+S} into kbuf[j % S] (K_j's, read
  // for the last time in round j-1) and V_{j+S-1} into vbuf[(j-1) % S]
  // (V_{j-1}'s, likewise); issued once both groups have finished round
  // j-1's matrix phase, needed by round j+S-1's.  Each round issues kLoads
  // instructions per wave; the waits leave the latest (S-2) rounds' loads in
  // flight, so each load has 2(S-1) phases to land.
  constexpr int kLoads = 2 * INSN_PER_WAVE;
  constexpr int kInFlight = (kStages - 2) * kLoads;
  auto issue = [&](int j, const int P) __attribute__((always_inline)) {
    issue_k(j + kStages, P);
    issue_v(j + kStages - 1, (P + kStages - 1) % kStages);
  };

  // Round j (P = j % S, a literal at every call).  Matrix phase: S_{j+1}
  // from kbuf[(P+1) % S] (unless j is the last tile) and O += V_j^T P_j
  // from vbuf[P].  Vector phase: P_{j+1} from S_{j+1}, masked first if
  // MASKED (a literal) and the tile needs it.  The leading group (LEAD) runs
  //   issue(j) | matrix | barrier | vector | wait | barrier
  // and the trailing group, whose phases sit one barrier later,
  //   matrix | wait | barrier | issue(j+1) | vector | barrier,
  // where each wait leaves only the loads of the round's own issue in
  // flight, so every load has landed, in every wave, by the barrier that
  // precedes the first matrix phase reading it.
  // Order of the matrix phase: each LDS operand read is issued kReadAhead
  // MFMAs before the MFMA that consumes it, so LDS latency hides behind
  // matrix work.
  auto matrix_schedule = [&]() __attribute__((always_inline)) {
    matrix_pipeline<0, kNkb * KS, kNt * NDB, kReadAhead>();
  };

  auto round = [&](int j, const int P, const bool MASKED, const bool LEAD) __attribute__((always_inline)) {
    const bool more = !MASKED || j + 1 < nkt;  // rounds of the plain loop always have a next tile
    if (LEAD) issue(j, P);
    // unmasked rounds always need both tiles (j + 1 < nfull <= nneed)
    if (more && (!MASKED || j + 1 < nneed)) scores((P + 1) % kStages);
    if (!MASKED || j < nneed) accumulate(P);
    if (!MASKED) matrix_schedule();
    if (!LEAD) wait_vmem_at_most<kInFlight>();
    lds_barrier();
    if (!LEAD) issue(j + 1, (P + 1) % kStages);
    if (more && (!MASKED || j + 1 < nneed)) {
      if (MASKED && j + 1 >= nfull) mask((j + 1) * kBc);
      probabilities();
    }
    if (LEAD) wait_vmem_at_most<kInFlight>();
    lds_barrier();
  };

  // The whole tile loop of one group (LEAD a literal: each group gets its
  // own straight-line code, so the compiler can see which LDS buffer every
  // read and every HBM->LDS load touches).
  auto run = [&](const bool LEAD) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kStages; ++t) issue_k(t, t);
#pragma unroll
    for (int t = 0; t + 1 < kStages; ++t) issue_v(t, t);
    wait_vmem_all();
    lds_barrier();
    if (nneed > 0) {
      scores(0);
      if (0 >= nfull) mask(0);
      if (LEAD) probabilities();
    }
    lds_barrier();
    if (!LEAD) {
      issue(0, 0);
      if (nneed > 0) probabilities();
      lds_barrier();
    }
    // Rounds j < nplain produce an S_{j+1} that needs no mask for this
    // wave; they run in a loop without masking code, the few others (causal
    // diagonal, ragged tail) in a second loop.  Unrolling by the stage
    // count keeps buffer indices literal.
    const int nplain = max(min(nfull, nkt) - 1, 0);
    int j = 0;
    for (; j + kStages <= nplain; j += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) round(j + u, u, false, LEAD);
    }
    for (; j < nkt; j += kStages) {
      round(j, 0, true, LEAD);
#pragma unroll
      for (int u = 1; u < kStages; ++u)
        if (j + u < nkt) round(j + u, u, true, LEAD);
    }
    if (LEAD) lds_barrier();  // the trailing group's last barrier
    wait_vmem_all();          // the zero-filling loads past the end
    lds_barrier();            // every wave's loads have landed: the tile buffers are free
  };

  if (nkt > 0) {
    if (lead)
      run(true);
    else
      run(false);
  }

  // ---- epilogue: one normalised write per row.  The wave stages its 32
  // rows of O (bf16) in its own 32*D-element part of the free tile buffers,
  // 16-byte chunks XOR-swizzled by row, then writes them back as whole rows:
  // each store instruction covers 1 KB of consecutive output.
  {
    const int qrow = wq0 + n;
    const float lt = sum_halves(l_run);
    const float lr = sum_halves(l_rnd);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    uint16_t* stage = (wave >> 1) == 0 ? k_lds0 : (wave >> 1) == 1 ? k_lds1 : (wave >> 1) == 2 ? v_lds0 : v_lds1;
    stage += (wave & 1) * 32 * D;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        // registers 4*rg .. 4*rg+3: head dims 32*db + 8*rg + 4*h + 0..3 of row n
        const uint32_t w0 = pack_bf16x2(acc_o[db][4 * rg + 0] * inv, acc_o[db][4 * rg + 1] * inv);
        const uint32_t w1 = pack_bf16x2(acc_o[db][4 * rg + 2] * inv, acc_o[db][4 * rg + 3] * inv);
        const int chunk = (4 * db + rg) ^ (n & (CPR - 1));
        *reinterpret_cast<lds_u32x2*>((__attribute__((address_space(3))) char*)stage + n * D * 2 + chunk * 16 + 8 * h) =
            u32x2{w0, w1};
      }
    if (a.lse != nullptr && h == 0 && qrow < a.Sq)
      a.lse[(size_t)(b * a.H + hq) * a.Sq + qrow] = lt > 0.f ? (m_ref + fast_log2(lt)) * kLn2 : -INFINITY;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's staging writes are done
    uint16_t* O = a.o + ((size_t)(b * a.H + hq) * a.Sq + wq0) * D;
    constexpr int ROWS_PER_STORE = 1024 / (D * 2);
#pragma unroll
    for (int i = 0; i < 32 / ROWS_PER_STORE; ++i) {
      const int r = i * ROWS_PER_STORE + lane / CPR, c = lane % CPR;
      const u32x4 val = *reinterpret_cast<const lds_u32x4*>(
          (const __attribute__((address_space(3))) char*)stage + r * D * 2 + ((c ^ (r & (CPR - 1))) * 16));
      if (wq0 + r < a.Sq) store16(O + (size_t)r * D + c * 8, val);
    }
  }
}

// The dynamic tail's counters (tail_pool.h): one per slot.
static __device__ __align__(256) unsigned fwd_tail[kTailSlots * kTailStride];
TailPoolState g_fwd_tail[kTailMaxDevices];

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& p, hipStream_t s) {
  FwdKernelArgs a{};  // every field zero/null until set
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.H = p.H;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.nqb = (p.Sq + kBr - 1) / kBr;
  a.c2 = p.scale * kLog2e;
  const long long nbh = (long long)p.B * p.H;
  const long long grid = nbh * a.nqb;
  a.pool = nullptr;
  a.nlight = a.nstatic = a.ndyn = 0;
  // the dynamic tail (the lightest quarter of every head's blocks) needs the
  // head-pair order over the heavier blocks: heads in pairs on every XCD and
  // an even number of heavier blocks
  if (!(CAUSAL && a.nqb >= 32 && a.nqb % 8 == 0 && nbh % 16 == 0 && grid < (1LL << 30))) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const int nlight = a.nqb / 4;
  const int npool = (int)(nbh * nlight);
  return with_tail_slot(
      g_fwd_tail, [](void** p) { return hipGetSymbolAddress(p, HIP_SYMBOL(fwd_tail)); }, s,
      [&](unsigned* counters) {
        long long g = grid;
        if (counters != nullptr) {
          a.pool = counters;
          a.nlight = nlight;
          a.nstatic = (int)(nbh * (a.nqb - nlight));
          a.ndyn = npool + npool / 4;  // a quarter more claimers than blocks: faster XCDs may take more
          g = a.nstatic + a.ndyn;
        }
        hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)g), dim3(kThreads), 0, s, a);
        return hipGetLastError();
      });
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& p, hipStream_t s) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return p.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace attn
