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
//   * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//     owns 32 rows; K/V tiles of 64 keys are shared by the four waves through
//     LDS, double-buffered and filled by direct HBM->LDS loads
//     (global_load_lds_dwordx4), so the next tile streams in while the
//     current one is consumed and no registers hold staged data;
//   * scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 MFMA,
//     so each lane holds one query column and 32 of the tile's 64 keys: the
//     row max is an in-lane reduction plus one exchange with the other wave
//     half, and the row sum stays per lane until the end;
//   * the output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     B operand straight from the score registers (rounded to bf16), the V^T
//     A operand comes from row-major V with the LDS transpose read
//     (ds_read_b64_tr_b16), and the rescale factor of a query is a per-lane
//     scalar;
//   * the softmax works in base 2 with scale*log2(e) folded into one FMA.
//     The reference max of a row is only raised when the tile max exceeds it
//     by more than 2^8 (the exponents then stay <= 8, far from overflow); the
//     final O/l and LSE are unchanged by the choice of reference, as in Ch.3's
//     rescaling identity, and most tiles skip the accumulator rescale;
//   * two denominators are kept: the fp32 sum of the probabilities (for LSE)
//     and the sum of the same probabilities rounded to bf16, i.e. of exactly
//     the weights the P.V product used (one v_dot2 per pair).  O is divided by
//     the latter, so O is a convex combination of V rows whose weights sum to
//     one; the bf16 rounding of a dominant weight then cancels instead of
//     showing up as an error of |v| * 2^-9.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

// Tile shape (build-time constants): waves per workgroup (32 query rows
// each), keys per K/V tile, and whether matrix-core clusters raise the wave's
// issue priority so they are not starved by the other wave's softmax.
#ifndef ATTN_FWD_WAVES
#define ATTN_FWD_WAVES 4
#endif
#ifndef ATTN_FWD_BC
#define ATTN_FWD_BC 64
#endif
#ifndef ATTN_FWD_PRIO
#define ATTN_FWD_PRIO 1
#endif
#ifndef ATTN_FWD_SCHED
#define ATTN_FWD_SCHED 0
#endif
#ifndef ATTN_FWD_QB
#define ATTN_FWD_QB 1
#endif
constexpr int kWaves = ATTN_FWD_WAVES;
constexpr int kQb = ATTN_FWD_QB;  // 32-query blocks per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kQb * kWaves;  // query rows per workgroup
constexpr int kBc = ATTN_FWD_BC;  // keys per K/V tile
constexpr int kNkb = kBc / 32;    // 32-key blocks per tile
constexpr int kMinBlocks = (kQb == 1 ? 8 : 4) / kWaves;  // waves per SIMD: 2 (one query block) or 1
constexpr float kRescaleSlack = 8.0f;  // log2 units

struct FwdKernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int H, Hkv, Sq, Sk;
  int nqb;   // query blocks per (batch, head)
  float c2;  // scale * log2(e)
};

__device__ __forceinline__ void prio_high() {
  if (ATTN_FWD_PRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ __forceinline__ void prio_low() {
  if (ATTN_FWD_PRIO) __builtin_amdgcn_s_setprio(0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, kMinBlocks) fwd_bf16_kernel(FwdKernelArgs a) {
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int KS = D / 16;   // MFMA steps over the head dim for S^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T (head dim)
  constexpr int QB = kQb;      // 32-query column blocks per wave
  constexpr int TILE = kBc * D;  // elements per K or V tile
  constexpr int ROWS_PER_INSN = 1024 / (D * 2);  // rows one wave-wide 1 KB load covers
  constexpr int INSN_PER_WAVE = TILE * 2 / 1024 / kWaves;

  // one LDS object per buffer, so the compiler can prove that loads into one
  // buffer never alias reads of the other
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int n = lane & 31;  // query column within a 32-row block
  const int h = lane >> 5;  // wave half

  const int blk = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = blk / a.nqb;
  int qblk = blk - bh * a.nqb;
  if (CAUSAL) qblk = a.nqb - 1 - qblk;  // heaviest query blocks of a head first
  const int b = bh / a.H;
  const int hq = bh - b * a.H;
  const int g = hq / (a.H / a.Hkv);

  const int q0 = qblk * kBr;
  const int wq0 = q0 + wave * 32 * QB;  // first query row of this wave
  const int shift = a.Sk - a.Sq;        // bottom-right causal alignment

  const uint16_t* Q = a.q + (size_t)(b * a.H + hq) * a.Sq * D;
  const uint16_t* K = a.k + (size_t)(b * a.Hkv + g) * a.Sk * D;
  const uint16_t* V = a.v + (size_t)(b * a.Hkv + g) * a.Sk * D;

  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, min(q0 + kBr, a.Sq) + shift);
  kend = max(kend, 0);
  const int nkt = (kend + kBc - 1) / kBc;

  // ---- direct HBM -> LDS tile loads (buffer_load ... lds).  Wave-wide
  // instruction i of this wave fills LDS bytes [1024*(wave*INSN_PER_WAVE+i),
  // +1024); lane l's 16 bytes land at offset 16*l, i.e. tile row
  // r = first row + l / CPR, chunk position l % CPR, which holds global chunk
  // (position ^ swizzle(r)).  The buffer descriptor of a tile starts at its
  // first key and ends at key Sk, so rows past Sk read as zeros.
  uint32_t k_voff[INSN_PER_WAVE], v_voff[INSN_PER_WAVE];
#pragma unroll
  for (int i = 0; i < INSN_PER_WAVE; ++i) {
    const int row = (wave * INSN_PER_WAVE + i) * ROWS_PER_INSN + lane / CPR;
    const int pos = lane % CPR;
    k_voff[i] = (row * D + ((pos ^ k_swz<D>(row)) * 8)) * 2;
    v_voff[i] = (row * D + ((pos ^ v_swz<D>(row)) * 8)) * 2;
  }
  // Q^T as the B operand: column n of block qb = query wq0 + 32qb + n, eight
  // head-dim values per step.
  u32x4 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = wq0 + 32 * qb + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = (qrow < a.Sq) ? load16(Q + (size_t)qrow * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 acc_o[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[qb][db] = f32x16{};
  float m_ref[QB], l_run[QB], l_rnd[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = -INFINITY;  // reference max, base-2 domain (scaled logits * log2 e)
    l_run[qb] = 0.f;        // running denominator, this lane's keys only
    l_rnd[qb] = 0.f;        // same, of the bf16-rounded probabilities
  }

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

  // Tiles [0, nfull) need no mask for any row of this workgroup; the rest
  // (causal diagonal, ragged tail) are masked.
  int nfull = a.Sk / kBc;
  if (CAUSAL) nfull = min(nfull, max(q0 + shift + 1, 0) / kBc);

  // Software pipeline.  Iteration j consumes K_{j+1} (scores of the next
  // tile) and V_j (output of this tile), so the matrix cores compute
  // S_{j+1} = K_{j+1} Q^T while the vector ALUs turn S_j into P_j, then
  // O += V_j^T P_j.  Score registers and LDS buffers alternate with the tile
  // parity: tile t's scores live in sreg[t & 1], its K in kbuf[t & 1], its V
  // in vbuf[t & 1].
  f32x16 sreg[2][QB][kNkb];

  auto scores = [&](f32x16 (&s)[QB][kNkb], const int KBUF) {
    lds_cchar* k_base = (lds_cchar*)(KBUF ? k_lds1 : k_lds0);
#pragma unroll
    for (int kb = 0; kb < kNkb; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            k_base + k_off[ks] + kb * 32 * D * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_32x32x16_bf16(kf, qf[qb][ks], s[qb][kb]);
      }
    }
  };

  // hide keys past a row's last visible key (causal diagonal, ragged tail)
  auto mask = [&](f32x16 (&s)[QB][kNkb], int j0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = wq0 + 32 * qb + n;
      const int lim = (CAUSAL ? min(a.Sk - 1, qrow + shift) : a.Sk - 1) - j0 - 4 * h;
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (kb * 32 + 8 * (r / 4) + (r % 4) > lim) s[qb][kb][r] = -INFINITY;
        }
    }
  };

  // row max of a score tile (base-2 domain)
  auto rowmax = [&](f32x16 (&s)[QB][kNkb], float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mx[qb] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx[qb] = fmaxf(mx[qb], s[qb][kb][r]);
      mx[qb] = max_halves(mx[qb]) * a.c2;
    }
  };

  // raise the reference max where the tile max exceeds it by more than the
  // slack (rare: a real branch around the accumulator rescale)
  auto raise_ref = [&](const float (&mx)[QB]) {
    bool raise_any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) raise_any |= mx[qb] > m_ref[qb] + kRescaleSlack;
    if (__builtin_expect(__any(raise_any), 0)) {
      asm volatile("");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool raise = mx[qb] > m_ref[qb] + kRescaleSlack;
        const float alpha = raise ? fast_exp2(m_ref[qb] - mx[qb]) : 1.f;  // 0 when m_ref = -inf
        m_ref[qb] = raise ? mx[qb] : m_ref[qb];
        l_run[qb] *= alpha;
        l_rnd[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[qb][db][r] *= alpha;
      }
    }
  };

  constexpr int NT = kBc / 16;  // 16-key MFMA steps per tile
  // probabilities in place (fp32), rounded to bf16 and packed as the B
  // operands of the P.V product; the sum of the rounded values
  auto exponentiate = [&](f32x16 (&s)[QB][kNkb], u32x4 (&pt)[QB][NT]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_use = (m_ref[qb] == -INFINITY) ? 0.f : m_ref[qb];  // nothing visible yet
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = fast_exp2(fmaf(s[qb][kb][r], a.c2, -m_use));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int kb = t >> 1, base = (t & 1) * 8;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pt[qb][t][w] = pack_bf16x2(s[qb][kb][base + 2 * w], s[qb][kb][base + 2 * w + 1]);
          l_rnd[qb] = sum_bf16x2(pt[qb][t][w], l_rnd[qb]);
        }
      }
    }
  };
  // fp32 sum of the (unrounded) probabilities
  auto sum_p = [&](f32x16 (&s)[QB][kNkb]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) l_run[qb] += s[qb][kb][r];
  };

  // O^T += V^T P^T over the tile's 16-key steps; each V read feeds all QB blocks
  auto accumulate = [&](const u32x4 (&pt)[QB][NT], const int VBUF) {
    lds_cchar* v_base = (lds_cchar*)(VBUF ? v_lds1 : v_lds0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
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
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc_o[qb][db] = mfma_32x32x16_bf16(vf, pt[qb][t], acc_o[qb][db]);
      }
    }
  };

  // DMA of K tile t into kbuf[t & 1] / V tile t into vbuf[t & 1]
  auto issue_k = [&](int t, const int BUF) {
    const int j0 = t * kBc;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(K + (size_t)j0 * D), (short)0, (a.Sk - j0) * D * 2, kBufferWord3);
    uint16_t* kd = BUF ? k_lds1 : k_lds0;
#pragma unroll
    for (int i = 0; i < INSN_PER_WAVE; ++i) buffer_load_lds16(kr, kd + (wave * INSN_PER_WAVE + i) * 512, k_voff[i]);
  };
  auto issue_v = [&](int t, const int BUF) {
    const int j0 = t * kBc;
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(V + (size_t)j0 * D), (short)0, (a.Sk - j0) * D * 2, kBufferWord3);
    uint16_t* vd = BUF ? v_lds1 : v_lds0;
#pragma unroll
    for (int i = 0; i < INSN_PER_WAVE; ++i) buffer_load_lds16(vr, vd + (wave * INSN_PER_WAVE + i) * 512, v_voff[i]);
  };

  // Scheduling hints: interleave each region's matrix instructions with its
  // vector/LDS work so the MFMA pipe stays fed from a single wave.
  constexpr int MF1 = kNkb * KS * QB;   // S MFMAs per tile
  constexpr int MF2 = NT * NDB * QB;    // P.V MFMAs per tile
  constexpr int V1 = (kNkb * 16 * 2 + NT * 8) * QB;  // fma+exp, pack+sum per tile
  constexpr int V2 = kNkb * 16 * QB + kNkb * 8 * QB; // fp32 sums + max3
  auto interleave1 = [&]() {
    if (!ATTN_FWD_SCHED) return;
#pragma unroll
    for (int i = 0; i < MF1 / QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);             // MFMA (one K operand)
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // K operand read
      __builtin_amdgcn_sched_group_barrier(0x002, V1 * QB / MF1, 0);  // VALU
    }
  };
  auto interleave2 = [&]() {
    if (!ATTN_FWD_SCHED) return;
#pragma unroll
    for (int i = 0; i < MF2 / QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);                       // MFMA (one V operand)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                        // V^T transpose reads
      __builtin_amdgcn_sched_group_barrier(0x002, (V2 * QB + MF2 - 1) / MF2, 0);  // VALU
    }
  };

  // Iteration j (P = j & 1, a literal at every call): scores of tile j are in
  // sreg[P] with the reference max already raised; K_{j+1} is in kbuf[P^1],
  // V_j in vbuf[P].
  auto step = [&](int j, const int P) {
    if (j + 2 < nkt) issue_k(j + 2, P);      // K_j's buffer was last read in iteration j-1
    if (j + 1 < nkt) issue_v(j + 1, P ^ 1);  // V_{j-1}'s buffer likewise
    u32x4 pt[QB][NT];
    // region 1: S_{j+1} on the matrix cores, P_j on the vector ALUs
    scores(sreg[P ^ 1], P ^ 1);
    exponentiate(sreg[P], pt);
    interleave1();
    // region 2: O += V_j^T P_j, the fp32 sums of P_j and the max of S_{j+1}
    accumulate(pt, P);
    sum_p(sreg[P]);
    float mx[QB];
    rowmax(sreg[P ^ 1], mx);
    interleave2();
    if (j + 1 >= nfull) {  // rare: the next tile is on the diagonal or the tail
      mask(sreg[P ^ 1], (j + 1) * kBc);
      rowmax(sreg[P ^ 1], mx);
    }
    raise_ref(mx);
    wait_vmem_all();
    __syncthreads();
  };
  // last tile: no next scores
  auto last = [&](const int P) {
    u32x4 pt[QB][NT];
    exponentiate(sreg[P], pt);
    accumulate(pt, P);
    sum_p(sreg[P]);
  };

  if (nkt > 0) {
    issue_k(0, 0);
    issue_v(0, 0);
    if (nkt > 1) issue_k(1, 1);
    wait_vmem_all();
    __syncthreads();
    scores(sreg[0], 0);
    if (0 >= nfull) mask(sreg[0], 0);
    {
      float mx[QB];
      rowmax(sreg[0], mx);
      raise_ref(mx);
    }
    wait_vmem_all();
    __syncthreads();
    int j = 0;
    for (; j + 2 < nkt; j += 2) {
      step(j, 0);
      step(j + 1, 1);
    }
    if (j + 1 < nkt) {
      step(j, 0);
      last(1);
    } else {
      last(0);
    }
  }

  // ---- epilogue: one normalised write per row
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = wq0 + 32 * qb + n;
    const float lt = sum_halves(l_run[qb]);
    const float lr = sum_halves(l_rnd[qb]);
    if (qrow < a.Sq) {
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      uint16_t* O = a.o + ((size_t)(b * a.H + hq) * a.Sq + qrow) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          // registers 4*rg .. 4*rg+3: head dims 32*db + 8*rg + 4*h + 0..3
          const uint32_t w0 = pack_bf16x2(acc_o[qb][db][4 * rg + 0] * inv, acc_o[qb][db][4 * rg + 1] * inv);
          const uint32_t w1 = pack_bf16x2(acc_o[qb][db][4 * rg + 2] * inv, acc_o[qb][db][4 * rg + 3] * inv);
          *reinterpret_cast<u32x2*>(O + 32 * db + 8 * rg + 4 * h) = u32x2{w0, w1};
        }
      if (a.lse != nullptr && h == 0) {
        a.lse[(size_t)(b * a.H + hq) * a.Sq + qrow] =
            lt > 0.f ? (m_ref[qb] + fast_log2(lt)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& p, hipStream_t s) {
  FwdKernelArgs a;
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
  const long long grid = (long long)p.B * p.H * a.nqb;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& p, hipStream_t s) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return p.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace attn
