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
//     owns 32 rows; K/V tiles of 64 keys are staged in LDS and shared by the
//     four waves;
//   * scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//     MFMA, so that each lane holds one query column and 32 of the tile's 64
//     keys: the row max is an in-lane reduction plus one exchange with the
//     other wave half, and the row sum is kept per lane until the end;
//   * the output is accumulated transposed too, O^T += V^T P^T: P^T is the
//     B operand straight from the score registers (rounded to bf16), and the
//     rescale factor of a query is a per-lane scalar;
//   * V^T operands are built from row-major V in LDS: lane m reads, for each
//     of its 8 keys, the head-dim elements [NDB*m, NDB*m + NDB) and
//     regroups them with byte permutes, so O^T row m of d-block db holds head
//     dim NDB*m + db;
//   * the softmax works in base 2 with scale*log2(e) folded into one FMA.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per K/V tile

struct FwdKernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int H, Hkv, Sq, Sk;
  int nqb;        // query blocks per (batch, head)
  float c2;       // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) fwd_bf16_kernel(FwdKernelArgs a) {
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int KS = D / 16;   // MFMA steps over the head dim for S^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T (head dim)
  constexpr int CPT = kBc * CPR / kThreads;  // staged chunks per thread per tile

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBc * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kBc * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;  // query column within the wave's 32 rows
  const int h = lane >> 5;  // wave half

  const int blk = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = blk / a.nqb;
  int qb = blk - bh * a.nqb;
  if (CAUSAL) qb = a.nqb - 1 - qb;  // heaviest query blocks of a head first
  const int b = bh / a.H;
  const int hq = bh - b * a.H;
  const int g = hq / (a.H / a.Hkv);

  const int q0 = qb * kBr;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + n;
  const int shift = a.Sk - a.Sq;  // bottom-right causal alignment

  const uint16_t* Q = a.q + (size_t)(b * a.H + hq) * a.Sq * D;
  const uint16_t* K = a.k + (size_t)(b * a.Hkv + g) * a.Sk * D;
  const uint16_t* V = a.v + (size_t)(b * a.Hkv + g) * a.Sk * D;

  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, min(q0 + kBr, a.Sq) + shift);
  kend = max(kend, 0);
  const int nkt = (kend + kBc - 1) / kBc;

  // Q^T as the B operand: column n = query, eight head-dim values per step.
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = (qrow < a.Sq) ? load16(Q + (size_t)qrow * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY;  // running max, base-2 domain (scaled logits * log2 e)
  float l_run = 0.f;        // running denominator, this lane's keys only

  u32x4 kst[CPT], vst[CPT];
  auto stage = [&](int j0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / CPR, c = ci % CPR;
      const bool ok = j0 + row < a.Sk;
      const size_t off = (size_t)(j0 + row) * D + c * 8;
      kst[i] = ok ? load16(K + off) : u32x4{0, 0, 0, 0};
      vst[i] = ok ? load16(V + off) : u32x4{0, 0, 0, 0};
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / CPR, c = ci % CPR;
      // K rows are XOR-swizzled in 16-byte chunks so that the 32 different
      // rows an MFMA A-operand read touches fall in distinct banks.
      store16(&k_lds[row * D + ((c ^ (row & (CPR - 1))) * 8)], kst[i]);
      store16(&v_lds[row * D + c * 8], vst[i]);
    }
  };

  if (nkt > 0) {
    stage(0);
    commit();
  }
  __syncthreads();

  for (int jt = 0; jt < nkt; ++jt) {
    const int j0 = jt * kBc;
    if (jt + 1 < nkt) stage(j0 + kBc);  // global loads overlap this tile's math

    const bool wave_live = (wq0 < a.Sq) && (!CAUSAL || j0 <= wq0 + 31 + shift);
    if (wave_live) {
      // ---- S^T = K Q^T for the two 32-key blocks of the tile
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int krow = kb * 32 + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = (ks * 2 + h) ^ (krow & (CPR - 1));
          const u32x4 kf = *reinterpret_cast<const u32x4*>(&k_lds[krow * D + c * 8]);
          s[kb] = mfma_32x32x16_bf16(kf, qf[ks], s[kb]);
        }
      }
      // ---- mask the causal diagonal and the ragged tail (only where needed)
      const bool need_mask = (j0 + kBc > a.Sk) || (CAUSAL && j0 + kBc - 1 > wq0 + shift);
      if (need_mask) {
        const int lim = CAUSAL ? min(a.Sk - 1, qrow + shift) : a.Sk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + 8 * (r / 4) + 4 * h + (r % 4);
            if (key > lim) s[kb][r] = -INFINITY;
          }
      }
      // ---- online softmax (base 2)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx * a.c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // all-masked so far
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], a.c2, -m_use));
          s[kb][r] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      }
      // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, base = (t & 1) * 8;
        u32x4 pt;
        pt[0] = pack_bf16x2(s[kb][base + 0], s[kb][base + 1]);
        pt[1] = pack_bf16x2(s[kb][base + 2], s[kb][base + 3]);
        pt[2] = pack_bf16x2(s[kb][base + 4], s[kb][base + 5]);
        pt[3] = pack_bf16x2(s[kb][base + 6], s[kb][base + 7]);
        // the 8 keys of this step held by this lane half (same order as pt)
        uint32_t x[8][NDB / 2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * t + 8 * (e / 4) + 4 * h + (e % 4);
          const uint16_t* src = &v_lds[key * D + NDB * n];
          if constexpr (NDB == 4) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(src);
            x[e][0] = w[0];
            x[e][1] = w[1];
          } else {
            x[e][0] = *reinterpret_cast<const uint32_t*>(src);
          }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x4 vf;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const uint32_t lo = x[2 * e2][db / 2], hi = x[2 * e2 + 1][db / 2];
            vf[e2] = (db & 1) ? pack_hi16(lo, hi) : pack_lo16(lo, hi);
          }
          acc_o[db] = mfma_32x32x16_bf16(vf, pt, acc_o[db]);
        }
      }
    }
    __syncthreads();
    if (jt + 1 < nkt) {
      commit();
      __syncthreads();
    }
  }

  // ---- epilogue: one normalised write per row
  const float lt = l_run + swap_halves(l_run);
  if (qrow < a.Sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* O = a.o + ((size_t)(b * a.H + hq) * a.Sq + qrow) * D;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      // registers 4*rg .. 4*rg+3 of every d-block: head dims
      // [NDB*(8*rg + 4*h), NDB*(8*rg + 4*h) + 4*NDB) contiguous
      uint32_t w[2 * NDB];
#pragma unroll
      for (int ri = 0; ri < 4; ++ri) {
#pragma unroll
        for (int db = 0; db < NDB; db += 2) {
          w[(ri * NDB + db) / 2] = pack_bf16x2(acc_o[db][4 * rg + ri] * inv, acc_o[db + 1][4 * rg + ri] * inv);
        }
      }
      uint16_t* dst = O + NDB * (8 * rg + 4 * h);
#pragma unroll
      for (int c = 0; c < NDB / 2; ++c) {
        store16(dst + c * 8, u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]});
      }
    }
    if (a.lse != nullptr && h == 0) {
      a.lse[(size_t)(b * a.H + hq) * a.Sq + qrow] =
          lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : -INFINITY;
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
