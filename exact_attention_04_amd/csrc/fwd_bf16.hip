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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per K/V tile
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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

// 16-byte chunk positions inside an LDS row (XOR swizzles).  K: the 32 rows
// an A-operand read touches spread over all banks.  V: the 8 rows x 64 bytes
// a transpose read touches spread over all banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0), other counters untouched
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) fwd_bf16_kernel(FwdKernelArgs a) {
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int KS = D / 16;   // MFMA steps over the head dim for S^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T (head dim)
  constexpr int TILE = kBc * D;  // elements per K or V tile
  constexpr int ROWS_PER_INSN = 1024 / (D * 2);  // rows one wave-wide 1 KB load covers
  constexpr int INSN_PER_WAVE = TILE * 2 / 1024 / kWaves;

  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][TILE];

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

  // ---- direct HBM -> LDS tile loads.  Wave-wide instruction i of this wave
  // fills LDS bytes [1024*(wave*INSN_PER_WAVE + i), +1024); lane l's 16
  // bytes land at offset 16*l, i.e. row r = first row + l / CPR, chunk
  // position l % CPR, which holds global chunk (position ^ swizzle(r)).
  // Rows past Sk re-read row Sk-1: finite data whose probability is 0.
  auto issue_tile = [&](int j0, int buf) {
#pragma unroll
    for (int i = 0; i < INSN_PER_WAVE; ++i) {
      const int insn = wave * INSN_PER_WAVE + i;
      const int row = insn * ROWS_PER_INSN + lane / CPR;
      const int pos = lane % CPR;
      const int grow = min(j0 + row, a.Sk - 1);
      const uint16_t* kg = K + (size_t)grow * D + ((pos ^ k_swz<D>(row)) * 8);
      const uint16_t* vg = V + (size_t)grow * D + ((pos ^ v_swz<D>(row)) * 8);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)kg,
                                       (lds_void*)(&k_lds[buf][insn * 512]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)vg,
                                       (lds_void*)(&v_lds[buf][insn * 512]), 16, 0, 0);
    }
  };

  // Q^T as the B operand: column n = query, eight head-dim values per step.
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = (qrow < a.Sq) ? load16(Q + (size_t)qrow * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_ref = -INFINITY;  // reference max, base-2 domain (scaled logits * log2 e)
  float l_run = 0.f;        // running denominator, this lane's keys only
  float l_rnd = 0.f;        // same, of the bf16-rounded probabilities

  // lane constants of the transpose read: group of 16 lanes gq, row r4 of
  // the 4x16 block this lane addresses, 4-element column chunk c4
  const int gq = lane >> 4, r4 = (lane >> 2) & 3, c4 = lane & 3;

  auto compute_tile = [&](int j0, int buf) {
    const bool wave_live = (wq0 < a.Sq) && (!CAUSAL || j0 <= wq0 + 31 + shift);
    if (!wave_live) return;
    const lds_u16* kt = (const lds_u16*)&k_lds[buf][0];
    const lds_u16* vt = (const lds_u16*)&v_lds[buf][0];
    // ---- S^T = K Q^T for the two 32-key blocks of the tile
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int krow = kb * 32 + n;
        const int c = (ks * 2 + h) ^ k_swz<D>(krow);
        const u32x4 kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kt + krow * D + c * 8);
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
    // ---- online softmax (base 2, lazily raised reference max)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, swap_halves(mx)) * a.c2;
    const bool raise = mx > m_ref + kRescaleSlack;
    if (__any(raise)) {
      const float m_new = raise ? mx : m_ref;
      const float alpha = raise ? fast_exp2(m_ref - mx) : 1.f;  // 0 when m_ref = -inf
      l_run *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;  // nothing visible yet
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], a.c2, -m_use));
        s[kb][r] = p;
        rs += p;
      }
    l_run += rs;
    // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, base = (t & 1) * 8;
      u32x4 pt;
      pt[0] = pack_bf16x2(s[kb][base + 0], s[kb][base + 1]);
      pt[1] = pack_bf16x2(s[kb][base + 2], s[kb][base + 3]);
      pt[2] = pack_bf16x2(s[kb][base + 4], s[kb][base + 5]);
      pt[3] = pack_bf16x2(s[kb][base + 6], s[kb][base + 7]);
#pragma unroll
      for (int w = 0; w < 4; ++w) l_rnd = sum_bf16x2(pt[w], l_rnd);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // items 0..3: keys 16t + 4h + r4; items 4..7: keys 16t + 8 + 4h + r4
        // column chunk: head dims 32*db + 16*(gq & 1) + 4*c4 .. +3
        const int dcol = 32 * db + 16 * (gq & 1) + 4 * c4;
        i16x4 lo, hi;
        {
          const int row = 16 * t + 4 * h + r4;
          const int pos = (dcol >> 3) ^ v_swz<D>(row);
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + row * D + pos * 8 + (dcol & 7)));
        }
        {
          const int row = 16 * t + 8 + 4 * h + r4;
          const int pos = (dcol >> 3) ^ v_swz<D>(row);
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + row * D + pos * 8 + (dcol & 7)));
        }
        u32x4 vf;
        vf[0] = __builtin_bit_cast(u32x2, lo)[0];
        vf[1] = __builtin_bit_cast(u32x2, lo)[1];
        vf[2] = __builtin_bit_cast(u32x2, hi)[0];
        vf[3] = __builtin_bit_cast(u32x2, hi)[1];
        acc_o[db] = mfma_32x32x16_bf16(vf, pt, acc_o[db]);
      }
    }
  };

  if (nkt > 0) issue_tile(0, 0);
  wait_vmem_all();
  __syncthreads();
  for (int jt = 0; jt < nkt; jt += 2) {
    // even tile from buffer 0, odd tile from buffer 1 (static buffer index)
    if (jt + 1 < nkt) issue_tile((jt + 1) * kBc, 1);
    compute_tile(jt * kBc, 0);
    wait_vmem_all();
    __syncthreads();
    if (jt + 1 < nkt) {
      if (jt + 2 < nkt) issue_tile((jt + 2) * kBc, 0);
      compute_tile((jt + 1) * kBc, 1);
      wait_vmem_all();
      __syncthreads();
    }
  }

  // ---- epilogue: one normalised write per row
  const float lt = l_run + swap_halves(l_run);
  const float lr = l_rnd + swap_halves(l_rnd);
  if (qrow < a.Sq) {
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    uint16_t* O = a.o + ((size_t)(b * a.H + hq) * a.Sq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        // registers 4*rg .. 4*rg+3: head dims 32*db + 8*rg + 4*h + 0..3
        const uint32_t w0 = pack_bf16x2(acc_o[db][4 * rg + 0] * inv, acc_o[db][4 * rg + 1] * inv);
        const uint32_t w1 = pack_bf16x2(acc_o[db][4 * rg + 2] * inv, acc_o[db][4 * rg + 3] * inv);
        *reinterpret_cast<u32x2*>(O + 32 * db + 8 * rg + 4 * h) = u32x2{w0, w1};
      }
    if (a.lse != nullptr && h == 0) {
      a.lse[(size_t)(b * a.H + hq) * a.Sq + qrow] =
          lt > 0.f ? (m_ref + fast_log2(lt)) * kLn2 : -INFINITY;
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
