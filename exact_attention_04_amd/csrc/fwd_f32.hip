// Forward attention for fp32 inputs (fp32 throughout, no down-conversion).
//
// Same algorithm as the bf16 kernel -- "Warmup Guide -- Inference
// Optimization at Depth", Ch.4 tiling with Ch.3's online softmax -- but on the
// vector ALUs: fp32 operands gain nothing from the bf16 matrix cores, and this
// path serves small fp32 problems where exactness to ~1e-6 matters more than
// throughput.  Each query row is owned by D/32 consecutive lanes, each lane
// holding 32 head-dim elements of q and of the accumulator; K/V tiles of 32
// keys are staged in LDS and read as broadcasts.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kTk = 32;  // keys per tile

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int H, Hkv, Sq, Sk;
  int nqb;
  float c2;  // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) fwd_f32_kernel(F32Args a) {
  constexpr int TPQ = D / 32;            // lanes per query row
  constexpr int QPB = kThreads / TPQ;    // query rows per workgroup
  __shared__ float k_lds[kTk][D];
  __shared__ float v_lds[kTk][D];

  const int tid = threadIdx.x;
  const int sub = tid % TPQ;
  const int bh = blockIdx.x / a.nqb;
  const int qb = blockIdx.x - bh * a.nqb;
  const int b = bh / a.H, hq = bh - b * a.H;
  const int g = hq / (a.H / a.Hkv);
  const int q0 = qb * QPB;
  const int qrow = q0 + tid / TPQ;
  const int shift = a.Sk - a.Sq;

  const float* Q = a.q + (size_t)(b * a.H + hq) * a.Sq * D;
  const float* K = a.k + (size_t)(b * a.Hkv + g) * a.Sk * D;
  const float* V = a.v + (size_t)(b * a.Hkv + g) * a.Sk * D;

  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, min(q0 + QPB, a.Sq) + shift);
  kend = max(kend, 0);
  const int lim = CAUSAL ? min(a.Sk - 1, qrow + shift) : a.Sk - 1;

  float q[32], acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    q[i] = (qrow < a.Sq) ? Q[(size_t)qrow * D + sub * 32 + i] : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  for (int j0 = 0; j0 < kend; j0 += kTk) {
    __syncthreads();
    for (int e = tid; e < kTk * D; e += kThreads) {
      const int r = e / D, c = e % D;
      const bool ok = j0 + r < a.Sk;
      k_lds[r][c] = ok ? K[(size_t)(j0 + r) * D + c] : 0.f;
      v_lds[r][c] = ok ? V[(size_t)(j0 + r) * D + c] : 0.f;
    }
    __syncthreads();

    float s[kTk];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kTk; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) dot = fmaf(q[i], k_lds[kk][sub * 32 + i], dot);
#pragma unroll
      for (int w = 1; w < TPQ; w <<= 1) dot += __shfl_xor(dot, w, 64);
      s[kk] = (j0 + kk <= lim) ? dot * a.c2 : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kTk; ++kk) {
      const float p = fast_exp2(s[kk] - m_use);
      l_run += p;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] = fmaf(p, v_lds[kk][sub * 32 + i], acc[i]);
    }
    m_run = m_new;
  }

  if (qrow < a.Sq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* O = a.o + ((size_t)(b * a.H + hq) * a.Sq + qrow) * D + sub * 32;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      *reinterpret_cast<f32x4*>(O + i) = f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
    }
    if (a.lse != nullptr && sub == 0) {
      a.lse[(size_t)(b * a.H + hq) * a.Sq + qrow] =
          l_run > 0.f ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& p, hipStream_t s) {
  constexpr int QPB = kThreads / (D / 32);
  F32Args a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.H = p.H;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.nqb = (p.Sq + QPB - 1) / QPB;
  a.c2 = p.scale * kLog2e;
  const long long grid = (long long)p.B * p.H * a.nqb;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& p, hipStream_t s) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return p.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace attn
