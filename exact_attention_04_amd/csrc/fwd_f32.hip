// Forward attention for fp32 inputs (fp32 throughout, no down-conversion).
//
// Same algorithm as the bf16 kernel -- "Warmup Guide -- Inference
// Optimization at Depth", Ch.4 tiling with Ch.3's online softmax -- but on the
// vector ALUs: fp32 operands gain nothing from the bf16 matrix cores, and this
// path serves small fp32 problems where exactness to ~1e-6 matters more than
// throughput.  It is therefore laid out for latency on few rows:
//   * a workgroup owns 16 query rows, so even a 2-head, 256-row problem
//     spreads over 32 workgroups;
//   * each row is held by TPQ lanes of every wave, each lane holding D/TPQ
//     head-dim elements of q and of the accumulator (a score is TPQ partial
//     dot products and two butterfly exchanges);
//   * K/V tiles of 64 keys go through LDS; each of the four waves takes 16 of
//     a tile's keys for the same 16 rows and keeps its own (m, l, O), and the
//     four partial states are combined at the end with Ch.3's two-block
//     update (the same rescaling by exp(m_w - m));
//   * the next tile is loaded into registers while the current one is
//     computed, so each tile costs one LDS store and one barrier pair.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTk = 64;                 // keys per LDS tile
constexpr int kKpw = kTk / kWaves;      // keys of a tile per wave
constexpr int kRows = 16;               // query rows per workgroup
constexpr int kTpq = 64 / kRows;        // lanes per query row within a wave

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
  constexpr int EPL = D / kTpq;                  // head-dim elements per lane
  constexpr int F4 = kTk * D / 4 / kThreads;     // float4 per thread per K (or V) tile
  __shared__ __attribute__((aligned(16))) float k_lds[kTk * D];
  __shared__ __attribute__((aligned(16))) float v_lds[kTk * D];
  __shared__ float red_m[kWaves][kRows], red_l[kWaves][kRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane / kTpq, sub = lane % kTpq;  // row within the block, lane within the row
  const int bh = blockIdx.x / a.nqb;
  const int qb = blockIdx.x - bh * a.nqb;
  const int b = bh / a.H, hq = bh - b * a.H;
  const int g = hq / (a.H / a.Hkv);
  const int q0 = qb * kRows;
  const int qrow = q0 + rr;
  const int shift = a.Sk - a.Sq;

  const float* Q = a.q + (size_t)(b * a.H + hq) * a.Sq * D;
  const float* K = a.k + (size_t)(b * a.Hkv + g) * a.Sk * D;
  const float* V = a.v + (size_t)(b * a.Hkv + g) * a.Sk * D;

  // keys the block visits, and this row's last visible key (may be < 0)
  int kend = a.Sk;
  if (CAUSAL) kend = min(a.Sk, min(q0 + kRows, a.Sq) + shift);
  kend = max(kend, 0);
  const int lim = qrow < a.Sq ? (CAUSAL ? min(a.Sk - 1, qrow + shift) : a.Sk - 1) : -1;

  float q[EPL], acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    q[i] = (qrow < a.Sq) ? Q[(size_t)qrow * D + sub * EPL + i] : 0.f;
    acc[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;  // base-2 domain

  // tile loads: thread t moves float4 number t + i * kThreads of the tile
  // (rows past Sk read as zeros)
  f32x4 kn[F4], vn[F4];
  auto fetch = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int e = (tid + i * kThreads) * 4;
      const int r = e / D;
      const bool ok = j0 + r < a.Sk;
      kn[i] = ok ? *reinterpret_cast<const f32x4*>(K + (size_t)j0 * D + e) : f32x4{0.f, 0.f, 0.f, 0.f};
      vn[i] = ok ? *reinterpret_cast<const f32x4*>(V + (size_t)j0 * D + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (kend > 0) fetch(0);

  for (int j0 = 0; j0 < kend; j0 += kTk) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const int e = (tid + i * kThreads) * 4;
      *reinterpret_cast<f32x4*>(k_lds + e) = kn[i];
      *reinterpret_cast<f32x4*>(v_lds + e) = vn[i];
    }
    __syncthreads();
    if (j0 + kTk < kend) fetch(j0 + kTk);  // lands while this tile is computed

    // this wave's keys of the tile: scores, one rescale, then P.V
    const int jw = j0 + wave * kKpw;
    float s[kKpw];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kKpw; ++kk) {
      const float* kr = k_lds + (wave * kKpw + kk) * D + sub * EPL;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) dot = fmaf(q[i], kr[i], dot);
#pragma unroll
      for (int w = 1; w < kTpq; w <<= 1) dot += __shfl_xor(dot, w, 64);
      s[kk] = (jw + kk <= lim) ? dot * a.c2 : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 while nothing was visible
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kKpw; ++kk) {
      const float p = fast_exp2(s[kk] - m_use);
      l_run += p;
      const float* vr = v_lds + (wave * kKpw + kk) * D + sub * EPL;
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[i] = fmaf(p, vr[i], acc[i]);
    }
    m_run = m_new;
  }

  // combine the four waves' states of each row (two-block update), through
  // LDS: the tile buffers hold the accumulators
  __syncthreads();
  if (sub == 0) {
    red_m[wave][rr] = m_run;
    red_l[wave][rr] = l_run;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) k_lds[(wave * kRows + rr) * D + sub * EPL + i] = acc[i];
  __syncthreads();
  if (wave == 0 && qrow < a.Sq) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][rr]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float f[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f[w] = fast_exp2(red_m[w][rr] - M_use);
      L = fmaf(f[w], red_l[w][rr], L);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* O = a.o + ((size_t)(b * a.H + hq) * a.Sq + qrow) * D + sub * EPL;
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
      f32x4 ov;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) x = fmaf(f[w], k_lds[(w * kRows + rr) * D + sub * EPL + i + u], x);
        ov[u] = x * inv;
      }
      *reinterpret_cast<f32x4*>(O + i) = ov;
    }
    if (a.lse != nullptr && sub == 0)
      a.lse[(size_t)(b * a.H + hq) * a.Sq + qrow] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& p, hipStream_t s) {
  F32Args a{};  // every field zero/null until set
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.H = p.H;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.nqb = (p.Sq + kRows - 1) / kRows;
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
