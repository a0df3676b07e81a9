// Speculative-verify attention: kq new queries per sequence against a long,
// ragged KV cache, as split-KV Flash-Decoding.
//
// "Making Decode Fast", §5 (Flash-Decoding): with very few queries a
// FlashAttention grid over query blocks leaves the GPU idle, so the keys of
// each sequence are split into chunks processed by different compute units,
// followed by a small final combine.  The combine is the two-block update of
// "Warmup Guide -- Inference Optimization at Depth", Ch.3 written with
// LSE = m + ln l.
//
// Split kernel -- one workgroup per (sequence b, KV head g, chunk of kChunk
// keys):
//   * the (H/Hkv)*kq query rows that read KV head g are packed into one
//     32-row tile, so each K/V byte of the chunk is read from HBM once;
//   * the four waves take interleaved 32-key steps of the chunk; K and V go
//     straight from HBM into matrix-core operands (each element is used by
//     one wave only, so LDS staging would buy nothing);
//   * S^T = K Q^T and O^T += V^T P^T on the 32x32x16 bf16 MFMA as in the
//     prefill kernel; V^T operands come from 8-byte row segments regrouped
//     with byte permutes;
//   * the waves' (m, l, O) are combined through LDS and the chunk writes one
//     fp32 partial (O_c normalised, base-2 LSE_c) per packed row.
// Merge kernel -- one wave per output row combines the partials of its
// sequence's chunks and writes O (bf16) and LSE (natural log).
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kChunk = 1024;  // keys per split-KV chunk
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;  // keys per wave step

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seqlens;
  float* part_o;    // [B][Hkv][nch][R][D]
  float* part_lse;  // [B][Hkv][nch][R]   base-2 domain: m2 + log2(l)
  int H, Hkv, kq, R, G;
  int max_seqlen, cache_stride, nch;
  float c2;  // scale * log2(e)
};

__device__ __forceinline__ int clamp_len(int s, int max_len) { return min(max(s, 0), max_len); }

template <int D>
__global__ void __launch_bounds__(kThreads, 2) verify_split_kernel(SplitArgs a) {
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ float red_o[kWaves][D][32];
  __shared__ float red_m[kWaves][32];
  __shared__ float red_l[kWaves][32];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int sk = clamp_len(a.seqlens[b], a.max_seqlen);
  const int cstart = c * kChunk;
  if (cstart >= sk) return;  // uniform over the workgroup
  const int cend = min(sk, cstart + kChunk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  // packed row n = (query head g*G + n / kq, new token n % kq)
  const bool row_ok = n < a.R;
  const int hh = n / a.kq, qi = n - hh * a.kq;
  const int row_lim = sk - a.kq + qi;  // last visible key of this row

  const uint16_t* Kb = a.k + (size_t)(b * a.Hkv + g) * a.cache_stride * D;
  const uint16_t* Vb = a.v + (size_t)(b * a.Hkv + g) * a.cache_stride * D;

  u32x4 qf[KS];
  {
    const uint16_t* qrow = a.q + ((size_t)(b * a.H + g * a.G + hh) * a.kq + qi) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? load16(qrow + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j0 = cstart + wave * kStep; j0 < cend; j0 += kWaves * kStep) {
    // ---- K operand: row j0 + n, eight head-dim values per step
    u32x4 kf[KS];
    const bool krow_ok = j0 + n < sk;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = krow_ok ? load16(Kb + (size_t)(j0 + n) * D + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
    // ---- V segments: for each of the 16 keys this lane half needs, head
    // dims [NDB*n, NDB*n + NDB)
    uint32_t x[2][8][NDB / 2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = j0 + 16 * t + 8 * (e / 4) + 4 * h + (e % 4);
        const bool ok = key < sk;
        const uint16_t* src = Vb + (size_t)key * D + NDB * n;
        if constexpr (NDB == 4) {
          const u32x2 w = ok ? *reinterpret_cast<const u32x2*>(src) : u32x2{0, 0};
          x[t][e][0] = w[0];
          x[t][e][1] = w[1];
        } else {
          x[t][e][0] = ok ? *reinterpret_cast<const uint32_t*>(src) : 0u;
        }
      }

    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma_32x32x16_bf16(kf[ks], qf[ks], s);

    // mask keys past a row's limit (only the chunk's last steps need it)
    if (j0 + kStep - 1 > sk - a.kq) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r / 4) + 4 * h + (r % 4);
        if (key > row_lim || key >= sk) s[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * a.c2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(fmaf(s[r], a.c2, -m_use));
      s[r] = p;
      rs += p;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;

#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 pt;
      pt[0] = pack_bf16x2(s[8 * t + 0], s[8 * t + 1]);
      pt[1] = pack_bf16x2(s[8 * t + 2], s[8 * t + 3]);
      pt[2] = pack_bf16x2(s[8 * t + 4], s[8 * t + 5]);
      pt[3] = pack_bf16x2(s[8 * t + 6], s[8 * t + 7]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x4 vf;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t lo = x[t][2 * e2][db / 2], hi = x[t][2 * e2 + 1][db / 2];
          vf[e2] = (db & 1) ? pack_hi16(lo, hi) : pack_lo16(lo, hi);
        }
        acc_o[db] = mfma_32x32x16_bf16(vf, pt, acc_o[db]);
      }
    }
  }

  // ---- combine the four waves through LDS
  const float l_tot = l_run + swap_halves(l_run);
  if (h == 0) {
    red_m[wave][n] = m_run;
    red_l[wave][n] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r / 4) + 4 * h + (r % 4);
      red_o[wave][NDB * m + db][n] = acc_o[db][r];
    }
  __syncthreads();

  {
    const int rn = tid & 31;     // packed row
    const int dg = tid >> 5;     // group of D/8 head dims
    constexpr int DPT = D / 8;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][rn]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float f[kWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f[w] = fast_exp2(red_m[w][rn] - M_use);
      L += f[w] * red_l[w][rn];
    }
    if (rn < a.R) {
      const size_t pidx = ((size_t)(b * a.Hkv + g) * a.nch + c) * a.R + rn;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* dst = a.part_o + pidx * D + dg * DPT;
#pragma unroll
      for (int d4 = 0; d4 < DPT; d4 += 4) {
        f32x4 vv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) acc = fmaf(f[w], red_o[w][dg * DPT + d4 + u][rn], acc);
          vv[u] = acc * inv;
        }
        *reinterpret_cast<f32x4*>(dst + d4) = vv;
      }
      if (dg == 0) a.part_lse[pidx] = L > 0.f ? M + fast_log2(L) : -INFINITY;
    }
  }
}

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* seqlens;
  uint16_t* o;
  float* lse;
  int B, H, Hkv, kq, R, G;
  int max_seqlen, nch;
};

// One wave per (b, query head, new token): combine the chunk partials.
template <int D>
__global__ void __launch_bounds__(256) verify_merge_kernel(MergeArgs a) {
  constexpr int EPL = D / 64;  // head dims per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int total = a.B * a.H * a.kq;
  if (row >= total) return;
  const int qi = row % a.kq;
  const int hq = (row / a.kq) % a.H;
  const int b = row / (a.kq * a.H);
  const int g = hq / a.G, hh = hq - g * a.G;
  const int rn = hh * a.kq + qi;
  const int sk = clamp_len(a.seqlens[b], a.max_seqlen);
  const int nc = (sk + kChunk - 1) / kChunk;
  const size_t base = (size_t)(b * a.Hkv + g) * a.nch;

  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_lse[(base + c) * a.R + rn]);
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t pidx = (base + c) * a.R + rn;
    const float w = fast_exp2(a.part_lse[pidx] - M_use);
    L += w;
    const float* src = a.part_o + pidx * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, src[e], acc[e]);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = a.o + ((size_t)(b * a.H + hq) * a.kq + qi) * D + lane * EPL;
  if constexpr (EPL == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    const __bf16 v = (__bf16)(acc[0] * inv);
    *dst = __builtin_bit_cast(uint16_t, v);
  }
  if (a.lse != nullptr && lane == 0) {
    a.lse[(size_t)(b * a.H + hq) * a.kq + qi] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
  }
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

template <int D>
hipError_t launch(const VerifyArgs& p, hipStream_t s) {
  const int G = p.H / p.Hkv;
  const int R = G * p.kq;
  const int nch = (p.max_seqlen_k + kChunk - 1) / kChunk;
  const size_t n_parts = (size_t)p.B * p.Hkv * nch * R;
  float* part_o = static_cast<float*>(p.workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + align_up(n_parts * D * 4));

  SplitArgs sa;
  sa.q = static_cast<const uint16_t*>(p.q);
  sa.k = static_cast<const uint16_t*>(p.k);
  sa.v = static_cast<const uint16_t*>(p.v);
  sa.seqlens = p.seqlens;
  sa.part_o = part_o;
  sa.part_lse = part_lse;
  sa.H = p.H;
  sa.Hkv = p.Hkv;
  sa.kq = p.kq;
  sa.R = R;
  sa.G = G;
  sa.max_seqlen = p.max_seqlen_k;
  sa.cache_stride = p.cache_stride;
  sa.nch = nch;
  sa.c2 = p.scale * kLog2e;
  if (nch > 0) {
    hipLaunchKernelGGL((verify_split_kernel<D>), dim3(nch, p.Hkv, p.B), dim3(kThreads), 0, s, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  MergeArgs ma;
  ma.part_o = part_o;
  ma.part_lse = part_lse;
  ma.seqlens = p.seqlens;
  ma.o = static_cast<uint16_t*>(p.o);
  ma.lse = p.lse;
  ma.B = p.B;
  ma.H = p.H;
  ma.Hkv = p.Hkv;
  ma.kq = p.kq;
  ma.R = R;
  ma.G = G;
  ma.max_seqlen = p.max_seqlen_k;
  ma.nch = nch;
  const int rows = p.B * p.H * p.kq;
  hipLaunchKernelGGL((verify_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, s, ma);
  return hipGetLastError();
}

}  // namespace

int verify_chunk_keys() { return kChunk; }

size_t verify_workspace_bytes(int B, int H, int kq, int d, int max_seqlen_k) {
  const size_t nch = (size_t)((max_seqlen_k + kChunk - 1) / kChunk);
  const size_t n_parts = (size_t)B * H * kq * nch;
  return align_up(n_parts * d * 4) + align_up(n_parts * 4);
}

hipError_t launch_verify_bf16(const VerifyArgs& p, hipStream_t s) {
  return p.d == 128 ? launch<128>(p, s) : launch<64>(p, s);
}

}  // namespace attn
