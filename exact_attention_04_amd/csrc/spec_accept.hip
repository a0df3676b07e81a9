// Speculative-decoding acceptance rule for a batch of sequences: accept or
// reject the k drafted tokens of each sequence against the target model's
// distributions, and sample the one extra token that every verify pass
// yields.
//
// "Warmup Guide -- Inference Optimization at Depth", Ch.6 (The Acceptance
// Rule): drafted token x, with draft probability q(x) and target probability
// p(x), is accepted with probability min(1, p(x)/q(x)); at the first rejection
// a replacement is sampled from norm(max(0, p - q)) and the rest of the draft
// is discarded.  "FlashAttention, speculative decoding, quantisation and
// parallelism", Mechanics / Speculative decoding (the three-step listing):
// when all k drafts are accepted, one more token is sampled from the target's
// distribution at position k.
//
// The random numbers are inputs: u_accept[b][i] is the uniform compared with
// min(1, p/q) at draft position i, u_sample[b] the uniform that picks the
// extra token.  Sampling is the inverse CDF of the (unnormalised) weights
// w_i on a fixed-point grid: W_i = floor(w_i * 2^40) as integers, T =
// floor(u * sum W), and the token is the first index whose running sum of W
// exceeds T.  The integer sums make the discrete choice independent of the
// summation order, so the parallel scan below and a sequential reference
// pick the same token.
//
// Two passes over the vocabulary, which is cut into chunks of kChunk entries:
//   pass 1 -- one workgroup per (sequence, chunk): find the sequence's first
//             rejection (one lane per draft position, a wave ballot), then
//             reduce the chunk's fixed-point weights of the distribution to
//             sample (the residual, or the target's bonus distribution) and of
//             the target distribution alone (the fallback when the residual
//             has no mass); the chunk-0 workgroup also records the rejection
//             index for pass 2;
//   pass 2 -- one workgroup per sequence: load the rejection index and the
//             chunk sums together (one memory round trip instead of the
//             dependent loads of the ballot), scan the sums, find the chunk
//             holding T, scan that chunk and write the outputs.
// Both passes read the vocabulary rows coalesced; the traffic is one read of
// the sampled rows.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 4096;                 // vocabulary entries per pass-1 workgroup
constexpr int kPerThread = kChunk / kThreads;  // 16
constexpr double kFix = 1099511627776.0;     // 2^40

struct SpecArgs {
  const int32_t* draft;  // [B][k]
  const float* q;        // [B][k][V]    draft distributions
  const float* p;        // [B][k+1][V]  target distributions
  const float* u_acc;    // [B][k]
  const float* u_smp;    // [B]
  int32_t* n_acc;        // [B]
  int32_t* tokens;       // [B][k+1]
  long long* sums;       // [B][nchunk][2]: weights to sample, target weights
  int32_t* first_rej;    // [B]: the first rejected position (k if none), from pass 1
  int B, k, V, nchunk;
};

// Index of the first rejected draft position of sequence b, k if none is
// rejected.  Every wave that calls it gets the same answer.
__device__ int first_rejection(const SpecArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  for (int i0 = 0; i0 < a.k; i0 += 64) {
    const int i = i0 + lane;
    bool rej = false;
    if (i < a.k) {
      const int x = a.draft[(size_t)b * a.k + i];
      if (x < 0 || x >= a.V) {
        rej = true;  // not a token of the vocabulary
      } else {
        const float qx = a.q[((size_t)b * a.k + i) * a.V + x];
        const float px = a.p[((size_t)b * (a.k + 1) + i) * a.V + x];
        const float u = a.u_acc[(size_t)b * a.k + i];
        // accept with probability min(1, p/q); a token the draft gave no
        // probability is kept iff the target gives it some
        const bool acc = qx > 0.f ? u < fminf(1.f, __fdiv_rn(px, qx)) : px > 0.f;
        rej = !acc;
      }
    }
    const uint64_t m = __ballot(rej);
    if (m != 0) return i0 + __ffsll((unsigned long long)m) - 1;
  }
  return a.k;
}

// fixed-point weight of a probability (clamped to [0, 1]; NaN counts 0)
__device__ __forceinline__ long long fix_weight(float w) {
  w = fminf(fmaxf(w, 0.f), 1.f);
  return (long long)((double)w * kFix);
}

// Inclusive sum over the workgroup of one int64 per thread, and the
// exclusive prefix of the calling thread; red holds kWaves partials.
__device__ long long block_scan(long long x, long long& excl, long long* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long long inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) red[w] = inc;
  __syncthreads();
  long long before = 0, total = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    before += v < w ? red[v] : 0;
    total += red[v];
  }
  __syncthreads();
  excl = before + inc - x;
  return total;
}

__global__ void __launch_bounds__(kThreads) spec_chunk_sums(SpecArgs a) {
  __shared__ long long red[2][kWaves];
  const int c = blockIdx.x, b = blockIdx.y;
  const int j = first_rejection(a, b);
  if (c == 0 && threadIdx.x == 0) a.first_rej[b] = j;
  const float* prow = a.p + ((size_t)b * (a.k + 1) + j) * a.V;
  const float* qrow = j < a.k ? a.q + ((size_t)b * a.k + j) * a.V : nullptr;
  long long ws = 0, wp = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = c * kChunk + i * kThreads + threadIdx.x;  // coalesced
    if (e < a.V) {
      const float pv = prow[e];
      const long long fp = fix_weight(pv);
      wp += fp;
      ws += qrow != nullptr ? fix_weight(pv - qrow[e]) : fp;
    }
  }
  // two reductions (order does not matter: integers)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ws += __shfl_xor(ws, off, 64);
    wp += __shfl_xor(wp, off, 64);
  }
  if (lane == 0) {
    red[0][w] = ws;
    red[1][w] = wp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long s0 = 0, s1 = 0;
    for (int v = 0; v < kWaves; ++v) {
      s0 += red[0][v];
      s1 += red[1][v];
    }
    long long* out = a.sums + ((size_t)b * a.nchunk + c) * 2;
    out[0] = s0;
    out[1] = s1;
  }
}

__global__ void __launch_bounds__(kThreads) spec_pick(SpecArgs a) {
  __shared__ long long red[kWaves];
  __shared__ long long s_found[2];  // chunk index, running sum before it
  const int b = blockIdx.x, tid = threadIdx.x;
  const int j = a.first_rej[b];  // written by pass 1's chunk-0 workgroup
  const long long* sums = a.sums + (size_t)b * a.nchunk * 2;
  constexpr int kChunksPerThread = 4;  // nchunk <= 1024 (V <= 2^22)

  // which distribution: the residual (or the bonus distribution when every
  // draft was accepted); the target's own if the residual has no mass
  long long g = 0;
  for (int cc = 0; cc < kChunksPerThread; ++cc) {
    const int c = tid * kChunksPerThread + cc;
    if (c < a.nchunk) g += sums[c * 2];
  }
  long long excl;
  long long total = block_scan(g, excl, red);
  int col = 0;
  if (total == 0) {
    col = 1;
    g = 0;
    for (int cc = 0; cc < kChunksPerThread; ++cc) {
      const int c = tid * kChunksPerThread + cc;
      if (c < a.nchunk) g += sums[c * 2 + 1];
    }
    total = block_scan(g, excl, red);
  }
  const bool use_q = j < a.k && col == 0;

  int token = -1;  // a distribution with no mass cannot be sampled
  if (total > 0) {
    float u = a.u_smp[b];
    if (!(u >= 0.f)) u = 0.f;  // NaN or negative: the first index with mass
    long long T = (long long)floor((double)u * (double)total);
    T = min(max(T, 0LL), total - 1);
    // the chunk whose running-sum interval holds T
    if (excl <= T && T < excl + g) {
      long long run = excl;
      for (int cc = 0; cc < kChunksPerThread; ++cc) {
        const int c = tid * kChunksPerThread + cc;
        const long long sc = c < a.nchunk ? sums[c * 2 + col] : 0;
        if (T < run + sc) {
          s_found[0] = c;
          s_found[1] = run;
          break;
        }
        run += sc;
      }
    }
    __syncthreads();
    const int c = (int)s_found[0];
    const long long base = s_found[1];
    // inside the chunk: thread t owns entries [t*16, t*16+16) in order
    const float* prow = a.p + ((size_t)b * (a.k + 1) + j) * a.V;
    const float* qrow = use_q ? a.q + ((size_t)b * a.k + j) * a.V : prow;
    long long wv[kPerThread];
    long long mine = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int e = c * kChunk + tid * kPerThread + i;
      long long wi = 0;
      if (e < a.V) {
        const float pv = prow[e];
        wi = use_q ? fix_weight(pv - qrow[e]) : fix_weight(pv);
      }
      wv[i] = wi;
      mine += wi;
    }
    long long ex2;
    block_scan(mine, ex2, red);
    const long long start = base + ex2;
    if (start <= T && T < start + mine) {
      long long run = start;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        run += wv[i];
        if (T < run) {
          s_found[0] = c * kChunk + tid * kPerThread + i;
          break;
        }
      }
    }
    __syncthreads();
    token = (int)s_found[0];
  }
  // outputs: the accepted prefix, the sampled token, -1 after it
  for (int i = tid; i <= a.k; i += kThreads) {
    int t = -1;
    if (i < j) t = a.draft[(size_t)b * a.k + i];
    if (i == j) t = token;
    a.tokens[(size_t)b * (a.k + 1) + i] = t;
  }
  if (tid == 0) a.n_acc[b] = j;
}

}  // namespace

// chunk sums, then the rejection indices (16-byte aligned)
static size_t spec_sums_bytes(int B, int V) {
  const size_t nchunk = ((size_t)V + kChunk - 1) / kChunk;
  return ((size_t)B * nchunk * 2 * sizeof(long long) + 15) & ~(size_t)15;
}

size_t spec_accept_workspace_bytes(int B, int V) { return spec_sums_bytes(B, V) + (size_t)B * sizeof(int32_t); }

hipError_t launch_spec_accept(const SpecAcceptArgs& p, hipStream_t s) {
  SpecArgs a{};  // every field zero/null until set
  a.draft = p.draft_tokens;
  a.q = p.draft_probs;
  a.p = p.target_probs;
  a.u_acc = p.u_accept;
  a.u_smp = p.u_sample;
  a.n_acc = p.n_accepted;
  a.tokens = p.out_tokens;
  a.sums = static_cast<long long*>(p.workspace);
  a.first_rej = reinterpret_cast<int32_t*>(static_cast<char*>(p.workspace) + spec_sums_bytes(p.B, p.V));
  a.B = p.B;
  a.k = p.k;
  a.V = p.V;
  a.nchunk = (p.V + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(spec_chunk_sums, dim3(a.nchunk, p.B), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_pick, dim3(p.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
