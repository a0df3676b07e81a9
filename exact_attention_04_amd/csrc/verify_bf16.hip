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
// Split kernel -- a fixed grid of kSplitWgs workgroups (one per CU on
// MI355X).  The keys of all (sequence b, KV head g) segments, laid end to
// end, are cut into kSplitWgs equal slices; a workgroup processes its slice,
// i.e. the pieces of the one or few segments that overlap it, and writes one
// partial per piece.  Every CU thus streams the same number of K/V bytes
// whatever the length mix of the batch.  Per piece:
//   * the (H/Hkv)*kq query rows that read KV head g are packed into one
//     32-row tile (two when there are more than 32), so each K/V byte is
//     read from HBM once;
//   * the four waves take interleaved 32-key steps of the piece.  Each wave
//     streams its own steps HBM -> LDS with coalesced 16-byte
//     buffer_load ... lds (one step ahead, two LDS stages per wave), so no
//     wave ever waits for another and a CU keeps 64 KB of loads in flight;
//     the loads are non-temporal, since every cache byte is read once;
//   * S^T = K Q^T and O^T += V^T P^T on the 32x32x16 bf16 MFMA as in the
//     prefill kernel (K as 16-byte LDS reads, V^T via transpose reads), with
//     the same base-2 online softmax, lazily raised reference max and the
//     two denominators (fp32 for LSE, bf16-rounded for O);
//   * the waves' (m, l, O) are combined through LDS into one fp32 partial
//     (O normalised, base-2 LSE) per packed row.
// Piece boundaries inside a segment fall on multiples of 32 keys, so every
// wave step is 32 consecutive keys starting at a multiple of 32.  That lets
// the same kernel read a paged cache ("Warmup Guide", Ch.8: fixed-size
// blocks of tokens, a per-sequence block table from logical to physical
// block): with a page size that is a power of two of at least 16 keys, each
// 16-key half of a step lies inside one page, so the table is consulted once
// per half step and each half's loads use one buffer descriptor, as for the
// contiguous cache (for pages of 32 keys or more both halves name the same
// page).  A wave keeps 64 consecutive table entries of its sequence in a
// VGPR (one per lane) and picks an entry with readlane.  A table entry that
// names no page (outside [0, num_pages)) means its keys do not exist: they
// are masked like keys past the end of the sequence.
// Merge kernel -- one wave per output row combines its segment's piece
// partials (weights exp(LSE_p - LSE)) and writes O (bf16) and LSE (natural
// log).
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

// One workgroup per slice; MI355X has 256 compute units, so the split runs
// in one round on the whole chip (on a partition with fewer units it simply
// takes several).  Four waves share a workgroup's LDS.
constexpr int kSplitWgs = 256;  // slices of the key range (one workgroup each)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;  // keys per wave step
constexpr float kRescaleSlack = 8.0f;  // log2 units

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;  // contiguous: [B][Hkv][cache_stride][D]; paged: [num_pages][Hkv][page][D]
  const uint16_t* v;
  const int32_t* seqlens;
  const int32_t* block_table;  // paged only: [B][max_blocks]
  int max_blocks, num_pages, page_shift;
  const uint32_t* tree_mask;   // [B][kq] ancestor bitmasks of the new tokens, or null (a chain)
  float* part_o;    // [B][Hkv][jmax][R][D]
  float* part_lse;  // [B][Hkv][jmax][R]   base-2 domain: m2 + log2(l)
  int32_t* seg_np;  // [B][Hkv]  pieces of each non-empty segment
  int B, H, Hkv, kq, R, G;
  int max_seqlen, cache_stride, jmax;
  float c2;  // scale * log2(e)
};

__device__ __forceinline__ int clamp_len(int s, int max_len) { return min(max(s, 0), max_len); }

// Work is divided in "cost" units: a key costs 1, and starting a segment
// piece costs kPieceCost more (the pipeline fill, the wave combine and the
// partial write of a piece).  Segment s occupies cost [C_s, C_s + P + L_s):
// its P start-up units, then its L_s keys.  A workgroup that takes the start
// of a second segment thus gets that many fewer keys, and all workgroups
// finish together.
// (512 was measured best over a sweep of 0..1024.)
constexpr int kPieceCost = 512;

// Maximum pieces of one segment: a segment of L keys meets at most
// L / T + 2 slices of length T = ceil(total_cost / kSplitWgs), and
// T >= Hkv * L / kSplitWgs.
__host__ __device__ inline int max_pieces(int Hkv) { return (kSplitWgs + Hkv - 1) / Hkv + 2; }

// Sequence lengths, wave-parallel: lane l holds the clamped length of
// sequence base + l (0 past B).  One vector load instead of a chain of
// dependent scalar loads.
__device__ __forceinline__ int lane_length(const int32_t* seqlens, int B, int max_len, int base) {
  const int b = base + (threadIdx.x & 63);
  return b < B ? clamp_len(seqlens[b], max_len) : 0;
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Total cost over all segments (Hkv segments of length seqlens[b] per
// non-empty sequence; the sum of the lengths is below 2^31, checked on the
// host) and the slice length T = ceil(total_cost / kSplitWgs).
__device__ __forceinline__ void slice_plan(const int32_t* seqlens, int B, int Hkv, int max_len,
                                           long long& total, long long& T) {
  int sum = 0, nonempty = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int x = lane_length(seqlens, B, max_len, b0);
    sum += wave_sum(x);
    nonempty += wave_sum(x > 0 ? 1 : 0);
  }
  total = ((long long)sum + (long long)nonempty * kPieceCost) * Hkv;
  T = (total + kSplitWgs - 1) / kSplitWgs;
}

// NS = 1 or 2 sets of 32 packed query rows: (H/Hkv)*kq <= 32 * NS.  With two
// sets every K and V operand read from LDS feeds one MFMA per set, so the
// cache is still streamed once per KV head.
template <int D, bool PAGED, int NS>
__global__ void __launch_bounds__(kThreads, 1) verify_split_kernel(SplitArgs a) {
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int STEP = kStep * D;              // elements per K (or V) stage
  constexpr int INSN = STEP * 2 / 1024;        // 1 KB HBM->LDS loads per stage
  constexpr int ROWS_PER_INSN = 1024 / (D * 2);
  constexpr int HALF = kStep / 2;              // keys per half step (the smallest page)
  static_assert(NS == 1 || NS == 2, "one or two 32-row query sets");
  static_assert(HALF % ROWS_PER_INSN == 0, "a load instruction stays inside one half step");
  // Per wave: two stages of K and two of V, one LDS object per stage so the
  // compiler can tell the next step's loads from this step's reads.
  __shared__ __attribute__((aligned(1024))) uint16_t k_st0[kWaves][STEP];
  __shared__ __attribute__((aligned(1024))) uint16_t k_st1[kWaves][STEP];
  __shared__ __attribute__((aligned(1024))) uint16_t v_st0[kWaves][STEP];
  __shared__ __attribute__((aligned(1024))) uint16_t v_st1[kWaves][STEP];
  __shared__ float red_m[kWaves][32 * NS];
  __shared__ float red_l[kWaves][32 * NS];
  __shared__ float red_lr[kWaves][32 * NS];

  long long total, T;
  slice_plan(a.seqlens, a.B, a.Hkv, a.max_seqlen, total, T);
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    // empty segments have no piece: record 0 for the merge
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int x = lane_length(a.seqlens, a.B, a.max_seqlen, b0);
      if (b0 + (int)threadIdx.x < a.B && x == 0)
        for (int g = 0; g < a.Hkv; ++g) a.seg_np[(b0 + threadIdx.x) * a.Hkv + g] = 0;
    }
  }
  const long long lo = (long long)blockIdx.x * T;
  const long long hi = min(lo + T, total);
  if (lo >= hi) return;  // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // packed row 32*r + n of set r = (query head g*G + row / kq, new token row % kq)
  bool row_ok[NS];
  int hh[NS], qi[NS];
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    const int row = 32 * r + n;
    row_ok[r] = row < a.R;
    hh[r] = row / a.kq;
    qi[r] = row - hh[r] * a.kq;
  }

  // HBM->LDS: instruction i of a stage covers stage rows
  // [i*ROWS_PER_INSN, +ROWS_PER_INSN); lane l fills row i*ROWS_PER_INSN + l/CPR,
  // chunk position l % CPR with global chunk (position ^ swizzle(row)).
  uint32_t k_voff[INSN], v_voff[INSN];
#pragma unroll
  for (int i = 0; i < INSN; ++i) {
    const int row = i * ROWS_PER_INSN + lane / CPR;
    const int pos = lane % CPR;
    k_voff[i] = (row * D + ((pos ^ k_swz<D>(row)) * 8)) * 2;
    v_voff[i] = (row * D + ((pos ^ v_swz<D>(row)) * 8)) * 2;
  }
  // per-lane LDS byte offsets of the operand reads (see the prefill kernel)
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

  // One piece: keys [k0, k1) of segment (b, g), whose length is sk; the
  // partial goes to slot j of the segment.
  auto piece = [&](int b, int g, int sk, int k0, int k1, int j) {
    // The new tokens' keys are the last kq of the sequence, from nk0 on.  Row
    // qi sees every earlier key and new key nk0 + t iff bit t of its mask is
    // set: the tokens before it for a chain (causal), its ancestors and
    // itself in a draft tree.
    const int nk0 = sk - a.kq;
    uint64_t vis_new[NS];
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      if (a.tree_mask != nullptr)
        vis_new[r] = row_ok[r] ? a.tree_mask[(size_t)b * a.kq + qi[r]] : 0u;
      else
        vis_new[r] = (2ull << qi[r]) - 1ull;  // qi < 64; 2 << 63 wraps to 0 and gives all ones
    }
    const uint16_t* Kb = a.k + (size_t)(b * a.Hkv + g) * a.cache_stride * D;
    const uint16_t* Vb = a.v + (size_t)(b * a.Hkv + g) * a.cache_stride * D;

    u32x4 qf[NS][KS];
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      const uint16_t* qrow = a.q + ((size_t)(b * a.H + g * a.G + hh[r]) * a.kq + qi[r]) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[r][ks] = row_ok[r] ? load16(qrow + ks * 16 + h * 8) : u32x4{0, 0, 0, 0};
    }

    // Paged cache: the wave's window of 64 block-table entries of sequence b
    // (lane i holds logical page win0 + i; -1 past the table).
    int win0 = 0, win = -1;
    auto load_window = [&](int page) {
      wait_vmem_all();  // keeps the counted waits of the step loop exact
      win0 = page;
      const int lp = page + lane;
      win = lp < a.max_blocks ? a.block_table[(size_t)b * a.max_blocks + lp] : -1;
      wait_vmem_all();
    };
    // Which of a stage's 32 keys exist (bit i: key key0 + i).  A key in a
    // block whose table entry names no page does not exist and is masked
    // like a key past the piece; a contiguous cache has every key.
    uint32_t present0 = 0xffffffffu, present1 = 0xffffffffu;
    // A step's buffer starts at its first key and ends at k1 (at most one
    // step): rows past the piece read as zero, and a step past the end reads
    // nothing.  In a paged cache each 16-key half of a step lies inside one
    // page (pages hold a power of two >= 16 keys): its rows are rows
    // key % page.. of physical page table[key / page], through a descriptor
    // of its own whose base sits 16*hf rows before them, so the stage's
    // per-lane offsets stay those of a contiguous step.
    auto issue = [&](int key0, const int ST) {
      const int nk = max(min(k1 - key0, kStep), 0);  // keys of the step inside the piece
      __amdgpu_buffer_rsrc_t kr[2], vr[2];
      uint32_t present = 0xffffffffu;
      if constexpr (PAGED) {
        const int p0 = key0 >> a.page_shift, p1 = (key0 + HALF) >> a.page_shift;
        if (nk > 0 && (p0 < win0 || p1 >= win0 + 64)) load_window(p0);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int key = key0 + HALF * hf;
          const int nh = max(min(nk - HALF * hf, HALF), 0);
          const uint16_t* kbase = a.k;
          const uint16_t* vbase = a.v;
          int bytes = 0;
          if (nh > 0) {
            const int phys = __builtin_amdgcn_readlane(win, (key >> a.page_shift) - win0);
            if ((unsigned)phys < (unsigned)a.num_pages) {
              const size_t row0 = (((size_t)phys * a.Hkv + g) << a.page_shift) + (key & ((1 << a.page_shift) - 1));
              kbase = a.k + (row0 - HALF * hf) * D;
              vbase = a.v + (row0 - HALF * hf) * D;
              bytes = (HALF * hf + nh) * D * 2;
            } else {
              present &= hf ? 0x0000ffffu : 0xffff0000u;
            }
          }
          kr[hf] = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, bytes, kBufferWord3);
          vr[hf] = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, bytes, kBufferWord3);
        }
      } else {
        kr[0] = kr[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(Kb + (size_t)key0 * D), (short)0, nk * D * 2,
                                                          kBufferWord3);
        vr[0] = vr[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(Vb + (size_t)key0 * D), (short)0, nk * D * 2,
                                                          kBufferWord3);
      }
      if (ST)
        present1 = present;
      else
        present0 = present;
      uint16_t* kd = ST ? k_st1[wave] : k_st0[wave];
      uint16_t* vd = ST ? v_st1[wave] : v_st0[wave];
#pragma unroll
      for (int i = 0; i < INSN; ++i) {
        const int hf = i * ROWS_PER_INSN >= HALF;
        buffer_load_lds16_stream(kr[hf], kd + i * 512, k_voff[i]);
        buffer_load_lds16_stream(vr[hf], vd + i * 512, v_voff[i]);
      }
    };

    f32x16 acc_o[NS][NDB];
    float m_ref[NS], l_run[NS], l_rnd[NS];
#pragma unroll
    for (int r = 0; r < NS; ++r) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[r][db] = f32x16{};
      m_ref[r] = -INFINITY;
      l_run[r] = 0.f;
      l_rnd[r] = 0.f;
    }

    auto compute = [&](int key0, const int ST) {
      lds_cchar* kt = (lds_cchar*)(ST ? k_st1[wave] : k_st0[wave]);
      lds_cchar* vt = (lds_cchar*)(ST ? v_st1[wave] : v_st0[wave]);
      const uint32_t present = ST ? present1 : present0;
      f32x16 s[NS];
#pragma unroll
      for (int r = 0; r < NS; ++r) s[r] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kf = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kt + k_off[ks]);
#pragma unroll
        for (int r = 0; r < NS; ++r) s[r] = mfma_32x32x16_bf16(kf, qf[r][ks], s[r]);
      }
      // mask among the new tokens, end of the piece, absent keys: bit i of
      // vis is set iff key key0 + i is visible to this lane's row (every key
      // before nk0, new key nk0 + t iff bit t of vis_new, nothing from k1
      // on, only keys that exist); register r holds key 4h + 8(r/4) + r%4 of
      // the step
      if (key0 + kStep - 1 >= nk0 || key0 + kStep > k1 || present != 0xffffffffu) {
        const int dn = nk0 - key0;  // step position of new key 0
        const int dk = k1 - key0;   // step positions [0, dk) are inside the piece
        const uint32_t old_keys = dn <= 0 ? 0u : (dn >= 32 ? 0xffffffffu : (1u << dn) - 1u);
        const uint32_t in_piece = dk <= 0 ? 0u : (dk >= 32 ? 0xffffffffu : (1u << dk) - 1u);
#pragma unroll
        for (int r = 0; r < NS; ++r) {
          const uint64_t shifted = dn >= 0 ? (vis_new[r] << min(dn, 32)) : (-dn >= 64 ? 0ull : vis_new[r] >> -dn);
          const uint32_t vis = ((old_keys | (uint32_t)shifted) & in_piece & present) >> (4 * h);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            s[r][e] = ((vis >> (8 * (e / 4) + (e % 4))) & 1u) ? s[r][e] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[r][e]);
        mx = max_halves(mx) * a.c2;
        const bool raise = mx > m_ref[r] + kRescaleSlack;
        if (__builtin_expect(__any(raise), 0)) {
          asm volatile("");
          const float alpha = raise ? fast_exp2(m_ref[r] - mx) : 1.f;  // 0 when m_ref = -inf
          m_ref[r] = raise ? mx : m_ref[r];
          l_run[r] *= alpha;
          l_rnd[r] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc_o[r][db][e] *= alpha;
        }
        const float m_use = (m_ref[r] == -INFINITY) ? 0.f : m_ref[r];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[r][e] = fast_exp2(fmaf(s[r][e], a.c2, -m_use));
          l_run[r] += s[r][e];
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 pt[NS];
#pragma unroll
        for (int r = 0; r < NS; ++r)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pt[r][w] = pack_bf16x2(s[r][8 * t + 2 * w], s[r][8 * t + 2 * w + 1]);
            l_rnd[r] = sum_bf16x2(pt[r][w], l_rnd[r]);
          }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          lds_cchar* vb = vt + v_off[db] + 16 * t * D * 2;
          const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vb);
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + 8 * D * 2));
          u32x4 vf;
          vf[0] = __builtin_bit_cast(u32x2, lo4)[0];
          vf[1] = __builtin_bit_cast(u32x2, lo4)[1];
          vf[2] = __builtin_bit_cast(u32x2, hi4)[0];
          vf[3] = __builtin_bit_cast(u32x2, hi4)[1];
#pragma unroll
          for (int r = 0; r < NS; ++r) acc_o[r][db] = mfma_32x32x16_bf16(vf, pt[r], acc_o[r][db]);
        }
      }
    };

    // this wave's steps: key0 = k0 + kStep * (wave + kWaves * i).  Every step
    // issues the next step's loads (past the end with an empty buffer: zeros
    // land in the idle stage) so the loop has no branch and the counted wait
    // is exact.
    const int first = k0 + kStep * wave;
    const int nsteps = first < k1 ? (k1 - first + kStep * kWaves - 1) / (kStep * kWaves) : 0;
    if (PAGED && nsteps > 0) load_window(first >> a.page_shift);
    auto step = [&](int i, const int ST) {
      const int key0 = first + kStep * kWaves * i;
      issue(key0 + kStep * kWaves, ST ^ 1);
      wait_vmem_at_most<2 * INSN>();  // this step's loads landed, the next step's may fly
      compute(key0, ST);
    };
    if (nsteps > 0) issue(first, 0);
    for (int i = 0; i < nsteps; i += 2) {
      step(i, 0);
      if (i + 1 < nsteps) step(i + 1, 1);
    }
    wait_vmem_all();  // the last (empty) loads are done before the stages are reused

    // ---- combine the waves through LDS.  Each wave parks its fp32
    // accumulator of set r, [D][32], in two of its own stages (set 0 in the
    // K stages, set 1 in the V stages; head dims < D/2 in the first, the
    // rest in the second); no other wave touches them before the barrier.
    auto red_at = [&](int w, int r, int d) -> float* {
      uint16_t* st = r == 0 ? (d < D / 2 ? k_st0[w] : k_st1[w]) : (d < D / 2 ? v_st0[w] : v_st1[w]);
      return reinterpret_cast<float*>(st) + (d % (D / 2)) * 32;
    };
    static_assert(STEP * 2 >= (D / 2) * 32 * 4, "a stage holds half of a wave's accumulator of one set");
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      const float l_tot = sum_halves(l_run[r]);
      const float lr_tot = sum_halves(l_rnd[r]);
      if (h == 0) {
        red_m[wave][32 * r + n] = m_ref[r];
        red_l[wave][32 * r + n] = l_tot;
        red_lr[wave][32 * r + n] = lr_tot;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int d = 32 * db + 8 * (e / 4) + 4 * h + (e % 4);
          red_at(wave, r, d)[n] = acc_o[r][db][e];
        }
    }
    __syncthreads();
    {
      constexpr int ROWS = 32 * NS;
      const int rn = tid % ROWS;  // packed row
      const int rs = rn / 32, rl = rn % 32;
      const int dg = tid / ROWS;  // group of DPT head dims
      constexpr int DPT = D / (kThreads / ROWS);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][rn]);
      const float M_use = (M == -INFINITY) ? 0.f : M;
      float f[kWaves];
      float L = 0.f, LR = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        f[w] = fast_exp2(red_m[w][rn] - M_use);
        L += f[w] * red_l[w][rn];
        LR += f[w] * red_lr[w][rn];
      }
      if (rn < a.R) {
        const size_t pidx = ((size_t)(b * a.Hkv + g) * a.jmax + j) * a.R + rn;
        const float inv = LR > 0.f ? 1.f / LR : 0.f;
        float* dst = a.part_o + pidx * D + dg * DPT;
#pragma unroll
        for (int d4 = 0; d4 < DPT; d4 += 4) {
          f32x4 vv;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) acc = fmaf(f[w], red_at(w, rs, dg * DPT + d4 + u)[rl], acc);
            vv[u] = acc * inv;
          }
          *reinterpret_cast<f32x4*>(dst + d4) = vv;
        }
        if (dg == 0) a.part_lse[pidx] = L > 0.f ? M + fast_log2(L) : -INFINITY;
      }
    }
    __syncthreads();  // the stages and red_* are free for the next piece
  };

  // Walk the segments overlapping this workgroup's cost slice [lo, hi)
  // (sequence-major, then KV head).
  long long seq0 = 0;  // cost start of sequence b's Hkv segments
  for (int b0 = 0; b0 < a.B && seq0 < hi; b0 += 64) {
    const int len_l = lane_length(a.seqlens, a.B, a.max_seqlen, b0);
    for (int bi = 0; bi < 64 && b0 + bi < a.B && seq0 < hi; ++bi) {
      const int b = b0 + bi;
      const int sk = __builtin_amdgcn_readlane(len_l, bi);
      if (sk == 0) continue;
      const long long seg = (long long)kPieceCost + sk;  // cost of one segment
      if (seq0 + seg * a.Hkv > lo) {
        for (int g = 0; g < a.Hkv; ++g) {
          const long long c0 = seq0 + (long long)g * seg + kPieceCost;  // cost of key 0
          const long long k0 = max(lo - c0, 0LL), k1 = min(hi - c0, (long long)sk);
          if (k0 < k1) {
            const int j = (int)((c0 + k0) / T - c0 / T);
            if (j == 0 && tid == 0) a.seg_np[b * a.Hkv + g] = (int)(1 + (c0 + sk - 1) / T - c0 / T);
            // boundaries between pieces move down to a multiple of 32 (the
            // neighbouring piece rounds the same boundary the same way); a
            // piece left empty still writes its (empty) partial
            const int k0r = (int)k0 & ~(kStep - 1);
            const int k1r = k1 == sk ? sk : ((int)k1 & ~(kStep - 1));
            piece(b, g, sk, k0r, k1r, j);
          }
        }
      }
      seq0 += seg * a.Hkv;
    }
  }
}

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* seg_np;
  const int32_t* seqlens;
  uint16_t* o;
  float* lse;
  int B, H, Hkv, kq, R, G;
  int max_seqlen, jmax;
};

// One wave per (b, query head, new token).  The split kernel recorded how
// many pieces the row's segment has; the wave loads that count, one piece LSE
// per lane and eight piece outputs at once, reduces the LSEs and accumulates
// its head dims with the broadcast weights exp2(LSE_p - LSE) (segments of
// more than eight pieces take further rounds of loads).
template <int D>
__global__ void __launch_bounds__(256) verify_merge_kernel(MergeArgs a) {
  constexpr int EPL = D / 64;  // head dims per lane
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int total = a.B * a.H * a.kq;
  if (row >= total) return;
  const int qi = row % a.kq;
  const int hq = (row / a.kq) % a.H;
  const int b = row / (a.kq * a.H);
  const int g = hq / a.G, hh = hq - g * a.G;
  const int rn = hh * a.kq + qi;
  // pieces of the row's segment (0 for an empty one; nothing was written
  // when the split kernel did not run).  The first piece LSE per lane and
  // the first eight piece outputs are loaded before the count, so the common
  // case costs one memory round trip; slots at or past the count (stale or
  // never written) are loaded but never used.
  const size_t base = (size_t)(b * a.Hkv + g) * a.jmax;
  const float lse_raw = a.part_lse[(base + min(lane, a.jmax - 1)) * a.R + rn];
  float v[8][EPL];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float* src = a.part_o + ((base + min(k, a.jmax - 1)) * a.R + rn) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[k][e] = src[e];
  }
  const int np_raw = a.max_seqlen > 0 ? a.seg_np[b * a.Hkv + g] : 0;
  const int nc = min(np_raw, a.jmax);
  // the largest piece LSE: the first 64 pieces from the values loaded
  // above, any others in further rounds
  float M = lane < nc ? lse_raw : -INFINITY;
  for (int c0 = 64; c0 < nc; c0 += 64)
    M = fmaxf(M, (c0 + lane < nc) ? a.part_lse[(base + c0 + lane) * a.R + rn] : -INFINITY);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float L = 0.f;
  // pieces in rounds of 64 (one weight per lane), eight outputs at a time;
  // the first eight are the ones loaded above
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const float x = c0 == 0 ? lse_raw : ((c0 + lane < nc) ? a.part_lse[(base + c0 + lane) * a.R + rn] : -INFINITY);
    const float w = (c0 + lane < nc) ? fast_exp2(x - M_use) : 0.f;
    L += w;
    const int cn = min(64, nc - c0);
    for (int k0 = 0; k0 < cn; k0 += 8) {
      if (c0 + k0 > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int kk = c0 + min(k0 + k, cn - 1);
          const float* src = a.part_o + ((base + kk) * a.R + rn) * D + lane * EPL;
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[k][e] = src[e];
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float wk = __shfl(w, min(k0 + k, 63), 64);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = k0 + k < cn ? fmaf(wk, v[k][e], acc[e]) : acc[e];
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
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

template <int D, bool PAGED, int NS>
hipError_t launch(const VerifyArgs& p, hipStream_t s) {
  const int G = p.H / p.Hkv;
  const int R = G * p.kq;
  const int jmax = max_pieces(p.Hkv);
  const size_t n_parts = (size_t)p.B * p.Hkv * jmax * R;
  char* ws = static_cast<char*>(p.workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + align_up(n_parts * D * 4));
  int32_t* seg_np = reinterpret_cast<int32_t*>(ws + align_up(n_parts * D * 4) + align_up(n_parts * 4));

  SplitArgs sa{};  // every field zero/null until set
  sa.q = static_cast<const uint16_t*>(p.q);
  sa.k = static_cast<const uint16_t*>(p.k);
  sa.v = static_cast<const uint16_t*>(p.v);
  sa.seqlens = p.seqlens;
  sa.block_table = p.block_table;
  sa.max_blocks = p.max_blocks;
  sa.num_pages = p.num_pages;
  sa.page_shift = p.page_shift;
  sa.tree_mask = p.tree_mask;
  sa.part_o = part_o;
  sa.part_lse = part_lse;
  sa.seg_np = seg_np;
  sa.B = p.B;
  sa.H = p.H;
  sa.Hkv = p.Hkv;
  sa.kq = p.kq;
  sa.R = R;
  sa.G = G;
  sa.max_seqlen = p.max_seqlen_k;
  sa.cache_stride = p.cache_stride;
  sa.jmax = jmax;
  sa.c2 = p.scale * kLog2e;
  if (p.max_seqlen_k > 0) {
    hipLaunchKernelGGL((verify_split_kernel<D, PAGED, NS>), dim3(kSplitWgs), dim3(kThreads), 0, s, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  MergeArgs ma{};  // every field zero/null until set
  ma.part_o = part_o;
  ma.part_lse = part_lse;
  ma.seg_np = seg_np;
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
  ma.jmax = jmax;
  const int rows = p.B * p.H * p.kq;
  hipLaunchKernelGGL((verify_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, s, ma);
  return hipGetLastError();
}

// ---- the allocation-free variant.  Its partials live in a file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy (at its own address) until the process ends; in host
// code the array's name is not a device address, so its address on the
// current device is looked up once per device with hipGetSymbolAddress and
// only that pointer is ever handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // on the current device
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

size_t verify_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t launch_verify_bf16_noalloc(const VerifyArgs& p, hipStream_t s) {
  // The split kernel writes every partial slot and piece count the merge
  // reads in the same call, so the scratch needs no clearing between calls.
  VerifyArgs a = p;
  hipError_t e = scratch_address(&a.workspace);
  if (e != hipSuccess) return e;
  return launch_verify_bf16(a, s);
}

int verify_split_workgroups() { return kSplitWgs; }

size_t verify_workspace_bytes(int B, int H, int Hkv, int kq, int d) {
  // fp32 O and LSE partials for every (sequence, query head, token, piece
  // slot), and the piece count of every (sequence, KV head) segment
  const size_t n_parts = (size_t)B * H * kq * max_pieces(Hkv);
  return align_up(n_parts * d * 4) + align_up(n_parts * 4) + align_up((size_t)B * Hkv * 4);
}

template <int D, bool PAGED>
hipError_t launch_sets(const VerifyArgs& p, hipStream_t s) {
  // one 32-row query set when the packed rows fit, two otherwise
  return (p.H / p.Hkv) * p.kq <= 32 ? launch<D, PAGED, 1>(p, s) : launch<D, PAGED, 2>(p, s);
}

hipError_t launch_verify_bf16(const VerifyArgs& p, hipStream_t s) {
  if (p.paged) return p.d == 128 ? launch_sets<128, true>(p, s) : launch_sets<64, true>(p, s);
  return p.d == 128 ? launch_sets<128, false>(p, s) : launch_sets<64, false>(p, s);
}

}  // namespace attn
