// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   * A operand (32 x 16): lane l holds row m = l % 32, eight k values
//     selected by the lane half h = l / 32;
//   * B operand (16 x 32): lane l holds column n = l % 32, the eight k values
//     of the same half h;
//   * C/D (32 x 32 fp32, 16 registers): register r of lane l holds
//     row 8*(r/4) + 4*h + r%4, column l % 32.
// A and B always map (half, item) to the contraction index the same way, so
// the order of the contraction inside one instruction never matters.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even fp32 -> bf16 of two values, packed lo | hi << 16
// (the compiler emits v_cvt_pk_bf16_f32 for this).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// c + lo + hi of a packed bf16 pair, exact products, fp32 accumulation
// (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, c, false);
}

// Low 16-bit halves of a and b packed as (a.lo, b.lo); high halves likewise.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Value of lane (l ^ 32) -- the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, swap_halves(x)); }
__device__ __forceinline__ float sum_halves(float x) { return x + swap_halves(x); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor flags (gfx9 family)

// 16-byte chunk positions inside an LDS row (XOR swizzles).  K: the 32 rows
// an A-operand read touches spread over all banks.  V: the 8 rows x 64 bytes
// a transpose read touches spread over all banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// 16 bytes per lane from a raw buffer straight into LDS: lane l writes
// lds_wave_base + 16*l (buffer_load_dwordx4 ... lds).  Out-of-range offsets
// read as zero.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint16_t* lds_wave_base,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, voffset, 0, 0, 0);
}

// The same for data read exactly once (a KV cache streamed by the verify
// kernel): the non-temporal hint keeps the lines from displacing what the
// caches hold, which measured 15% faster on a 414 MB stream.
__device__ __forceinline__ void buffer_load_lds16_stream(__amdgpu_buffer_rsrc_t r, uint16_t* lds_wave_base,
                                                         uint32_t voffset) {
  constexpr int kNonTemporal = 2;  // cache-policy operand: NT
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, voffset, 0, 0, kNonTemporal);
}

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0), other counters untouched
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations
// (including HBM->LDS loads) still outstanding; other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// A wave-uniform value the compiler cannot prove uniform, moved to scalar
// registers (buffer descriptors built from it then need no per-lane loop).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Scheduling pipeline of a matrix phase: KM MFMAs that take one LDS
// operand read each (16-byte row reads) and VM MFMAs that take two
// (transpose reads), the one-read group first unless TWO_FIRST, every read
// issued L MFMAs ahead of the MFMA that consumes it, so LDS latency hides
// behind matrix work.  The reads and MFMAs must appear in that order in
// the code the phase is built from.
template <int KM, int VM, bool TWO_FIRST>
__device__ constexpr int reads_needed(int i) {  // reads consumed by MFMAs 0..i
  if constexpr (TWO_FIRST) return i < VM ? 2 * (i + 1) : 2 * VM + (i - VM + 1);
  return i < KM ? i + 1 : KM + 2 * (i - KM + 1);
}
template <int I, int KM, int VM, int L, bool TWO_FIRST = false>
__device__ __forceinline__ void matrix_pipeline() {
  if constexpr (I < KM + VM) {
    constexpr int last = KM + VM - 1;
    constexpr int hi = I + L < last ? I + L : last;
    constexpr int lo = I == 0 ? 0
                              : (I - 1 + L < last ? reads_needed<KM, VM, TWO_FIRST>(I - 1 + L)
                                                  : reads_needed<KM, VM, TWO_FIRST>(last));
    constexpr int n = reads_needed<KM, VM, TWO_FIRST>(hi) - lo;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // one MFMA
    matrix_pipeline<I + 1, KM, VM, L, TWO_FIRST>();
  }
}

// Workgroup index remapped so that the workgroups the hardware sends to one
// XCD (dispatch is round-robin over the 8 XCDs) get consecutive logical ids:
// neighbouring tiles of one head then share that XCD's L2.
__device__ __forceinline__ int xcd_grouped_block(int bid, int nblocks) {
  constexpr int kXcds = 8;
  if (nblocks % kXcds != 0) return bid;
  return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

// One claim from a dynamic-tail counter (tail_pool.h) by the whole
// workgroup; every thread must call it (it synchronises the workgroup).
// Returns the claim's index.  Exactly nclaim workgroups claim from a counter
// in one call, so the one that draws index nclaim - 1 is the last, and it
// returns the counter to zero for the next call that uses it.
__device__ __forceinline__ int claim_tail_block(unsigned* counter, int nclaim) {
  __shared__ int s_claim;
  if (threadIdx.x == 0) {
    const unsigned c = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c == (unsigned)nclaim - 1u) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_claim = (int)c;
  }
  __syncthreads();
  return s_claim;
}

// Order of causal work split into units (heads) of nper blocks each, block
// 0 of a unit the heaviest; returns unit * nper + block.  Workgroup i runs
// on XCD i % 8, and each XCD hands its ids, in order, to its four shader
// engines in turn, waiting for a free CU on the next engine of that rotation
// even while another engine has one.  Unless the engines receive equal work
// they fall out of step and CUs idle between workgroups (9 us per workgroup
// measured with one head at a time, heaviest block first, at B4 H32 S8192).
// So with `paired`, an XCD runs its heads two at a time in groups of four
// ids: blocks 2k and 2k+1 of both heads, the heavier pair first in even
// groups and last in odd ones.  Over any two groups every engine then gets
// the same work, and the two heads' blocks still share the XCD's L2.
// Otherwise one head at a time.  Either way each XCD gets a contiguous range
// of heads.
__device__ __forceinline__ int causal_block_order(int bid, int nblocks, int nper, bool paired) {
  constexpr int kXcds = 8;
  const int nunits = nblocks / nper;
  if (paired && nunits % (2 * kXcds) == 0 && nper % 2 == 0) {
    const int x = bid % kXcds, i = bid / kXcds, hx = nunits / kXcds;
    const int pr = i / (2 * nper), r = i - pr * 2 * nper;  // head pair, position within its 2*nper ids
    const int grp = r / 4;
    const int j = ((r & 3) + ((grp & 1) ? 2 : 0)) & 3;    // odd groups: lighter pair first
    return (x * hx + 2 * pr + (j & 1)) * nper + 2 * grp + (j >> 1);
  }
  return xcd_grouped_block(bid, nblocks);
}

}  // namespace attn
