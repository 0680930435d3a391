// quant.hip -- amax, scale, per-tensor / blockwise / MX casts and the
// delayed-scaling history update, as gfx950 kernels.
//
// What is computed follows the FP8 quantisation training guide (sections
// "three scaling algorithms", "blockwise scaling", "MXFP8 scaling") and the
// Colossal-AI FP8 story (paragraph on delayed vs real-time scaling); the exact
// rules are restated in include/fp8sg.h.  All of these kernels are bound by
// HBM bandwidth: every element is read once as BF16 (2 B) and written once per
// FP8 copy (1 B); they use 16-byte vector loads, grid-stride loops sized to
// the CU count, and reduce maxima as unsigned magnitude bits (exact and
// order-independent).  A kernel that produces an amax writes one partial
// maximum per workgroup into the caller's workspace and a one-block finalize
// kernel reduces them; same-address device atomics from thousands of
// workgroups serialise (about 10 ns each on MI355X) and would cost more than
// the pass itself.
#include <atomic>
#include <mutex>

#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

namespace {

constexpr int kThreads = 256;


// Streaming kernels walk the tensor in contiguous chunks of 16 KB per
// workgroup (kChunkLoads 16-byte loads per thread in flight), chunk c going to
// workgroup c mod gridDim.x; the last chunk is predicated.
constexpr int kChunkLoads = 4;

// Input element types: BF16 (the activations, gradients and BF16 master
// weights) or FP32 (an FP32 master weight).  Maxima are kept as FP32
// magnitude bits (a BF16 magnitude shifted left by 16), which order like the
// values: NaN > inf > finite.
enum : int { kInBF16 = 0, kInF32 = 1 };

// Largest magnitude (FP32 bits) in one 16-byte vector of either type.
template <int IN>
__device__ __forceinline__ uint32_t vec_absmax(uint4 v) {
  if constexpr (IN == kInBF16) {
    return absmax8(v) << 16;
  } else {
    return max(max(v.x & 0x7fffffffu, v.y & 0x7fffffffu), max(v.z & 0x7fffffffu, v.w & 0x7fffffffu));
  }
}

// amax over n values: nvec 16-byte vectors plus a tail of fewer elements than
// a vector holds.  part[blockIdx.x] = the workgroup's largest magnitude.
template <int IN>
__global__ __launch_bounds__(kThreads) void k_amax(const uint4* __restrict__ x, int64_t nvec,
                                                   const void* __restrict__ tail, int ntail,
                                                   uint32_t* __restrict__ part) {
  __shared__ uint32_t red[kThreads / 64];
  constexpr int U = kChunkLoads;
  uint32_t m = 0;
  const int64_t nchunks = (nvec + kThreads * U - 1) / (kThreads * U);
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int64_t i = c * (kThreads * U) + threadIdx.x;
    if (i + (U - 1) * kThreads < nvec) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_stream(&x[i + u * kThreads]);
#pragma unroll
      for (int u = 0; u < U; ++u) m = max(m, vec_absmax<IN>(v[u]));
    } else {
      for (int u = 0; u < U; ++u)
        if (i + u * kThreads < nvec) m = max(m, vec_absmax<IN>(ld_stream(&x[i + u * kThreads])));
    }
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) {
    if constexpr (IN == kInBF16)
      m = max(m, (uint32_t)(static_cast<const uint16_t*>(tail)[threadIdx.x] & 0x7fffu) << 16);
    else
      m = max(m, static_cast<const uint32_t*>(tail)[threadIdx.x] & 0x7fffffffu);
  }
  m = block_max_u32<kThreads>(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// Reduce n partial maxima (FP32 magnitude bits) to the tensor's amax and,
// where asked, the scale pair derived from it.
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_amax_finalize(const uint32_t* __restrict__ part,
                                                            int n, float* __restrict__ amax,
                                                            float* __restrict__ scale,
                                                            float* __restrict__ scale_inv) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) m = max(m, part[i]);
  m = block_max_u32<kThreads>(m, red);
  if (threadIdx.x == 0) {
    const float a = __uint_as_float(m);
    *amax = a;
    if (scale || scale_inv) {
      const float s = scale_from_amax<FMT>(a);
      if (scale) *scale = s;
      if (scale_inv) *scale_inv = 1.0f / s;
    }
  }
}

// Current scaling inside the cast: every workgroup reduces the amax
// launch's npart partial maxima (FP32 magnitude bits, at most kMaxPartials,
// read from L2) and derives the same scale; workgroup 0 also writes amax,
// scale and scale_inv.  All threads must call it.
template <int FMT, int NT>
__device__ __forceinline__ float scale_from_partials(const uint32_t* __restrict__ part, int npart,
                                                     float* amax, float* scale, float* scale_inv,
                                                     uint32_t* red) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npart; i += NT) m = max(m, part[i]);
  m = block_max_u32<NT>(m, red);
  const float a = __uint_as_float(m);
  const float s = scale_from_amax<FMT>(a);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *amax = a;
    if (scale) *scale = s;
    *scale_inv = 1.0f / s;
  }
  return s;
}

// Where a cast takes its scale from: a device float, or (current scaling)
// the partial maxima of the amax launch just before it.
struct ScaleSrc {
  const float* scale;                 // NULL: current scaling
  const uint32_t* part;
  int npart;
  float* amax;
  float* scale_out;
  float* scale_inv_out;
};

// 16 consecutive elements (16-byte aligned) times s -> 16 FP8 bytes; m takes
// their largest magnitude.  BF16: two 16-byte loads; FP32: four.
template <int FMT, int IN>
struct Row16 {
  static constexpr int V = IN == kInBF16 ? 2 : 4;   // 16-byte vectors per 16 elements
  uint4 v[V];
  __device__ __forceinline__ void load(const void* p) {
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = ld_stream(static_cast<const uint4*>(p) + k);
  }
  __device__ __forceinline__ uint32_t absmax() const {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < V; ++k) m = max(m, vec_absmax<IN>(v[k]));
    return m;
  }
  // the four output words (bytes of elements 4k .. 4k+3 in word k)
  __device__ __forceinline__ void cast(float s, uint32_t (&w)[4]) const {
    if constexpr (IN == kInBF16) {
      const uint2 lo = cast8<FMT>(v[0], s), hi = cast8<FMT>(v[1], s);
      w[0] = lo.x; w[1] = lo.y; w[2] = hi.x; w[3] = hi.y;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = cvt4<FMT>(__uint_as_float(v[k].x) * s, __uint_as_float(v[k].y) * s,
                         __uint_as_float(v[k].z) * s, __uint_as_float(v[k].w) * s);
    }
  }
};

// Per-tensor cast without a transposed copy: a thread casts 16 elements (one
// 16-byte store) per group; n16 = number of 16-element groups; chunks of
// kThreads * 2 groups per workgroup step.
template <int FMT, bool AMAX, int IN>
__global__ __launch_bounds__(kThreads) void k_cast(const uint8_t* __restrict__ x, int64_t n16,
                                                   ScaleSrc src, uint4* __restrict__ q,
                                                   uint32_t* __restrict__ part) {
  __shared__ uint32_t red[kThreads / 64];
  constexpr int U = 2;
  constexpr int64_t GB = 16 * (IN == kInBF16 ? 2 : 4);   // input bytes per group
  const int64_t nchunks = (n16 + kThreads * U - 1) / (kThreads * U);
  // The first chunk's loads go out before the scale is known (with current
  // scaling its reduction would otherwise sit in front of every workgroup).
  Row16<FMT, IN> r[U];
  bool first_loaded = false;
  if ((int64_t)blockIdx.x < nchunks) {
    const int64_t i = (int64_t)blockIdx.x * (kThreads * U) + threadIdx.x;
    if (i + (U - 1) * kThreads < n16) {
#pragma unroll
      for (int u = 0; u < U; ++u) r[u].load(x + (i + u * kThreads) * GB);
      first_loaded = true;
    }
  }
  const float s = src.scale ? *src.scale
                            : scale_from_partials<FMT, kThreads>(src.part, src.npart, src.amax,
                                                                 src.scale_out,
                                                                 src.scale_inv_out, red);
  uint32_t m = 0;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int64_t i = c * (kThreads * U) + threadIdx.x;
    if (i + (U - 1) * kThreads < n16) {
      if (!(first_loaded && c == (int64_t)blockIdx.x)) {
#pragma unroll
        for (int u = 0; u < U; ++u) r[u].load(x + (i + u * kThreads) * GB);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (AMAX) m = max(m, r[u].absmax());
        uint32_t w[4];
        r[u].cast(s, w);
        q[i + u * kThreads] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      for (int u = 0; u < U; ++u) {
        const int64_t j = i + u * kThreads;
        if (j < n16) {
          Row16<FMT, IN> r;
          r.load(x + j * GB);
          if (AMAX) m = max(m, r.absmax());
          uint32_t w[4];
          r.cast(s, w);
          q[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  }
  if (AMAX) {
    m = block_max_u32<kThreads>(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
  }
}

// Current scaling in one launch (BF16 input, no transposed copy), for
// tensors that fit in the registers of a grid small enough to be resident at
// once (occupancy times CUs): each thread loads U 16-byte vectors and keeps
// them; a grid-wide maximum gives every workgroup the tensor's amax, from
// which it derives the scale and casts the vectors it holds.  The input is
// read once instead of twice (amax pass, then cast).
//
// The grid-wide maximum uses device-coherent atomics only (agent-scope
// fences would write back and invalidate whole L2s, which costs more than
// the pass it saves).  Its words live in the caller's workspace after the
// partials, each in a cache line of its own (kLine words), all zero before
// first use.  Workgroups form groups of kGroup; group g has a line with its
// arrival mask (bit i: workgroup kGroup*g + i has arrived) and its maximum,
// and a flag line holding (generation, amax) as one 64-bit word; a top line
// holds the count of complete groups, the grand maximum, the publish and
// rescue claims and the generation of the call.
//   * arrival: a workgroup reads the generation G, atomically maxes its
//     maximum into its group's word and, once that has returned, sets its
//     bit in the group's mask; the group's last arrival moves the group
//     maximum into the top word and counts the group in; the last group's
//     last arrival reads the top word (the amax) and publishes it;
//   * publishing: whoever moves the publish claim from G to G + 1 (a
//     compare-and-swap) writes (G + 1, amax) to every group's flag;
//   * waiting: the others poll their group's flag with relaxed loads until
//     it shows G + 1 (at most kGroup pollers per line, so no memory channel
//     is flooded);
//   * the last arrival then sets the rescue claim to G + 1, clears the
//     masks, maxima and top count, and advances the generation to G + 1.
// No word needs clearing between calls: flags and claims are tagged by the
// generation, and every workgroup reads G before its arrival, hence before
// the last arrival advances it.  A returning atomic has been performed when
// it returns, and each feeds the next through a register dependency, so a
// maximum is in place before its mask bit.  Same-address atomics serialize,
// so a flat counter would cost every arrival in turn; here a chain is at
// most kGroup + kMaxGroups long.
// Rescue.  The wait is bounded: a grid that is not all resident (other work
// holding CUs, such as a second such launch on another stream) would
// otherwise wait for ever.  The first workgroup whose wait runs out moves
// the rescue claim from G to G + 1 and computes the amax without the
// missing workgroups: the group maxima hold every arrived workgroup's
// maximum, and it reads the inputs of the others itself; then it tries the
// publish claim.  If it wins, its reads came before the last arrival's
// claim, hence before the clearing, and its amax is complete; if it loses,
// it takes the last arrival's.  Its waiting peers proceed, finish and
// leave, which lets the missing workgroups run; these find the flag
// published at once.  Other workgroups whose wait ran out wait again, for
// the rescuer.  The first wait's bound is the workspace's config word, or
// kSpinLimit polls (about a millisecond) when that is 0.
constexpr uint32_t kSpinLimit = 1u << 12;
constexpr uint32_t kRescueSpinLimit = 1u << 20;       // the rescuer is running
constexpr int kLine = 32;                             // words per 128-byte line
constexpr int kGroup = 32;                            // workgroups per group (mask bits)
constexpr int kMaxGroups = kMaxPartials / kGroup;     // 64
constexpr uint32_t kNoMax = 0xFFFFFFFFu;              // above any magnitude: the wait ran out
// words of one grid-wide maximum (kGridSetWords); the paired launch uses two
// such sets
static_assert(kGridSetWords == (2 * kMaxGroups + 1) * kLine, "grid-wide maximum words");
static_assert(2 * kGridSetWords <= kGridMaxWords, "grid-wide maximum words");
__device__ __forceinline__ uint32_t* gm_mask(uint32_t* w, int g) { return w + g * kLine; }
__device__ __forceinline__ uint32_t* gm_max(uint32_t* w, int g) { return w + g * kLine + 1; }
__device__ __forceinline__ uint64_t* gm_flag(uint32_t* w, int g) {
  return reinterpret_cast<uint64_t*>(w + (kMaxGroups + g) * kLine);
}
// top line: [0] complete groups, [1] maximum, [2] publish claim, [3] rescue
// claim, [4] generation
__device__ __forceinline__ uint32_t* gm_top(uint32_t* w) { return w + 2 * kMaxGroups * kLine; }
// 0, computed from v in a way the compiler cannot see through: an atomic
// (or address) that takes it waits for v, i.e. for the atomic that produced v.
__device__ __forceinline__ uint32_t after(uint32_t v) {
  uint32_t z;
  asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(v));
  return z;
}
__device__ __forceinline__ uint32_t atomic_max_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_or_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// true if this call moved *p from `from` to from + 1
__device__ __forceinline__ bool claim_agent(uint32_t* p, uint32_t from) {
  uint32_t expected = from;
  return __hip_atomic_compare_exchange_strong(p, &expected, from + 1u, __ATOMIC_RELAXED,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish amax (FP32 magnitude bits) for generation gen + 1 to every group's
// flag, if this call wins the publish claim (thread 0).
__device__ __forceinline__ bool gm_publish(uint32_t* w, uint32_t ngroups, uint32_t gen,
                                           uint32_t amax) {
  if (!claim_agent(gm_top(w) + 2, gen + after(amax))) return false;
  const uint64_t f = ((uint64_t)(gen + 1u) << 32) | amax;
  for (uint32_t i = 0; i < ngroups; ++i)
    __hip_atomic_store(gm_flag(w, (int)i), f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Poll group g's flag up to `limit` times for generation gen + 1: the amax,
// or kNoMax (thread 0).
__device__ __forceinline__ uint32_t gm_wait(uint32_t* w, int g, uint32_t gen, uint32_t limit) {
  for (uint32_t spin = 0; spin < limit; ++spin) {
    const uint64_t f = __hip_atomic_load(gm_flag(w, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(f >> 32) == gen + 1u) return (uint32_t)f;
    __builtin_amdgcn_s_sleep(4);
  }
  return kNoMax;
}

// The largest m over the nblocks workgroups that share the words at w, in
// every one of them, or kNoMax if the wait ran out (then grid_rescue); block
// is the calling workgroup's index among them; cfg[0] bounds the polls (0:
// kSpinLimit).  sh[1] receives the call's generation.  All threads call it;
// thread 0 does the work.
__device__ __forceinline__ uint32_t grid_max(uint32_t* w, const uint32_t* cfg, uint32_t m,
                                             uint32_t block, uint32_t nblocks, uint32_t* sh) {
  if (threadIdx.x == 0) {
    const int g = (int)(block / kGroup);
    const uint32_t ngroups = (nblocks + kGroup - 1) / kGroup;
    const uint32_t gsize = min((uint32_t)kGroup, nblocks - (uint32_t)g * kGroup);
    const uint32_t bit = 1u << (block % kGroup);
    const uint32_t gen = load_agent(gm_top(w) + 4);
    const uint32_t mo = atomic_max_agent(gm_max(w, g), m + after(gen));
    const uint32_t mask = atomic_or_agent(gm_mask(w, g), bit | after(mo)) | bit;
    bool last = false;
    if ((uint32_t)__builtin_popcount(mask) == gsize) {
      const uint32_t gmx = atomic_max_agent(gm_max(w, g), after(mask));
      const uint32_t to = atomic_max_agent(gm_top(w) + 1, gmx);
      last = atomic_add_agent(gm_top(w), 1u + after(to)) + 1 == ngroups;
    }
    uint32_t res;
    if (last) {
      res = atomic_max_agent(gm_top(w) + 1, 0u);
      const uint32_t z = after((uint32_t)gm_publish(w, ngroups, gen, res));
      // after the publish claim: close the rescue claim, clear the arrival
      // words, advance the generation
      store_agent(gm_top(w) + 3, gen + 1u + z);
      for (uint32_t i = 0; i < ngroups; ++i) {
        store_agent(gm_mask(w, (int)i), z);
        store_agent(gm_max(w, (int)i), z);
      }
      store_agent(gm_top(w), z);
      store_agent(gm_top(w) + 1, z);
      store_agent(gm_top(w) + 4, gen + 1u + z);
    } else {
      const uint32_t c = *cfg;
      res = gm_wait(w, g, gen, c != 0 ? c : kSpinLimit);
    }
    sh[0] = res;
    sh[1] = gen;
  }
  __syncthreads();
  const uint32_t r = sh[0];
  __syncthreads();
  return r;
}

// After a wait that ran out (all threads call it; sh[1] holds the call's
// generation): the first such workgroup computes the amax from the group
// maxima (every arrived workgroup's maximum) and the inputs of the
// workgroups that have not arrived, which it reads itself, and publishes it
// unless the last arrival did first; the others wait for the flag.
// share(b, lo, hi) gives workgroup b's range of 16-byte vectors of x; ms is
// two words of LDS.
template <class Share>
__device__ __forceinline__ uint32_t grid_rescue(uint32_t* w, const uint4* x, Share share,
                                                uint32_t block, uint32_t nblocks, uint32_t* ms,
                                                uint32_t* red, uint32_t* sh) {
  const int t = threadIdx.x;
  const int g = (int)(block / kGroup);
  const uint32_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const uint32_t gen = sh[1];
  __syncthreads();
  if (t == 0) sh[0] = claim_agent(gm_top(w) + 3, gen) ? 1u : 0u;
  __syncthreads();
  const bool rescuer = sh[0] != 0u;
  __syncthreads();
  uint32_t a = kNoMax;
  if (rescuer) {
    // group by group: stop if the amax has been published meanwhile (the
    // missing workgroups have arrived), else read the inputs of the group's
    // workgroups that have not arrived yet; a bit read as set was set after
    // that workgroup's maximum was in its group's word, which is read last
    uint32_t m = 0;
    bool done = false;
    for (uint32_t i = 0; i < ngroups && !done; ++i) {
      if (t == 0) {
        const uint32_t gsize = min((uint32_t)kGroup, nblocks - i * kGroup);
        const uint32_t all = gsize == 32u ? 0xFFFFFFFFu : (1u << gsize) - 1u;
        const uint64_t f =
            __hip_atomic_load(gm_flag(w, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ms[0] = (uint32_t)(f >> 32) == gen + 1u ? (uint32_t)f : kNoMax;
        ms[1] = ~load_agent(gm_mask(w, (int)i)) & all;
      }
      __syncthreads();
      const uint32_t f = ms[0];
      uint32_t bits = ms[1];
      __syncthreads();
      if (f != kNoMax) {
        a = f;
        done = true;
      } else {
        while (bits) {
          const uint32_t b = i * kGroup + (uint32_t)(__builtin_ffs((int)bits) - 1);
          bits &= bits - 1u;
          int64_t lo, hi;
          share(b, lo, hi);
          for (int64_t k = lo + t; k < hi; k += kThreads) m = max(m, absmax8(x[k]) << 16);
        }
      }
    }
    if (!done) {
      if ((uint32_t)t < ngroups) m = max(m, load_agent(gm_max(w, t)));
      m = block_max_u32<kThreads>(m, red);
      // a lost claim means the last arrival published first: take its amax
      if (t == 0) sh[0] = gm_publish(w, ngroups, gen, m) ? m : gm_wait(w, g, gen, kRescueSpinLimit);
      __syncthreads();
      a = sh[0];
      __syncthreads();
    }
  } else {
    if (t == 0) sh[0] = gm_wait(w, g, gen, kRescueSpinLimit);
    __syncthreads();
    a = sh[0];
    __syncthreads();
  }
  if (a != kNoMax) return a;
  // the flag did not come (not expected: the rescuer or the last arrival is
  // running): reduce the whole input here, which gives the same value
  int64_t lo, end;
  share(nblocks - 1, lo, end);
  uint32_t m = 0;
  for (int64_t i = t; i < end; i += kThreads) m = max(m, absmax8(x[i]) << 16);
  return block_max_u32<kThreads>(m, red);
}

// One tensor of the paired current-scaling launch.
struct PairTensor {
  const uint4* x;       // BF16 input, 16-byte vectors
  int64_t nvec;
  uint2* q;             // FP8 output, 8 bytes per vector
  uint32_t* gw;         // its grid-wide maximum words
  const uint32_t* cfg;  // the workspace's config word (wait bound)
  float* amax;
  float* scale;
  float* scale_inv;
  uint32_t nblocks;     // its workgroups
};
struct PairArgs {
  PairTensor t[2];
};

// Per-tensor current scaling of one tensor of a pair: as k_amax_cast, with
// each thread holding U vectors in VGPRs and L more in LDS.  The LDS share is
// moved there by LDS DMA (buffer_load ... lds), so it never occupies VGPRs:
// with U = 24, L = 8 four workgroups fit a CU (VGPRs and 128 KB of LDS), so
// 256 CUs hold 67M BF16 values at once (a LLaMA2-7B up-projection's X and W
// together), against 50M with registers alone.  Vector u of thread t is the
// workgroup's vector
// u * kThreads + t, so every load and store instruction covers 4 KB of
// contiguous memory per workgroup.
template <int FMT, int U, int L>
__device__ __forceinline__ void amax_cast_held(const PairTensor& T, uint32_t b,
                                               uint4 (*lv)[kThreads], uint32_t* red,
                                               uint32_t* sh, uint32_t* ms) {
  constexpr int V = U + L;
  const int64_t wg0 = (int64_t)b * (V * kThreads);
  const int nv = (int)min<int64_t>(T.nvec - wg0, (int64_t)V * kThreads);
  const int t = threadIdx.x;
  // LDS share first (vectors U .. V-1): lane i of a wave lands at m0 + 16 i,
  // i.e. at lv[l][t]; reads past the range give zeros
  if constexpr (L > 0) {
    const v4i xr4 = make_rsrc(T.x + wg0, (uint32_t)nv * 16u);
    const uint32_t l0 = lds_addr(&lv[0][t & ~63]);
#pragma unroll
    for (int l = 0; l < L; ++l)
      dma16(xr4, l0 + (uint32_t)(l * kThreads * 16), ((U + l) * kThreads + t) * 16);
  }
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(T.x + wg0), (short)0, nv * 16, 0x00020000);
  const __amdgpu_buffer_rsrc_t qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(T.q + wg0), (short)0, nv * 8, 0x00020000);
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u32x4_t r = __builtin_amdgcn_raw_buffer_load_b128(xr, t * 16, u * kThreads * 16, 0);
    v[u] = make_uint4(r[0], r[1], r[2], r[3]);
  }
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) m = max(m, absmax8(v[u]));
  if constexpr (L > 0) {
    wait_vm<0>();     // the DMA is not tracked by the compiler
    __syncthreads();
#pragma unroll
    for (int l = 0; l < L; ++l) m = max(m, absmax8(lv[l][t]));
  }
  m = block_max_u32<kThreads>(m << 16, red);
  uint32_t a = grid_max(T.gw, T.cfg, m, b, T.nblocks, sh);
  if (a == kNoMax) {
    const int64_t nvec = T.nvec;
    auto share = [nvec](uint32_t blk, int64_t& lo, int64_t& hi) {
      lo = (int64_t)blk * (V * kThreads);
      hi = min<int64_t>(nvec, lo + (int64_t)V * kThreads);
    };
    a = grid_rescue(T.gw, T.x, share, b, T.nblocks, ms, red, sh);
  }
  const float am = __uint_as_float(a);
  const float s = scale_from_amax<FMT>(am);
  if (b == 0 && t == 0) {
    *T.amax = am;
    if (T.scale) *T.scale = s;
    *T.scale_inv = 1.0f / s;
  }
  auto store = [&](uint4 x8, int u) {
    const uint2 c = cast8<FMT>(x8, s);
    u32x2_t w;
    w[0] = c.x;
    w[1] = c.y;
    __builtin_amdgcn_raw_buffer_store_b64(w, qr, t * 8, u * kThreads * 8, 0);
  };
#pragma unroll
  for (int u = 0; u < U; ++u) store(v[u], u);
  if constexpr (L > 0) {
#pragma unroll
    for (int l = 0; l < L; ++l) store(lv[l][t], U + l);
  }
}

// Current scaling of two tensors (a GEMM's two operands) in one launch:
// workgroups 0 .. t[0].nblocks - 1 quantise the first tensor, the others the
// second, each tensor with a grid-wide maximum of its own.  The grid is at
// most what the device holds at once, like k_amax_cast's.
template <int FA, int FB, int U, int L>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void
k_amax_cast_pair(PairArgs a) {
  __shared__ uint32_t red[kThreads / 64];
  __shared__ uint32_t sh[2];
  __shared__ uint32_t ms[2];
  __shared__ __attribute__((aligned(16))) uint4 lv[L][kThreads];
  if (blockIdx.x < a.t[0].nblocks)
    amax_cast_held<FA, U, L>(a.t[0], blockIdx.x, lv, red, sh, ms);
  else
    amax_cast_held<FB, U, L>(a.t[1], blockIdx.x - a.t[0].nblocks, lv, red, sh, ms);
}

// Current scaling in one launch of one tensor: the body above with every
// vector in VGPRs (U = 16 or 24, no LDS share), all workgroups on the tensor.
template <int FMT, int U>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(U >= 24 ? 4 : 1, 8))) void k_amax_cast(
    const uint4* __restrict__ x, int64_t nvec, uint2* __restrict__ q, uint32_t* __restrict__ gw,
    const uint32_t* __restrict__ cfg, float* __restrict__ amax,
    float* __restrict__ scale, float* __restrict__ scale_inv) {
  __shared__ uint32_t red[kThreads / 64];
  __shared__ uint32_t sh[2];
  __shared__ uint32_t ms[2];
  const PairTensor T{x, nvec, q, gw, cfg, amax, scale, scale_inv, gridDim.x};
  amax_cast_held<FMT, U, 0>(T, blockIdx.x, nullptr, red, sh, ms);
}

// 4x4 byte transpose of rows a,b,c,d (one 32-bit word each, byte i = column i)
// into columns: out[i] = bytes (a_i, b_i, c_i, d_i).
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t out[4]) {
  uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);     // a0 b0 c0 d0
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);     // a1 b1 c1 d1
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Per-tensor cast with the transposed copy.  The tensor is cut into tiles of
// 128 rows x 128 columns, visited grid-stride (tile t: row tile t / ntx,
// column tile t % ntx).  In a tile, thread t owns rows 4a .. 4a+3 (a = t / 8)
// and columns 16c .. 16c+15 (c = t % 8):
//   1. two 16-byte loads per row (8 lanes read a row's 256 bytes), the cast,
//      and one 16-byte q store per row (8 lanes write its 128 bytes);
//   2. each 4x4 byte block is transposed in registers, giving for each of the
//      thread's 16 columns the word of rows 4a .. 4a+3, which goes to an LDS
//      copy of the qT tile (128 columns x 32 words, word a of column col at
//      col*32 + (a ^ 4*((col >> 4) & 7)): two lanes per bank at most);
//   3. after a barrier, thread t reads 16 bytes (words 4k .. 4k+3, k = t % 8)
//      of qT rows (t / 8) + 32p, p = 0..3, and stores them: 8 lanes write a
//      qT row's 128 bytes.
// The LDS tile is double-buffered, so one barrier per tile suffices.
// Requires cols % 16 == 0 and rows % 16 == 0 (edge tiles then hold whole
// 16-row / 16-column groups).
__device__ __forceinline__ int qt_word(int col, int a) { return col * 32 + (a ^ (((col >> 4) & 7) << 2)); }

template <int FMT, bool AMAX, int IN>
__global__ __launch_bounds__(kThreads) void k_cast_t(const uint8_t* __restrict__ x, int64_t rows,
                                                     int64_t cols, int64_t ntx, int64_t ntiles,
                                                     ScaleSrc src, uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ qT,
                                                     uint32_t* __restrict__ part) {
  constexpr int64_t EB = IN == kInBF16 ? 2 : 4;   // bytes per input element
  __shared__ uint32_t red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint32_t tile[2][128 * 32];
  const float s = src.scale ? *src.scale
                            : scale_from_partials<FMT, kThreads>(src.part, src.npart, src.amax,
                                                                 src.scale_out,
                                                                 src.scale_inv_out, red);
  const int t = threadIdx.x;
  const int a = t >> 3, c = t & 7;
  uint32_t m = 0;
  int buf = 0;
  for (int64_t tt = blockIdx.x; tt < ntiles; tt += gridDim.x, buf ^= 1) {
    const int64_t r0 = (tt / ntx) * 128, c0 = (tt % ntx) * 128;
    const int rv = (int)min<int64_t>(128, rows - r0), cv = (int)min<int64_t>(128, cols - c0);
    uint32_t* T = tile[buf];
    uint32_t b[4][4];   // [row i][word k] = columns 16c + 4k .. +3 of row 4a + i
    if (4 * a < rv && 16 * c < cv) {
      Row16<FMT, IN> v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i].load(x + ((r0 + 4 * a + i) * cols + c0 + 16 * c) * EB);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (AMAX) m = max(m, v[i].absmax());
        v[i].cast(s, b[i]);
        *reinterpret_cast<uint4*>(q + (r0 + 4 * a + i) * cols + c0 + 16 * c) =
            make_uint4(b[i][0], b[i][1], b[i][2], b[i][3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) b[i][k] = 0;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t col4[4];
      transpose4x4(b[0][k], b[1][k], b[2][k], b[3][k], col4);
#pragma unroll
      for (int i = 0; i < 4; ++i) T[qt_word(16 * c + 4 * k + i, a)] = col4[i];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int col = (t >> 3) + 32 * p, k = t & 7;
      if (col < cv && 16 * k < rv) {
        const uint4 w = *reinterpret_cast<const uint4*>(&T[qt_word(col, 4 * k)]);
        *reinterpret_cast<uint4*>(qT + (c0 + col) * rows + r0 + 16 * k) = w;
      }
    }
  }
  if (AMAX) {
    m = block_max_u32<kThreads>(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
  }
}

// Delayed-scaling step (one block of 256 threads).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_history(float* __restrict__ hist, int hlen,
                                                      int64_t step,
                                                      const float* __restrict__ amax,
                                                      float* __restrict__ scale,
                                                      float* __restrict__ scale_inv) {
  __shared__ uint32_t red[kThreads / 64];
  const int slot = (int)(step % hlen);
  const float a = *amax;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < hlen; i += kThreads) {
    float v = (i == slot) ? a : hist[i];
    m = max(m, __float_as_uint(v) & 0x7fffffffu);
  }
  m = block_max_u32<kThreads>(m, red);
  if (threadIdx.x == 0) {
    hist[slot] = a;
    float s = scale_from_amax<FMT>(__uint_as_float(m));
    *scale = s;
    *scale_inv = 1.0f / s;
  }
}

// Blockwise 1x128: tile t covers the 128 contiguous elements [128t, 128t+128)
// (cols % 128 == 0), handled by 8 lanes with two 16-byte loads each (so one
// wave instruction covers 8 tiles and the per-tile scale division is shared
// by 16 elements per lane); a lane group keeps two tiles' loads in flight.
template <int FMT>
__device__ __forceinline__ void block_1x128_tile(uint4 v0, uint4 v1, int64_t t, int sub,
                                                 uint4* __restrict__ q,
                                                 float* __restrict__ sinv) {
  const uint32_t m = group_max_u32<8>(max(absmax8(v0), absmax8(v1)));
  const float s = scale_from_amax<FMT>(__uint_as_float(m << 16));
  const uint2 lo = cast8<FMT>(v0, s), hi = cast8<FMT>(v1, s);
  q[t * 8 + sub] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  if (sub == 0) sinv[t] = 1.0f / s;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_block_1x128(const uint4* __restrict__ x,
                                                          int64_t ntiles,
                                                          uint4* __restrict__ q,
                                                          float* __restrict__ sinv) {
  constexpr int U = kChunkLoads / 2, G = kThreads / 8;   // G tiles per load step
  const int sub = threadIdx.x & 7;
  const int64_t nchunks = (ntiles + G * U - 1) / (G * U);
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int64_t t = c * (G * U) + (threadIdx.x >> 3);
    if (t + (U - 1) * G < ntiles) {
      uint4 v[U][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u][0] = ld_stream(&x[(t + u * G) * 16 + 2 * sub]);
        v[u][1] = ld_stream(&x[(t + u * G) * 16 + 2 * sub + 1]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) block_1x128_tile<FMT>(v[u][0], v[u][1], t + u * G, sub, q, sinv);
    } else {
      for (int u = 0; u < U; ++u)
        if (t + u * G < ntiles)
          block_1x128_tile<FMT>(ld_stream(&x[(t + u * G) * 16 + 2 * sub]),
                                ld_stream(&x[(t + u * G) * 16 + 2 * sub + 1]), t + u * G, sub,
                                q, sinv);
    }
  }
}

// Blockwise 128x128: one 256-thread block per tile, thread (tr, tc) owns the
// 8x8 sub-block at rows 8*tr.., columns 8*tc.. (rows % 128 == cols % 128 == 0).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_block_128(const uint16_t* __restrict__ x,
                                                        int64_t cols, uint8_t* __restrict__ q,
                                                        float* __restrict__ sinv) {
  __shared__ uint32_t red[kThreads / 64];
  const int tc = threadIdx.x & 15, tr = threadIdx.x >> 4;
  const int64_t r0 = (int64_t)blockIdx.y * 128 + tr * 8;
  const int64_t c0 = (int64_t)blockIdx.x * 128 + tc * 8;
  uint4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = ld_stream((x + (r0 + i) * cols + c0));
    m = max(m, absmax8(v[i]));
  }
  m = block_max_u32<kThreads>(m, red);
  const float s = scale_from_amax<FMT>(__uint_as_float(m << 16));
#pragma unroll
  for (int i = 0; i < 8; ++i) *(uint2*)(q + (r0 + i) * cols + c0) = cast8<FMT>(v[i], s);
  if (threadIdx.x == 0) sinv[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = 1.0f / s;
}

// MX 1x32: block b covers elements [32b, 32b+32) (cols % 32 == 0), handled by
// 4 lanes with one 16-byte load each.  The shared exponent is computed with
// integer operations on the FP32 bits of the block's BF16 amax a:
//   a = (1 + f) * 2^(E-127) with biased exponent E and fraction f; writing
//   fmax = 1.75 * 2^P (P = 8 for E4M3, 15 for E5M2), the smallest integer e
//   with a <= fmax * 2^e is (E - 127) - P when 1 + f <= 1.75 (fraction field
//   <= 0x600000), else one more; clamped to [-127, 127].  Subnormal amax
//   (E = 0) is far below fmax * 2^-127 and gets -127.
template <int FMT>
__device__ __forceinline__ int mx_exponent_bits(uint32_t abits) {
  const int E = (int)(abits >> 23);
  const uint32_t frac = abits & 0x7fffffu;
  int e = (E - 127) - FmtTraits<FMT>::max_exp + (frac > 0x600000u ? 1 : 0);
  if (E == 0) e = -127;
  return min(127, max(-127, e));
}

// Scale 2^-e of an MX block from its BF16 magnitude bits m, and the E8M0
// byte: inf/NaN in the block -> 0xFF (elements cast unscaled), all-zero ->
// 127, else e from mx_exponent_bits.
template <int FMT>
__device__ __forceinline__ float mx_scale(uint32_t m, uint32_t& byte) {
  int e;
  if (m >= 0x7f80u) {
    e = 0;
    byte = 0xffu;
  } else if (m == 0u) {
    e = 0;
    byte = 127u;
  } else {
    e = mx_exponent_bits<FMT>(m << 16);
    byte = (uint32_t)(e + 127);
  }
  return __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, e in [-127, 120]
}

// One 32-element block held by 4 lanes (one 16-byte load each).
template <int FMT>
__device__ __forceinline__ void mx_block(uint4 v, int64_t b, int sub, uint2* __restrict__ q,
                                         uint8_t* __restrict__ e8m0) {
  uint32_t byte;
  const float s = mx_scale<FMT>(group_max_u32<4>(absmax8(v)), byte);
  q[b * 4 + sub] = cast8<FMT>(v, s);
  if (sub == 0) e8m0[b] = (uint8_t)byte;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_mx(const uint4* __restrict__ x, int64_t nblocks,
                                                 uint2* __restrict__ q,
                                                 uint8_t* __restrict__ e8m0) {
  constexpr int U = kChunkLoads, G = kThreads / 4;   // G blocks per load step
  const int sub = threadIdx.x & 3;
  const int64_t nchunks = (nblocks + G * U - 1) / (G * U);
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int64_t b = c * (G * U) + (threadIdx.x >> 2);
    if (b + (U - 1) * G < nblocks) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_stream(&x[(b + u * G) * 4 + sub]);
#pragma unroll
      for (int u = 0; u < U; ++u) mx_block<FMT>(v[u], b + u * G, sub, q, e8m0);
    } else {
      for (int u = 0; u < U; ++u)
        if (b + u * G < nblocks)
          mx_block<FMT>(ld_stream(&x[(b + u * G) * 4 + sub]), b + u * G, sub, q, e8m0);
    }
  }
}

// Quantise with a transposed, column-wise copy, for the backward GEMMs
// (guide, "blockwise scaling": gradients and inputs in 1x128 tiles, weights
// in 128x128 blocks; "MXFP8 scaling": 1x32 blocks).  dgrad contracts over the
// output features and wgrad over the tokens, so besides the row-wise copy
// (q, blocks along the columns) they need qT = the quantisation of x^T, whose
// blocks run along x's rows:
//   kTBlock1   q: 1x128 blocks per row; qT: per column, 128-row blocks
//   kTBlock128 one scale per 128x128 block; qT is the transpose of q
//   kTMX       q: 1x32 E8M0 blocks per row; qT: per column, 32-row blocks
// A 256-thread workgroup handles a 128 x 128 tile; thread t owns the 8 x 8
// block of rows 8r .. 8r+7 (r = t / 16) and columns 8c .. 8c+7 (c = t % 16),
// one 16-byte load per row.  So a wave holds 32 whole rows, a 16-lane row of
// the wave holds 8 whole tile rows (one 1x128 block each), a lane quad 8 rows
// of one 1x32 block, and the 4 lanes c, c+16, c+32, c+48 one 32-row column
// block.  BF16 magnitudes are reduced two at a time (v_pk_max_u16): per
// thread row and column maxima, then row maxima across the quad (MX) or the
// 16-lane row (1x128) with DPP, column maxima across the wave with the
// gfx950 row / half swaps (v_permlane16_swap, v_permlane32_swap), and for
// 128-row column blocks across the 4 waves through LDS.  Each scale is
// computed by one lane and broadcast (DPP in a quad, ds_swizzle in a 16-lane
// row, the swaps across rows), so a thread performs 2-6 scale computations
// instead of 16.  The column-wise cast builds each FP8 word from 4 rows of
// one column, so the transpose itself costs nothing in registers (128x128
// blocks, whose two copies hold the same bytes, transpose q's words 4 x 4
// instead of casting twice).  The 8 bytes (rows 8r .. 8r+7) of each of the
// thread's 8 qT rows go to an LDS tile, from which 8 lanes store each
// 128-byte qT row: stored directly, those 8-byte pieces made the kernel 40 %
// slower.  MX column scales leave the same way, one dword per column.  A wave
// whose elements hold no NaN saturates with the clamp alone.
enum : int { kTBlock1 = 0, kTBlock128 = 1, kTMX = 2 };

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
// Per-half maximum of two pairs of 16-bit magnitudes.
__device__ __forceinline__ uint32_t pmax16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}
// DPP lane move inside rows of 16 lanes (quad_perm / row_ror controls).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;
// Maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (one column block of a wave).
__device__ __forceinline__ uint32_t rows_max(uint32_t v) {
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = pmax16(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return pmax16(b[0], b[1]);
}
// Every lane gets the values x, y of all four 16-lane rows of the wave:
// out[2r] = x of row r, out[2r + 1] = y of row r (row r = lanes 16r .. 16r+15).
__device__ __forceinline__ void rows_gather(float x, float y, float (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t v = __float_as_uint(e ? y : x);
    auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);    // rows 0|2, 1|3
    auto b0 = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);  // rows 0, 2
    auto b1 = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);  // rows 1, 3
    out[0 + e] = __uint_as_float(b0[0]);
    out[4 + e] = __uint_as_float(b0[1]);
    out[2 + e] = __uint_as_float(b1[0]);
    out[6 + e] = __uint_as_float(b1[1]);
  }
}
// out[i] = x of lane i of the lane's 16-lane row, i < 8 (ds_swizzle in
// bitmask mode: source lane = (lane & 0x10) | i within each 32-lane half).
template <int I>
__device__ __forceinline__ float swz_lane(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (I << 5)));
}
__device__ __forceinline__ void row_bcast8(float x, float (&out)[8]) {
  out[0] = swz_lane<0>(x); out[1] = swz_lane<1>(x); out[2] = swz_lane<2>(x); out[3] = swz_lane<3>(x);
  out[4] = swz_lane<4>(x); out[5] = swz_lane<5>(x); out[6] = swz_lane<6>(x); out[7] = swz_lane<7>(x);
}
__device__ __forceinline__ uint32_t pick4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                          int i) {
  const uint32_t lo = (i & 1) ? a1 : a0, hi = (i & 1) ? a3 : a2;
  return (i & 2) ? hi : lo;
}
__device__ __forceinline__ uint32_t word_of(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// LDS copy of a qT tile: 128 qT rows (x's columns) of 32 words; the 8 bytes
// of rows 8r .. 8r+7 of column col are words 2r, 2r+1, stored at
// col*32 + (2r ^ 4*((col >> 3) & 7)), which spreads a wave's 8-byte writes
// over all banks and keeps every aligned group of 4 words whole for the
// 16-byte reads.
__device__ __forceinline__ int qt8_word(int col, int w2) { return col * 32 + (w2 ^ (((col >> 3) & 7) << 2)); }

// The two casts of a thread's 8 x 8 block: row i of q with scale sr[i]
// (skipped when q is null), column j of qT with scale sc[j] into the LDS
// qT tile T.
template <int FMT, bool NANS>
__device__ __forceinline__ void quant_t_emit(const uint4 (&v)[8], const float (&sr)[8],
                                             const float (&sc)[8], uint8_t* qrow, int64_t cols,
                                             uint32_t* T, int tc, int tr) {
  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[i][2 * k] = bf_lo(word_of(v[i], k));
      f[i][2 * k + 1] = bf_hi(word_of(v[i], k));
    }
  if (qrow != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = sr[i];
      *reinterpret_cast<uint2*>(qrow + i * cols) =
          make_uint2(cvt4<FMT, NANS>(f[i][0] * s, f[i][1] * s, f[i][2] * s, f[i][3] * s),
                     cvt4<FMT, NANS>(f[i][4] * s, f[i][5] * s, f[i][6] * s, f[i][7] * s));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float s = sc[j];
    *reinterpret_cast<uint2*>(&T[qt8_word(8 * tc + j, 2 * tr)]) =
        make_uint2(cvt4<FMT, NANS>(f[0][j] * s, f[1][j] * s, f[2][j] * s, f[3][j] * s),
                   cvt4<FMT, NANS>(f[4][j] * s, f[5][j] * s, f[6][j] * s, f[7][j] * s));
  }
}

// The same with one scale for the whole block (128x128 blocks): qT's bytes
// are q's, transposed 4 x 4 bytes at a time in registers.
template <int FMT, bool NANS>
__device__ __forceinline__ void quant_t_emit_uniform(const uint4 (&v)[8], float s, uint8_t* qrow,
                                                     int64_t cols, uint32_t* T, int tc, int tr) {
  uint32_t b[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 r = cast8<FMT, NANS>(v[i], s);
    b[i][0] = r.x;
    b[i][1] = r.y;
    if (qrow != nullptr) *reinterpret_cast<uint2*>(qrow + i * cols) = r;
  }
  uint32_t lo[8], hi[8];   // column j: rows 0..3 in lo[j], rows 4..7 in hi[j]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    transpose4x4(b[0][h], b[1][h], b[2][h], b[3][h], &lo[4 * h]);
    transpose4x4(b[4][h], b[5][h], b[6][h], b[7][h], &hi[4 * h]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint2*>(&T[qt8_word(8 * tc + j, 2 * tr)]) = make_uint2(lo[j], hi[j]);
}

template <int FMT, int KIND>
__global__ __launch_bounds__(kThreads) void k_quant_t(const uint16_t* __restrict__ x,
                                                      int64_t rows, int64_t cols, int64_t ntx,
                                                      int64_t ntiles, uint8_t* __restrict__ q,
                                                      void* __restrict__ sq,
                                                      uint8_t* __restrict__ qT,
                                                      void* __restrict__ sqT) {
  constexpr int RB = KIND == kTMX ? 32 : 128;   // block length along a row / a column
  constexpr uint32_t kMag = 0x7fff7fffu;
  __shared__ uint32_t red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint4 cmax[2][4][16];
  __shared__ __attribute__((aligned(16))) uint32_t tile[2][128 * 32];
  __shared__ uint32_t colb[KIND == kTMX ? 2 : 1][128];   // MX: a column's 4 E8M0 bytes
  __shared__ uint32_t rowb[KIND == kTMX ? 2 : 1][128];   // MX: a row's 4 E8M0 bytes
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int tc = t & 15, tr = t >> 4, qd = lane >> 4;   // qd: the lane's 16-lane row
  const int64_t row_blocks = cols / RB, col_blocks = rows / RB;
  int buf = 0;
  for (int64_t tt = blockIdx.x; tt < ntiles; tt += gridDim.x, buf ^= 1) {
    const int64_t r0 = (tt / ntx) * 128, c0 = (tt % ntx) * 128;
    const int rv = (int)min<int64_t>(128, rows - r0), cv = (int)min<int64_t>(128, cols - c0);
    // rv, cv are multiples of 32 (only MX tiles can be partial): a wave's
    // rows and a quad's columns are valid or invalid together, so the
    // reductions below never mix a valid lane with an invalid one.  Invalid
    // lanes read the tile's first 8 x 8 block instead (in bounds) and store
    // nothing.
    const bool valid = 8 * tr < rv && 8 * tc < cv;
    const int64_t row = r0 + 8 * tr, col = c0 + 8 * tc;
    const uint16_t* src = valid ? x + row * cols + col : x + r0 * cols + c0;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld_stream(src + i * cols);

    // P[i]: row i's magnitude maxima (even, odd columns); C[k]: columns 2k, 2k+1
    uint32_t P[8], C[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a[k] = word_of(v[i], k) & kMag;
        C[k] = i == 0 ? a[k] : pmax16(C[k], a[k]);
      }
      P[i] = pmax16(pmax16(a[0], a[1]), pmax16(a[2], a[3]));
    }
    const uint32_t cl = pmax16(pmax16(C[0], C[1]), pmax16(C[2], C[3]));
    const uint32_t mloc = max(cl & 0xffffu, cl >> 16);
    const bool nan_wave = __builtin_amdgcn_ballot_w64(mloc > 0x7f80u) != 0;

    float sr[8], sc[8];
    if constexpr (KIND == kTBlock128) {
      const uint32_t m = block_max_u32<kThreads>(mloc, red);
      const float st = scale_from_amax<FMT>(__uint_as_float(m << 16));
#pragma unroll
      for (int i = 0; i < 8; ++i) sr[i] = sc[i] = st;
      if (t == 0) {
        const float inv = 1.0f / st;
        if (q != nullptr) static_cast<float*>(sq)[(r0 / 128) * row_blocks + c0 / 128] = inv;
        static_cast<float*>(sqT)[(c0 / 128) * col_blocks + r0 / 128] = inv;
      }
    } else {
      // R[k]: maxima of rows 2k (low half) and 2k+1 (high half)
      uint32_t R[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        R[k] = pmax16(__builtin_amdgcn_perm(P[2 * k + 1], P[2 * k], 0x05040100u),
                      __builtin_amdgcn_perm(P[2 * k + 1], P[2 * k], 0x07060302u));
        R[k] = pmax16(R[k], dpp<kDppXor1>(R[k]));
        R[k] = pmax16(R[k], dpp<kDppXor2>(R[k]));
        if constexpr (KIND == kTBlock1) {
          R[k] = pmax16(R[k], dpp<kDppRor4>(R[k]));
          R[k] = pmax16(R[k], dpp<kDppRor8>(R[k]));
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) C[k] = rows_max(C[k]);   // this wave's 32 rows
      if constexpr (KIND == kTBlock1) {
        if (lane < 16) cmax[buf][w][tc] = make_uint4(C[0], C[1], C[2], C[3]);
        __syncthreads();
        uint4 m4 = cmax[buf][0][tc];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
          const uint4 o = cmax[buf][ww][tc];
          m4 = make_uint4(pmax16(m4.x, o.x), pmax16(m4.y, o.y), pmax16(m4.z, o.z),
                          pmax16(m4.w, o.w));
        }
        C[0] = m4.x; C[1] = m4.y; C[2] = m4.z; C[3] = m4.w;
        // row scales: lane c of a 16-lane row computes tile row 8r + (c & 7)
        const int ri = tc & 7;
        const uint32_t pr = pick4(R[0], R[1], R[2], R[3], ri >> 1);
        const float s = scale_from_amax<FMT>(__uint_as_float(((ri & 1) ? pr >> 16 : pr & 0xffffu) << 16));
        row_bcast8(s, sr);
        if (q != nullptr && valid && tc < 8)
          static_cast<float*>(sq)[(row + tc) * row_blocks + c0 / 128] = 1.0f / s;
        // column scales: lanes of 16-lane row qd compute columns 2qd, 2qd+1
        const uint32_t pc = pick4(C[0], C[1], C[2], C[3], qd);
        const float s0 = scale_from_amax<FMT>(__uint_as_float(pc << 16));
        const float s1 = scale_from_amax<FMT>(__uint_as_float(pc & 0xffff0000u));
        rows_gather(s0, s1, sc);
        if (w == 0 && valid) {
          float* o = static_cast<float*>(sqT) + (col + 2 * qd) * col_blocks + r0 / 128;
          o[0] = 1.0f / s0;
          o[col_blocks] = 1.0f / s1;
        }
      } else {
        // MX rows: lane b of a quad computes rows 2b, 2b+1 of its 32-column block
        const int b = tc & 3;
        const uint32_t pr = pick4(R[0], R[1], R[2], R[3], b);
        uint32_t by0, by1;
        const float s0 = mx_scale<FMT>(pr & 0xffffu, by0), s1 = mx_scale<FMT>(pr >> 16, by1);
        sr[0] = __uint_as_float(dpp<0x00>(__float_as_uint(s0)));
        sr[1] = __uint_as_float(dpp<0x00>(__float_as_uint(s1)));
        sr[2] = __uint_as_float(dpp<0x55>(__float_as_uint(s0)));
        sr[3] = __uint_as_float(dpp<0x55>(__float_as_uint(s1)));
        sr[4] = __uint_as_float(dpp<0xAA>(__float_as_uint(s0)));
        sr[5] = __uint_as_float(dpp<0xAA>(__float_as_uint(s1)));
        sr[6] = __uint_as_float(dpp<0xFF>(__float_as_uint(s0)));
        sr[7] = __uint_as_float(dpp<0xFF>(__float_as_uint(s1)));
        // byte k of rowb[r] is tile row r's scale for column block k; written
        // out after the tile's barrier, one dword per row
        if (valid) {
          uint8_t* rb = reinterpret_cast<uint8_t*>(rowb[buf]) + (8 * tr + 2 * b) * 4 + (tc >> 2);
          rb[0] = (uint8_t)by0;
          rb[4] = (uint8_t)by1;
        }
        // MX columns: lanes of 16-lane row qd compute columns 2qd, 2qd+1
        const uint32_t pc = pick4(C[0], C[1], C[2], C[3], qd);
        uint32_t cb0, cb1;
        const float t0 = mx_scale<FMT>(pc & 0xffffu, cb0), t1 = mx_scale<FMT>(pc >> 16, cb1);
        rows_gather(t0, t1, sc);
        // byte w of colb[c] is column c's scale for this wave's 32 rows;
        // written out after the tile's barrier, one dword per column
        uint8_t* cb = reinterpret_cast<uint8_t*>(colb[buf]) + (8 * tc + 2 * qd) * 4 + w;
        cb[0] = (uint8_t)cb0;
        cb[4] = (uint8_t)cb1;
      }
    }

    uint32_t* T = tile[buf];
    if (valid) {
      uint8_t* qrow = q != nullptr ? q + row * cols + col : nullptr;
      if constexpr (KIND == kTBlock128) {
        if (nan_wave)
          quant_t_emit_uniform<FMT, true>(v, sr[0], qrow, cols, T, tc, tr);
        else
          quant_t_emit_uniform<FMT, false>(v, sr[0], qrow, cols, T, tc, tr);
      } else {
        if (nan_wave)
          quant_t_emit<FMT, true>(v, sr, sc, qrow, cols, T, tc, tr);
        else
          quant_t_emit<FMT, false>(v, sr, sc, qrow, cols, T, tc, tr);
      }
    }
    // qT stores: thread t writes 16 bytes (rows 16k .. 16k+15, k = t % 8) of
    // qT rows t / 8 + 32p, so 8 lanes write a qT row's 128 bytes.  The tile
    // is double-buffered: the next tile's writes go to the other half, and
    // the one after waits for this tile's barrier.
    __syncthreads();
    if constexpr (KIND == kTMX) {
      // column scales: thread c < cv writes column c's bytes for the tile's
      // rv / 32 row blocks, as one dword when they are whole and aligned
      if (t < cv) {
        const uint32_t b4 = colb[buf][t];
        uint8_t* o = static_cast<uint8_t*>(sqT) + (c0 + t) * col_blocks + r0 / 32;
        if (rv == 128 && (col_blocks & 3) == 0) {
          *reinterpret_cast<uint32_t*>(o) = b4;
        } else {
          for (int ww = 0; ww < rv / 32; ++ww) o[ww] = (uint8_t)(b4 >> (8 * ww));
        }
      }
      // row scales likewise: thread 128 + r < 128 + rv writes row r's bytes
      // for the tile's cv / 32 column blocks
      if (q != nullptr && t >= 128 && t - 128 < rv) {
        const int r = t - 128;
        const uint32_t b4 = rowb[buf][r];
        uint8_t* o = static_cast<uint8_t*>(sq) + (r0 + r) * row_blocks + c0 / 32;
        if (cv == 128 && (row_blocks & 3) == 0) {
          *reinterpret_cast<uint32_t*>(o) = b4;
        } else {
          for (int k = 0; k < cv / 32; ++k) o[k] = (uint8_t)(b4 >> (8 * k));
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c = (t >> 3) + 32 * p, k = t & 7;
      if (c < cv && 16 * k < rv)
        *reinterpret_cast<uint4*>(qT + (c0 + c) * rows + r0 + 16 * k) =
            *reinterpret_cast<const uint4*>(&T[qt8_word(c, 4 * k)]);
    }
  }
}

// FP32 -> FP8 codes, 4 per thread, plus a scalar tail in block 0.
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_convert(const float4* __restrict__ x, int64_t n4,
                                                      const float* __restrict__ tail, int ntail,
                                                      uint32_t* __restrict__ q,
                                                      uint8_t* __restrict__ qtail) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 v = x[i];
    q[i] = cvt4<FMT>(v.x, v.y, v.z, v.w);
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail)
    qtail[threadIdx.x] = (uint8_t)(cvt4<FMT>(tail[threadIdx.x], 0.f, 0.f, 0.f) & 0xffu);
}

// Workgroups for a grid-stride launch: enough for the work, at most eight per
// CU and never more than the partial buffer holds.
int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  int64_t cap = (int64_t)device_cu_count() * 8;
  if (cap > kMaxPartials) cap = kMaxPartials;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

// Workspace set-up: every word zero except the config word, which holds the
// grid-wide wait's poll bound.  A fill kernel rather than a memset, so the
// call may be captured in a graph.
__global__ __launch_bounds__(kThreads) void k_workspace_init(uint32_t* __restrict__ ws,
                                                             uint32_t wait_polls) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < kWorkspaceTotalWords;
       i += gridDim.x * kThreads)
    ws[i] = i == kConfigAt ? wait_polls : 0u;
}

hipError_t launch_workspace_init(uint32_t* ws, uint32_t wait_polls, hipStream_t s) {
  hipLaunchKernelGGL(k_workspace_init, dim3(64), dim3(kThreads), 0, s, ws, wait_polls);
  return hipGetLastError();
}

// Static scratch of fp8_quantize_tensor_current_noalloc, for callers that
// cannot allocate: partial maxima, one set of grid-wide maximum words, the
// config word (kScratchWords words, 24.8 KB per device, held until the
// process ends).  Every GPU has its own copy at its own address; host code
// uses only the address hipGetSymbolAddress returns for the current device
// (the symbol's name is a host-side stand-in, not a device address).
static __device__ __align__(256) uint32_t scratch[kScratchWords];
static_assert(kMaxPartials % 32 == 0, "grid words start on a 128-byte line");

__global__ __launch_bounds__(kThreads) void k_zero_words(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0u;
}

hipError_t noalloc_scratch(hipStream_t s, CurrentWs* out) {
  static std::mutex mu;
  static uint32_t* ptr[64];   // per device, set once
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    // the grid-wide maximum's counters, maxima and flags start at zero, and
    // a zero config word selects the default wait bound (static storage
    // starts zeroed; this clears it again on the caller's stream, with a
    // kernel rather than a memset so that a first call may be captured)
    hipLaunchKernelGGL(k_zero_words, dim3(8), dim3(kThreads), 0, s, static_cast<uint32_t*>(p),
                       kScratchWords);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    ptr[dev] = static_cast<uint32_t*>(p);
  }
  uint32_t* w = ptr[dev];
  *out = CurrentWs{w, w + kMaxPartials, w + kMaxPartials + kGridSetWords};
  return hipSuccess;
}

int device_cu_count() {
  static std::atomic<int> cached[64];   // per device; 0 = not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return cached[dev].load(std::memory_order_relaxed);
}

#define FP8SG_FMT_DISPATCH(fmt, ...)                   \
  do {                                                 \
    if ((fmt) == kE4M3) {                              \
      constexpr int F = kE4M3;                         \
      __VA_ARGS__;                                     \
    } else {                                           \
      constexpr int F = kE5M2;                         \
      __VA_ARGS__;                                     \
    }                                                  \
  } while (0)

hipError_t launch_amax(const void* x, int64_t n, int fmt, float* amax, float* scale,
                       float* scale_inv, uint32_t* ws, hipStream_t s, int in) {
  uint32_t* part = ws;
  const int per = in == kInBF16 ? 8 : 4;   // elements per 16-byte vector
  const int64_t nvec = n / per;
  const int ntail = (int)(n - nvec * per);
  const void* tail = static_cast<const uint8_t*>(x) + nvec * 16;
  int g = 1;
  if (n > 0) {
    g = grid_for(nvec > 0 ? nvec : 1, kThreads * kChunkLoads);
    if (in == kInBF16)
      hipLaunchKernelGGL(k_amax<kInBF16>, dim3(g), dim3(kThreads), 0, s,
                         static_cast<const uint4*>(x), nvec, tail, ntail, part);
    else
      hipLaunchKernelGGL(k_amax<kInF32>, dim3(g), dim3(kThreads), 0, s,
                         static_cast<const uint4*>(x), nvec, tail, ntail, part);
  }
  FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_amax_finalize<F>, dim3(1), dim3(kThreads), 0, s,
                                             part, n > 0 ? g : 0, amax, scale, scale_inv));
  return hipGetLastError();
}

// Workgroups of k_cast_t the current device holds at once (at most the
// partial buffer), cached per device: its grid-stride tile loop then runs
// on a grid that is all resident (on the LLaMA2-13B-width X, 2560 tiles:
// 38.0 instead of 39.7 us with a grid of 2048).
template <int IN>
static int cast_t_capacity() {
  static std::atomic<int> cached[64];   // per device; 0 = not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMaxPartials;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_cast_t<kE4M3, true, IN>, kThreads,
                                                     0) != hipSuccess)
      per_cu = 0;
    const int cap = per_cu * device_cu_count();
    cached[dev].store(cap >= 1 && cap <= kMaxPartials ? cap : kMaxPartials,
                      std::memory_order_relaxed);
  }
  return cached[dev].load(std::memory_order_relaxed);
}

template <int IN>
static void cast_kernels(const void* x, int64_t rows, int64_t cols, int fmt, ScaleSrc src,
                         uint8_t* q, uint8_t* qT, uint32_t* part, int& g, hipStream_t s) {
  const int64_t n = rows * cols;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (qT) {
    const int64_t ntx = (cols + 127) / 128;
    const int64_t ntiles = ntx * ((rows + 127) / 128);
    g = grid_for(ntiles, 1);
    const int cap = cast_t_capacity<IN>();
    if (g > cap) g = cap;
    FP8SG_FMT_DISPATCH(fmt, {
      if (part)
        hipLaunchKernelGGL((k_cast_t<F, true, IN>), dim3(g), dim3(kThreads), 0, s, xb, rows, cols,
                           ntx, ntiles, src, q, qT, part);
      else
        hipLaunchKernelGGL((k_cast_t<F, false, IN>), dim3(g), dim3(kThreads), 0, s, xb, rows,
                           cols, ntx, ntiles, src, q, qT, part);
    });
  } else {
    const int64_t n16 = n / 16;
    g = grid_for(n16, kThreads * 2);
    FP8SG_FMT_DISPATCH(fmt, {
      if (part)
        hipLaunchKernelGGL((k_cast<F, true, IN>), dim3(g), dim3(kThreads), 0, s, xb, n16, src,
                           reinterpret_cast<uint4*>(q), part);
      else
        hipLaunchKernelGGL((k_cast<F, false, IN>), dim3(g), dim3(kThreads), 0, s, xb, n16, src,
                           reinterpret_cast<uint4*>(q), part);
    });
  }
}

hipError_t launch_quantize_tensor(const void* x, int64_t rows, int64_t cols, int fmt,
                                  const float* scale, uint8_t* q, uint8_t* qT, float* amax_out,
                                  uint32_t* ws, hipStream_t s, int in) {
  uint32_t* part = amax_out ? ws : nullptr;
  ScaleSrc src{scale, nullptr, 0, nullptr, nullptr, nullptr};
  int g = 0;
  if (rows * cols > 0) {
    if (in == kInBF16)
      cast_kernels<kInBF16>(x, rows, cols, fmt, src, q, qT, part, g, s);
    else
      cast_kernels<kInF32>(x, rows, cols, fmt, src, q, qT, part, g, s);
  }
  if (part)
    FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_amax_finalize<F>, dim3(1), dim3(kThreads), 0, s,
                                               part, g, amax_out, nullptr, nullptr));
  return hipGetLastError();
}

// Current scaling: the amax launch writes partials, the cast reduces them
// itself (no separate finalize launch).
// Largest grid of k_amax_cast<FMT, U> the current device holds at once
// (0 if unknown), cached per device.
template <int FMT, int U>
static int coop_capacity() {
  static std::atomic<int> cached[64];   // per device; 0 = not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_amax_cast<FMT, U>, kThreads, 0) !=
        hipSuccess)
      per_cu = 0;
    cached[dev].store(per_cu > 0 ? per_cu * device_cu_count() : -1, std::memory_order_relaxed);
  }
  const int c = cached[dev].load(std::memory_order_relaxed);
  return c > 0 ? c : 0;
}

// One launch of k_amax_cast<FMT, U> if nvec vectors fit a grid the device
// holds at once (and the partial buffer); *done tells whether it ran.
// (A cooperative launch would guarantee residency but costs this runtime
// far more than the pass it saves; the grid maximum's bounded wait covers
// the rare grid that is not all resident.)
template <int FMT, int U>
static hipError_t try_amax_cast(const void* x, int64_t nvec, uint8_t* q, const CurrentWs& ws,
                                float* amax, float* scale, float* scale_inv, hipStream_t s,
                                bool* done) {
  const int64_t g = (nvec + (int64_t)U * kThreads - 1) / ((int64_t)U * kThreads);
  const int cap = coop_capacity<FMT, U>();
  if (g > cap || g > kMaxPartials) return hipSuccess;
  const uint4* xv = static_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  hipLaunchKernelGGL((k_amax_cast<FMT, U>), dim3((unsigned)g), dim3(kThreads), 0, s, xv, nvec,
                     qv, ws.grid, ws.cfg, amax, scale, scale_inv);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) *done = true;
  return err;
}

hipError_t launch_quantize_current(const void* x, int64_t rows, int64_t cols, int fmt,
                                   uint8_t* q, uint8_t* qT, float* amax, float* scale,
                                   float* scale_inv, const CurrentWs& ws, hipStream_t s, int in) {
  const int64_t n = rows * cols;
  if (n == 0) return launch_amax(x, 0, fmt, amax, scale, scale_inv, ws.part, s, in);
  uint32_t* part = ws.part;
  hipError_t err = hipSuccess;
  // One launch when the tensor fits the registers of a co-resident grid:
  // BF16, whole 16-byte vectors, no transposed copy.
  if (in == kInBF16 && qT == nullptr && n % 8 == 0) {
    bool done = false;
    FP8SG_FMT_DISPATCH(fmt, {
      // 16 vectors per thread (fewer workgroups, a shorter arrival chain; on
      // MI355X up to ~50M elements), then 24
      err = try_amax_cast<F, 16>(x, n / 8, q, ws, amax, scale, scale_inv, s, &done);
      if (err == hipSuccess && !done)
        err = try_amax_cast<F, 24>(x, n / 8, q, ws, amax, scale, scale_inv, s, &done);
    });
    if (err != hipSuccess) return err;
    if (done) return hipSuccess;
  }
  const int per = in == kInBF16 ? 8 : 4;
  const int64_t nvec = n / per;
  const int ntail = (int)(n - nvec * per);
  const void* tail = static_cast<const uint8_t*>(x) + nvec * 16;
  const int ga = grid_for(nvec > 0 ? nvec : 1, kThreads * kChunkLoads);
  if (in == kInBF16)
    hipLaunchKernelGGL(k_amax<kInBF16>, dim3(ga), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), nvec, tail, ntail, part);
  else
    hipLaunchKernelGGL(k_amax<kInF32>, dim3(ga), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), nvec, tail, ntail, part);
  ScaleSrc src{nullptr, part, ga, amax, scale, scale_inv};
  int g = 0;
  if (in == kInBF16)
    cast_kernels<kInBF16>(x, rows, cols, fmt, src, q, qT, nullptr, g, s);
  else
    cast_kernels<kInF32>(x, rows, cols, fmt, src, q, qT, nullptr, g, s);
  return hipGetLastError();
}

// The paired launch: U = 24 vectors per thread in VGPRs, L = 8 in LDS.
constexpr int kPairU = 24, kPairL = 8;

template <int FA, int FB>
static int pair_capacity() {
  static std::atomic<int> cached[64];   // per device; 0 = not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, k_amax_cast_pair<FA, FB, kPairU, kPairL>, kThreads, 0) != hipSuccess)
      per_cu = 0;
    cached[dev].store(per_cu > 0 ? per_cu * device_cu_count() : -1, std::memory_order_relaxed);
  }
  const int c = cached[dev].load(std::memory_order_relaxed);
  return c > 0 ? c : 0;
}

template <int FA, int FB>
static hipError_t try_pair(PairArgs& a, hipStream_t s, bool* done) {
  constexpr int64_t per = (int64_t)(kPairU + kPairL) * kThreads;
  int64_t g[2];
  for (int i = 0; i < 2; ++i) {
    g[i] = (a.t[i].nvec + per - 1) / per;
    if (g[i] > kMaxPartials) return hipSuccess;
    a.t[i].nblocks = (uint32_t)g[i];
  }
  if (g[0] + g[1] > pair_capacity<FA, FB>()) return hipSuccess;
  hipLaunchKernelGGL((k_amax_cast_pair<FA, FB, kPairU, kPairL>), dim3((unsigned)(g[0] + g[1])),
                     dim3(kThreads), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) *done = true;
  return err;
}

hipError_t launch_quantize_pair_current(const CurrentTensor& ta, const CurrentTensor& tb,
                                        uint32_t* ws, hipStream_t s) {
  const int64_t na = ta.rows * ta.cols, nb = tb.rows * tb.cols;
  if (na > 0 && nb > 0) {
    hipError_t err = hipSuccess;
    PairArgs a;
    const CurrentTensor* in[2] = {&ta, &tb};
    for (int i = 0; i < 2; ++i) {
      a.t[i].x = static_cast<const uint4*>(in[i]->x);
      a.t[i].nvec = in[i]->rows * in[i]->cols / 8;
      a.t[i].q = reinterpret_cast<uint2*>(in[i]->q);
      a.t[i].gw = ws + kGridWordsAt + i * kGridSetWords;
      a.t[i].cfg = ws + kConfigAt;
      a.t[i].amax = in[i]->amax;
      a.t[i].scale = in[i]->scale;
      a.t[i].scale_inv = in[i]->scale_inv;
      a.t[i].nblocks = 0;
    }
    bool done = false;
    if (ta.fmt == kE4M3 && tb.fmt == kE4M3)
      err = try_pair<kE4M3, kE4M3>(a, s, &done);
    else if (ta.fmt == kE4M3)
      err = try_pair<kE4M3, kE5M2>(a, s, &done);
    else if (tb.fmt == kE4M3)
      err = try_pair<kE5M2, kE4M3>(a, s, &done);
    else
      err = try_pair<kE5M2, kE5M2>(a, s, &done);
    if (err != hipSuccess || done) return err;
  }
  // an empty tensor, or a pair the device cannot hold at once: one call each
  hipError_t err = launch_quantize_current(ta.x, ta.rows, ta.cols, ta.fmt, ta.q, nullptr, ta.amax,
                                           ta.scale, ta.scale_inv, current_ws(ws), s, kInBF16);
  if (err != hipSuccess) return err;
  return launch_quantize_current(tb.x, tb.rows, tb.cols, tb.fmt, tb.q, nullptr, tb.amax, tb.scale,
                                 tb.scale_inv, current_ws(ws), s, kInBF16);
}

hipError_t launch_amax_finalize(const uint32_t* part, int n, float* amax, hipStream_t s) {
  hipLaunchKernelGGL(k_amax_finalize<kE4M3>, dim3(1), dim3(kThreads), 0, s, part, n, amax,
                     nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_history_update(float* hist, int hlen, int64_t step, const float* amax, int fmt,
                                 float* scale, float* scale_inv, hipStream_t s) {
  FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_history<F>, dim3(1), dim3(kThreads), 0, s, hist,
                                             hlen, step, amax, scale, scale_inv));
  return hipGetLastError();
}

hipError_t launch_quantize_block(const void* x, int64_t rows, int64_t cols, int fmt, int br,
                                 uint8_t* q, float* scale_inv, hipStream_t s) {
  if (rows * cols == 0) return hipSuccess;
  if (br == 1) {
    const int64_t ntiles = rows * (cols / 128);
    // one chunk per workgroup (see launch_quantize_mx)
    const int64_t per = (kThreads / 8) * (kChunkLoads / 2);
    const int64_t nc = (ntiles + per - 1) / per;
    const int g = (int)(nc < ((int64_t)1 << 30) ? nc : ((int64_t)1 << 30));
    FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_block_1x128<F>, dim3(g), dim3(kThreads), 0, s,
                                               static_cast<const uint4*>(x), ntiles,
                                               reinterpret_cast<uint4*>(q), scale_inv));
  } else {
    dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128));
    FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_block_128<F>, grid, dim3(kThreads), 0, s,
                                               static_cast<const uint16_t*>(x), cols, q,
                                               scale_inv));
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                              uint8_t* e8m0, hipStream_t s) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  // one 16 KB chunk per workgroup, the hardware dispatcher balancing them:
  // on the GPT-175B MX weight (604M elements) 301 instead of 337 us with
  // 2048 workgroups walking the chunks (same run)
  const int64_t per = (kThreads / 4) * kChunkLoads;
  const int64_t nc = (nblocks + per - 1) / per;
  const int g = (int)(nc < ((int64_t)1 << 30) ? nc : ((int64_t)1 << 30));
  FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_mx<F>, dim3(g), dim3(kThreads), 0, s,
                                             static_cast<const uint4*>(x), nblocks,
                                             reinterpret_cast<uint2*>(q), e8m0));
  return hipGetLastError();
}

hipError_t launch_quantize_t(const void* x, int64_t rows, int64_t cols, int fmt, int kind,
                             uint8_t* q, void* sq, uint8_t* qT, void* sqT, hipStream_t s) {
  if (rows * cols == 0) return hipSuccess;
  const int64_t ntx = (cols + 127) / 128;
  const int64_t ntiles = ntx * ((rows + 127) / 128);
  // one tile per workgroup, the hardware dispatcher balancing them (on the
  // GPT-175B MX weight's 36864 tiles: 512 instead of 562 us with a grid of
  // 2048 workgroups walking them)
  const int g = (int)(ntiles < (1 << 30) ? ntiles : (1 << 30));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  FP8SG_FMT_DISPATCH(fmt, {
    if (kind == kTBlock1)
      hipLaunchKernelGGL((k_quant_t<F, kTBlock1>), dim3(g), dim3(kThreads), 0, s, xp, rows, cols,
                         ntx, ntiles, q, sq, qT, sqT);
    else if (kind == kTBlock128)
      hipLaunchKernelGGL((k_quant_t<F, kTBlock128>), dim3(g), dim3(kThreads), 0, s, xp, rows,
                         cols, ntx, ntiles, q, sq, qT, sqT);
    else
      hipLaunchKernelGGL((k_quant_t<F, kTMX>), dim3(g), dim3(kThreads), 0, s, xp, rows, cols, ntx,
                         ntiles, q, sq, qT, sqT);
  });
  return hipGetLastError();
}

hipError_t launch_convert(const float* x, int64_t n, int fmt, uint8_t* q, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t n4 = n / 4;
  const int ntail = (int)(n - n4 * 4);
  const int g = grid_for(n4 > 0 ? n4 : 1, kThreads * 4);
  FP8SG_FMT_DISPATCH(fmt, hipLaunchKernelGGL(k_convert<F>, dim3(g), dim3(kThreads), 0, s,
                                             reinterpret_cast<const float4*>(x), n4,
                                             x + n4 * 4, ntail,
                                             reinterpret_cast<uint32_t*>(q), q + n4 * 4));
  return hipGetLastError();
}

}  // namespace fp8sg
