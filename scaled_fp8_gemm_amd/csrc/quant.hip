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
// maximum per workgroup into a small per-stream workspace and a one-block
// finalize kernel reduces them; same-address device atomics from thousands of
// workgroups serialise (about 10 ns each on MI355X) and would cost more than
// the pass itself.
#include <mutex>
#include <vector>

#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

namespace {

constexpr int kThreads = 256;

// Workgroups of a partial-producing launch (the partial buffer's length).
constexpr int kMaxPartials = 2048;

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
// A 256-thread workgroup handles a 128 x 128 tile as k_cast_t does (thread t:
// rows 4a .. 4a+3, a = t / 8, columns 16c .. 16c+15, c = t % 8): row maxima
// reduce over the 8 lanes of a row (1x128) or 2 lanes (1x32); column maxima
// over the thread's 4 rows, then over the 8 lanes of a column in the wave
// (32 rows: one MX block), then across the 4 waves through LDS (128 rows).
// The column-scaled bytes go through the LDS transpose of k_cast_t.
enum : int { kTBlock1 = 0, kTBlock128 = 1, kTMX = 2 };

// Element j (0..15) of a thread's row held as two 16-byte loads.
__device__ __forceinline__ float row_elem(const uint4 (&v)[2], int j) {
  const uint4 h = v[j >> 3];
  const int wd = (j & 7) >> 1;
  const uint32_t w = wd == 0 ? h.x : wd == 1 ? h.y : wd == 2 ? h.z : h.w;
  return (j & 1) ? bf_hi(w) : bf_lo(w);
}
__device__ __forceinline__ uint32_t row_mag(const uint4 (&v)[2], int j) {
  const uint4 h = v[j >> 3];
  const int wd = (j & 7) >> 1;
  const uint32_t w = wd == 0 ? h.x : wd == 1 ? h.y : wd == 2 ? h.z : h.w;
  return ((j & 1) ? (w >> 16) : w) & 0x7fffu;
}

template <int FMT, int KIND>
__global__ __launch_bounds__(kThreads) void k_quant_t(const uint16_t* __restrict__ x,
                                                      int64_t rows, int64_t cols, int64_t ntx,
                                                      int64_t ntiles, uint8_t* __restrict__ q,
                                                      void* __restrict__ sq,
                                                      uint8_t* __restrict__ qT,
                                                      void* __restrict__ sqT) {
  constexpr int RB = KIND == kTMX ? 32 : 128;   // block length along a row / a column
  __shared__ uint32_t red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint32_t tile[2][128 * 32];
  __shared__ __attribute__((aligned(16))) uint32_t cmax[KIND == kTBlock1 ? 2 : 1][4][128];
  const int t = threadIdx.x;
  const int a = t >> 3, c = t & 7, w = t >> 6, lane = t & 63;
  const int64_t row_blocks = cols / RB, col_blocks = rows / RB;
  int buf = 0;
  for (int64_t tt = blockIdx.x; tt < ntiles; tt += gridDim.x, buf ^= 1) {
    const int64_t r0 = (tt / ntx) * 128, c0 = (tt % ntx) * 128;
    const int rv = (int)min<int64_t>(128, rows - r0), cv = (int)min<int64_t>(128, cols - c0);
    const bool valid = 4 * a < rv && 16 * c < cv;
    uint4 v[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (valid) {
        const uint16_t* src = x + (r0 + 4 * a + i) * cols + c0 + 16 * c;
        v[i][0] = ld_stream(src);
        v[i][1] = ld_stream(src + 8);
      } else {
        v[i][0] = v[i][1] = make_uint4(0, 0, 0, 0);
      }
    }
    uint32_t rm[4], cm[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) rm[i] = max(absmax8(v[i][0]), absmax8(v[i][1]));
#pragma unroll
    for (int j = 0; j < 16; ++j)
      cm[j] = max(max(row_mag(v[0], j), row_mag(v[1], j)), max(row_mag(v[2], j), row_mag(v[3], j)));

    // ---- row-wise copy
    float st = 1.0f;   // kTBlock128: the tile's scale (rows and columns alike)
    if constexpr (KIND == kTBlock128) {
      const uint32_t m = block_max_u32<kThreads>(max(max(rm[0], rm[1]), max(rm[2], rm[3])), red);
      st = scale_from_amax<FMT>(__uint_as_float(m << 16));
    }
    if (q != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sr;
        uint32_t byte = 0;
        if constexpr (KIND == kTBlock1) sr = scale_from_amax<FMT>(__uint_as_float(group_max_u32<8>(rm[i]) << 16));
        else if constexpr (KIND == kTMX) sr = mx_scale<FMT>(group_max_u32<2>(rm[i]), byte);
        else sr = st;
        if (valid) {
          const uint2 lo = cast8<FMT>(v[i][0], sr), hi = cast8<FMT>(v[i][1], sr);
          const int64_t row = r0 + 4 * a + i;
          *reinterpret_cast<uint4*>(q + row * cols + c0 + 16 * c) = make_uint4(lo.x, lo.y, hi.x, hi.y);
          if constexpr (KIND == kTBlock1) {
            if (c == 0) static_cast<float*>(sq)[row * row_blocks + c0 / 128] = 1.0f / sr;
          } else if constexpr (KIND == kTMX) {
            if ((c & 1) == 0) static_cast<uint8_t*>(sq)[row * row_blocks + (c0 + 16 * c) / 32] = (uint8_t)byte;
          }
        }
      }
      if constexpr (KIND == kTBlock128)
        if (t == 0) static_cast<float*>(sq)[(r0 / 128) * row_blocks + c0 / 128] = 1.0f / st;
    }

    // ---- column scales
    float sc[16];
    uint32_t cbyte[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (KIND == kTBlock128) {
        sc[j] = st;
      } else {
        uint32_t m = cm[j];
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
        if constexpr (KIND == kTMX) {
          sc[j] = mx_scale<FMT>(m, cbyte[j]);
        } else {
          cm[j] = m;   // this wave's 32 rows
        }
      }
    }
    if constexpr (KIND == kTBlock1) {
      if (lane < 8) {
#pragma unroll
        for (int j = 0; j < 16; j += 4)
          *reinterpret_cast<uint4*>(&cmax[buf][w][16 * c + j]) = make_uint4(cm[j], cm[j + 1], cm[j + 2], cm[j + 3]);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        uint4 m4 = *reinterpret_cast<const uint4*>(&cmax[buf][0][16 * c + j]);
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
          const uint4 o = *reinterpret_cast<const uint4*>(&cmax[buf][ww][16 * c + j]);
          m4.x = max(m4.x, o.x); m4.y = max(m4.y, o.y); m4.z = max(m4.z, o.z); m4.w = max(m4.w, o.w);
        }
        sc[j] = scale_from_amax<FMT>(__uint_as_float(m4.x << 16));
        sc[j + 1] = scale_from_amax<FMT>(__uint_as_float(m4.y << 16));
        sc[j + 2] = scale_from_amax<FMT>(__uint_as_float(m4.z << 16));
        sc[j + 3] = scale_from_amax<FMT>(__uint_as_float(m4.w << 16));
      }
    }

    // ---- column-wise copy: scale, cast, transpose through LDS, qT stores
    uint32_t* T = tile[buf];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        b[i] = cvt4<FMT>(row_elem(v[i], 4 * k) * sc[4 * k], row_elem(v[i], 4 * k + 1) * sc[4 * k + 1],
                         row_elem(v[i], 4 * k + 2) * sc[4 * k + 2], row_elem(v[i], 4 * k + 3) * sc[4 * k + 3]);
      uint32_t col4[4];
      transpose4x4(b[0], b[1], b[2], b[3], col4);
#pragma unroll
      for (int i = 0; i < 4; ++i) T[qt_word(16 * c + 4 * k + i, a)] = col4[i];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int col = (t >> 3) + 32 * p, k = t & 7;
      if (col < cv && 16 * k < rv) {
        const uint4 wv = *reinterpret_cast<const uint4*>(&T[qt_word(col, 4 * k)]);
        *reinterpret_cast<uint4*>(qT + (c0 + col) * rows + r0 + 16 * k) = wv;
      }
    }
    // column scales of the transposed copy
    if constexpr (KIND == kTBlock1) {
      if (t < 8)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          static_cast<float*>(sqT)[(c0 + 16 * c + j) * col_blocks + r0 / 128] = 1.0f / sc[j];
    } else if constexpr (KIND == kTMX) {
      if (lane < 8 && 32 * w < rv && 16 * c < cv)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          static_cast<uint8_t*>(sqT)[(c0 + 16 * c + j) * col_blocks + r0 / 32 + w] = (uint8_t)cbyte[j];
    } else {
      if (t == 0) static_cast<float*>(sqT)[(c0 / 128) * col_blocks + r0 / 128] = 1.0f / st;
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

// One partial-maximum buffer (kWorkspaceWords words: a quantise launch uses
// at most kMaxPartials, a GEMM with a fused amax one per output tile) per
// (device, stream), allocated on first use and kept until the process ends.
// Work on one stream runs in order, so successive calls on a stream share its
// buffer safely; calls on different streams never share one.
struct StreamBuffer {
  int dev;
  hipStream_t stream;
  uint32_t* p;
};
static std::mutex g_partials_mu;
static std::vector<StreamBuffer> g_partials;

hipError_t stream_partials(hipStream_t s, uint32_t** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_partials_mu);
  for (const StreamBuffer& b : g_partials)
    if (b.dev == dev && b.stream == s) {
      *out = b.p;
      return hipSuccess;
    }
  void* p = nullptr;
  err = hipMalloc(&p, kWorkspaceWords * sizeof(uint32_t));
  if (err != hipSuccess) return err;
  g_partials.push_back({dev, s, static_cast<uint32_t*>(p)});
  *out = static_cast<uint32_t*>(p);
  return hipSuccess;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
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
                       float* scale_inv, hipStream_t s, int in) {
  uint32_t* part = nullptr;
  hipError_t err = stream_partials(s, &part);
  if (err != hipSuccess) return err;
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

template <int IN>
static void cast_kernels(const void* x, int64_t rows, int64_t cols, int fmt, ScaleSrc src,
                         uint8_t* q, uint8_t* qT, uint32_t* part, int& g, hipStream_t s) {
  const int64_t n = rows * cols;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (qT) {
    const int64_t ntx = (cols + 127) / 128;
    const int64_t ntiles = ntx * ((rows + 127) / 128);
    g = grid_for(ntiles, 1);
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
                                  hipStream_t s, int in) {
  uint32_t* part = nullptr;
  if (amax_out) {
    hipError_t err = stream_partials(s, &part);
    if (err != hipSuccess) return err;
  }
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
hipError_t launch_quantize_current(const void* x, int64_t rows, int64_t cols, int fmt,
                                   uint8_t* q, uint8_t* qT, float* amax, float* scale,
                                   float* scale_inv, hipStream_t s, int in) {
  const int64_t n = rows * cols;
  if (n == 0) return launch_amax(x, 0, fmt, amax, scale, scale_inv, s, in);
  uint32_t* part = nullptr;
  hipError_t err = stream_partials(s, &part);
  if (err != hipSuccess) return err;
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
    const int g = grid_for(ntiles, (kThreads / 8) * (kChunkLoads / 2));
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
  const int g = grid_for(nblocks, (kThreads / 4) * kChunkLoads);
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
  const int g = grid_for(ntiles, 1);
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
