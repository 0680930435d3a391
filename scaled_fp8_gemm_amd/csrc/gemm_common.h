// gemm_common.h -- pieces shared by the FP8 MFMA GEMM kernels of libfp8sg
// (gfx950): kernel arguments, the XCD-aware tile order, LDS DMA of operand
// tiles (buffer_load ... lds) and the 16x16x128 MFMA fragment reads.
//
// MFMA operand layout of v_mfma_*_16x16x128_f8f6f4 (measured on gfx950):
// lane l holds row l%16 of its operand; bytes 0..15 hold K [16g, 16g+16) and
// bytes 16..31 hold K [64+16g, 64+16g+16) of the 128-K step, with g = l/16.
// The E8M0 scale of lane l applies to row l%16 and 32-K block l/16.  The 4
// outputs of lane l are rows 4g..4g+3 of the first operand against row l%16
// of the second.
#pragma once

#include "fp8_device.h"

namespace fp8sg {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum : int { kTensor = 0, kBlock = 1, kMX = 2 };

// Bytes of K per main-loop step of the BK = 128 kernels.
constexpr int BK = 128;

struct Args {
  const uint8_t* A;
  const uint8_t* B;
  const void* sa;
  const void* sb;
  void* C;
  int64_t M, N, K;
  int tiles_m, tiles_n;
  int out;      // 0: BF16 C; 1: FP32 C; 2: FP32 C += result
  // fused epilogue of the BF16 mode (next layer's quantisation):
  uint8_t* Cq;          // FP8 copy of the BF16-rounded output, or NULL
  const float* q_scale; // its scale
  int q_fmt;            // its format
  uint32_t* part;       // per-tile maxima of |BF16 output| (FP32 bits), or NULL
};

// Four consecutive outputs of row m, columns n .. n+3 (columns past N are
// dropped): rounded to BF16 (nearest even), stored as FP32, or added in FP32
// to what C holds.  16-byte / 8-byte vector stores when N % 4 == 0.  In the
// BF16 mode the fused epilogue also takes mx = max(mx, |BF16 value|) (FP32
// bits) and writes Cq = cast(BF16 value * qs) (N % 16 == 0 there); C may then
// be NULL.
__device__ __forceinline__ void store4(const Args& p, int64_t m, int64_t n, float a0, float a1,
                                       float a2, float a3, float qs, uint32_t& mx) {
  const int64_t off = m * p.N + n;
  const bool vec = (p.N & 3) == 0;
  const float v[4] = {a0, a1, a2, a3};
  if (p.out == 0) {
    const uint32_t w0 = pack_bf16x2(a0, a1), w1 = pack_bf16x2(a2, a3);
    if (p.C != nullptr) {
      uint16_t* dst = static_cast<uint16_t*>(p.C) + off;
      if (vec) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) dst[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xffffu);
      }
    }
    if (p.part != nullptr)
      mx = max(mx, max(max(w0 & 0x7fffu, (w0 >> 16) & 0x7fffu),
                       max(w1 & 0x7fffu, (w1 >> 16) & 0x7fffu)) << 16);
    if (p.Cq != nullptr) {
      const float b0 = bf_lo(w0) * qs, b1 = bf_hi(w0) * qs, b2 = bf_lo(w1) * qs, b3 = bf_hi(w1) * qs;
      const uint32_t q4 = p.q_fmt == kE4M3 ? cvt4<kE4M3>(b0, b1, b2, b3) : cvt4<kE5M2>(b0, b1, b2, b3);
      *reinterpret_cast<uint32_t*>(p.Cq + off) = q4;
    }
  } else {
    float* dst = static_cast<float*>(p.C) + off;
    const bool acc = p.out == 2;
    if (vec) {
      float4 o = make_float4(a0, a1, a2, a3);
      if (acc) {
        const float4 c = *reinterpret_cast<const float4*>(dst);
        o = make_float4(c.x + a0, c.y + a1, c.z + a2, c.w + a3);
      }
      *reinterpret_cast<float4*>(dst) = o;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < p.N) dst[r] = acc ? dst[r] + v[r] : v[r];
    }
  }
}

// End of the fused epilogue: the workgroup's largest |output| goes to
// part[tile].  All NT threads must call it.
template <int NT>
__device__ __forceinline__ void tile_amax(const Args& p, int tm, int tn, uint32_t mx,
                                          uint32_t* red) {
  if (p.part == nullptr) return;
  mx = block_max_u32<NT>(mx, red);
  if (threadIdx.x == 0) p.part[tm * p.tiles_n + tn] = mx;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// 128-byte rows of a BK = 128 stage; 16-byte chunks XOR-swizzled by row so
// the 16 rows a fragment read touches fall in different banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 4);
}

// Operand tile loader for BK = 128 stages.  A ROWS x 128-byte tile is ROWS/8
// chunks of 8 rows (1 KB); with NW loading waves, wave w moves chunks
// w*L .. w*L+L-1, L = ROWS / (8 * NW).  Lane l of a chunk lands at LDS byte
// l*16 of it, i.e. row l/8 and physical 16-byte slot l%8, so it loads logical
// chunk (l%8) ^ (row & 7) of that row.  The buffer descriptor covers exactly
// the tile's valid rows, so the hardware range check zero-fills rows past the
// matrix edge; lanes whose chunk lies past K are pointed at the end of the
// range and get zeros too.  Offsets are 32-bit: the ABI keeps K <= 2^23.
template <int ROWS, int NW>
struct TileLoader {
  static constexpr int L = ROWS / (8 * NW);
  v4i rsrc;
  uint32_t records;
  int64_t K;
  int voff[L];      // byte offset of this lane's chunk in each of its loads (k0 = 0)
  int kchunk;       // logical 16-byte chunk this lane loads
  int w;            // index of this wave among the NW loading waves

  __device__ __forceinline__ void init(const uint8_t* base, int64_t rows_left, int64_t K_,
                                       int wave) {
    K = K_;
    w = wave;
    const int64_t rows = rows_left < ROWS ? rows_left : ROWS;
    records = __builtin_amdgcn_readfirstlane((uint32_t)(rows * K));
    rsrc = make_rsrc(base, records);
    const int lane = threadIdx.x & 63;
    kchunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int row = (w * L + i) * 8 + (lane >> 3);
      voff[i] = (int)(row * K) + kchunk * 16;
    }
  }

  // live = false: every lane reads past the range, so the hardware fetches
  // nothing and zero-fills the tile (a load that need not happen, issued
  // without a branch around it).
  __device__ __forceinline__ void load(const uint8_t* tile, int64_t k0, bool live = true) const {
#pragma unroll
    for (int i = 0; i < L; ++i) load_one(tile, k0, i, live);
  }
  // The i-th of this wave's L loads of the tile (so that a step's loads can
  // be spread over its MFMAs).
  __device__ __forceinline__ void load_one(const uint8_t* tile, int64_t k0, int i,
                                           bool live = true) const {
    const bool kin = live && k0 + kchunk * 16 < K;
    const uint32_t base = lds_addr(tile) + (uint32_t)(w * L * 1024);
    dma16(rsrc, base + i * 1024, kin ? voff[i] + (int)k0 : (int)records);
  }
};

// Per-row scale words of one operand for four steps: wave `part` (0..3)
// moves rows 64*part .. 64*part + 63 of the tile, 16 bytes per row (the words
// of steps 4c .. 4c+3), landing at LDS words 4*row .. 4*row + 3.
//   block: the FP32 scales of the row's 128-K blocks (rows grouped by BR:
//          BR = 1 one scale per row, BR = 128 one per 128 rows);
//   MX:    the dwords holding the row's four E8M0 bytes of each step.
// One 16-byte load per row and four steps rather than a 4-byte load per step
// cuts the scale requests, which touch one cache line per row, by four.
// Rows past the matrix edge, and words past the scale array, read past the
// descriptor range and get 0; words past the row's last step are not used.
struct ScaleRows {
  v4i rsrc;
  int voff;
  uint32_t records;
  __device__ __forceinline__ void init(const void* scales, int64_t row0, int64_t rows_left,
                                       int br, int64_t words_per_row, int part) {
    const int64_t first = row0 / br;
    const int64_t rows = rows_left < 256 ? rows_left : 256;
    const int64_t groups = (rows + br - 1) / br;
    records = (uint32_t)(groups * words_per_row * 4);
    rsrc = make_rsrc(static_cast<const uint8_t*>(scales) + first * words_per_row * 4, records);
    const int r = part * 64 + (int)(threadIdx.x & 63);
    voff = r < rows ? (int)((r / br) * words_per_row * 4) : -1;
  }
  // live = false: nothing is fetched and zeros land at `lds`
  __device__ __forceinline__ void load(uint32_t lds, int chunk, bool live = true) const {
    dma16(rsrc, lds, live && voff >= 0 ? voff + chunk * 16 : (int)records);
  }
};

// MFMA operand of 16 rows starting at `row0` of a BK = 128 LDS tile.
__device__ __forceinline__ v8i load_frag(const uint8_t* __restrict__ s, int row0) {
  const int l = threadIdx.x & 63;
  const int r = row0 + (l & 15), g = l >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(s + swz(r, g));
  const uint4 hi = *reinterpret_cast<const uint4*>(s + swz(r, g + 4));
  v8i o;
  o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
  o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
  return o;
}

template <int FA_OP, int FB_OP>
__device__ __forceinline__ v4f mfma(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA_OP, FB_OP, 0, 0, 0, 0);
}
template <int FA_OP, int FB_OP>
__device__ __forceinline__ v4f mfma_mx(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA_OP, FB_OP, 0, sa, 0, sb);
}

// Tile order: consecutive workgroups land on different XCDs (round robin over
// 8), so workgroup b is first mapped to a contiguous range of tiles per XCD,
// then tiles are walked in groups of 8 tile-rows so that neighbours share
// A rows and B rows in that XCD's L2.
__device__ __forceinline__ bool tile_coords(const Args& p, int& tm, int& tn) {
  const int T = p.tiles_m * p.tiles_n;
  const int per = (T + 7) / 8;
  const int b = blockIdx.x;
  const int t = (b & 7) * per + (b >> 3);
  if (t >= T) return false;
  constexpr int G = 8;
  const int group = t / (G * p.tiles_n);
  const int first_m = group * G;
  const int gsize = min(p.tiles_m - first_m, G);
  const int in_group = t - group * G * p.tiles_n;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
  return true;
}

// Workgroups for T tiles: a multiple of 8 so every XCD gets the same count.
inline int grid_for_tiles(int T) { return ((T + 7) / 8) * 8; }

}  // namespace
}  // namespace fp8sg
