// gemm.hip -- scaled FP8 GEMM C[M][N] = A[M][K] . B[N][K]^T on gfx950 MFMA,
// FP32 accumulation, BF16 output.  One kernel serves fprop, dgrad and wgrad of
// a linear layer (FP8 quantisation training guide, section "code changes":
// the three GEMMs take quantised inputs and keep BF16 outputs; fp8+bf8
// search-result snippet on the forward pass: output cast back to BF16 after
// accumulation).  Scaling modes:
//   tensor: C = (sa * sb) * sum_k a b                       (per-tensor scales)
//   block : C = sum_b sa(i,b) sb(j,b) sum_{k in b} a b      (guide, "blockwise
//           scaling": 1x128 and 128x128 blocks; 128-wide K blocks)
//   MX    : C = sum_k a 2^ea(i,k/32) b 2^eb(j,k/32)         (guide, "MXFP8
//           scaling": 1x32 blocks, E8M0 scales), on the block-scaled MFMA.
//
// Design (gfx950): a 512-thread workgroup computes a 256x256 output tile with
// K steps of 128 bytes.  Both operands are staged through LDS (2 x 64 KB,
// double buffered, 16-byte chunks XOR-swizzled by row to spread banks).  Each
// of the 8 waves owns a 128 (M) x 64 (N) sub-tile as 8 x 4 blocks of
// v_mfma_f32_16x16x128_f8f6f4 (the full-rate FP8 MFMA of CDNA4).  The weight
// side is the MFMA's A operand so that each lane ends up holding four
// consecutive output columns of one row (8-byte BF16 stores).
//
// MFMA operand layout (measured on gfx950): lane l holds row l%16 of its
// operand; bytes 0..15 hold K [16g, 16g+16) and bytes 16..31 hold K
// [64+16g, 64+16g+16) of the 128-K step, with g = l/16.  The E8M0 scale of
// lane l applies to row l%16 and 32-K block l/16.  The 4x4 outputs of lane l
// are rows 4g..4g+3 of the A operand against column l%16 of the B operand.
#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128, NT = 512;
constexpr int kTileBytes = BM * BK;   // one operand tile in LDS (BM == BN)

enum : int { kTensor = 0, kBlock = 1, kMX = 2 };

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// Global -> registers: thread t loads 16-byte chunk (t % 8) of rows t/8 + 64i.
__device__ __forceinline__ void load_tile(const uint8_t* __restrict__ g, int64_t rows, int64_t K,
                                          int64_t r0, int64_t k0, uint4 (&v)[4]) {
  const int c = threadIdx.x & 7;
  const int64_t kk = k0 + c * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + (threadIdx.x >> 3) + 64 * i;
    if (r < rows && kk < K)
      v[i] = *reinterpret_cast<const uint4*>(g + r * K + kk);
    else
      v[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void store_tile(uint8_t* __restrict__ s, const uint4 (&v)[4]) {
  const int c = threadIdx.x & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (threadIdx.x >> 3) + 64 * i;
    *reinterpret_cast<uint4*>(s + swz(r, c)) = v[i];
  }
}

// MFMA operand of 16 rows starting at `row0` of an LDS tile.
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

struct Args {
  const uint8_t* A;
  const uint8_t* B;
  const void* sa;
  const void* sb;
  uint16_t* C;
  int64_t M, N, K;
  int tiles_m, tiles_n;
};

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

template <int MODE, int FA, int FB, int BRA, int BRB>
__global__ __launch_bounds__(NT) void k_gemm(Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];
  int tm, tn;
  if (!tile_coords(p, tm, tn)) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3;           // wave sub-tile: rows wm*128, cols wn*64
  const int g = lane >> 4, lr = lane & 15;
  const int64_t K = p.K;
  const int nk = (int)((K + BK - 1) / BK);
  const int64_t kb32 = K / 32, kb128 = K / 128;

  v4f acc[8][4];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[4];
  load_tile(p.A, p.M, K, m0, 0, ra);
  load_tile(p.B, p.N, K, n0, 0, rb);
  store_tile(lds[0][0], ra);
  store_tile(lds[0][1], rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_tile(p.A, p.M, K, m0, (int64_t)(kt + 1) * BK, ra);
      load_tile(p.B, p.N, K, n0, (int64_t)(kt + 1) * BK, rb);
    }
    const uint8_t* As = lds[buf][0];
    const uint8_t* Bs = lds[buf][1];

    v8i bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = load_frag(Bs, wn * 64 + j * 16);

    if constexpr (MODE == kTensor) {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const v8i af = load_frag(As, wm * 128 + f * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[f][j] = mfma<FB, FA>(bf[j], af, acc[f][j]);
      }
    } else if constexpr (MODE == kMX) {
      // E8M0 bytes: lane supplies row lr of its operand and 32-K block g.
      const int64_t kblk = (int64_t)kt * 4 + g;
      const bool kin = kblk < kb32;
      const uint8_t* ea = static_cast<const uint8_t*>(p.sa);
      const uint8_t* eb = static_cast<const uint8_t*>(p.sb);
      int sbj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + lr;
        sbj[j] = (kin && n < p.N) ? (int)eb[n * kb32 + kblk] : 127;
      }
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int64_t m = m0 + wm * 128 + f * 16 + lr;
        const int saf = (kin && m < p.M) ? (int)ea[m * kb32 + kblk] : 127;
        const v8i af = load_frag(As, wm * 128 + f * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[f][j] = mfma_mx<FB, FA>(bf[j], af, acc[f][j], sbj[j], saf);
      }
    } else {  // kBlock: promote each 128-K partial sum with its block scales
      const float* sa = static_cast<const float*>(p.sa);
      const float* sb = static_cast<const float*>(p.sb);
      float sbv[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t nb = n0 + wn * 64 + j * 16 + 4 * g;   // first of this lane's 4 columns
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t n = nb + r;
          const int64_t nr = (BRB == 1) ? n : (n / 128);
          sbv[j][r] = (n < p.N) ? sb[nr * kb128 + kt] : 0.f;
        }
      }
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int64_t m = m0 + wm * 128 + f * 16 + lr;
        const int64_t mr = (BRA == 1) ? m : (m / 128);
        const float saf = (m < p.M) ? sa[mr * kb128 + kt] : 0.f;
        const v8i af = load_frag(As, wm * 128 + f * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f part = mfma<FB, FA>(bf[j], af, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[f][j][r] += (saf * sbv[j][r]) * part[r];
        }
      }
    }

    if (kt + 1 < nk) {
      store_tile(lds[buf ^ 1][0], ra);
      store_tile(lds[buf ^ 1][1], rb);
    }
    __syncthreads();
  }

  // Epilogue: scale (tensor mode), round to BF16, 8-byte stores.
  float s = 1.0f;
  if constexpr (MODE == kTensor)
    s = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sb)[0];
  const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int64_t m = m0 + wm * 128 + f * 16 + lr;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + j * 16 + 4 * g;
      if (n >= p.N) continue;
      const v4f a = acc[f][j];
      uint16_t* dst = p.C + m * p.N + n;
      if (vec_ok) {
        uint2 o;
        o.x = pack_bf16x2(a[0] * s, a[1] * s);
        o.y = pack_bf16x2(a[2] * s, a[3] * s);
        *reinterpret_cast<uint2*>(dst) = o;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.N) dst[r] = (uint16_t)(pack_bf16x2(a[r] * s, 0.f) & 0xffffu);
      }
    }
  }
}

template <int MODE, int FA, int FB, int BRA, int BRB>
hipError_t run(const GemmProblem& q, hipStream_t s) {
  Args a;
  a.A = q.A; a.B = q.B; a.sa = q.sa; a.sb = q.sb; a.C = q.C;
  a.M = q.M; a.N = q.N; a.K = q.K;
  a.tiles_m = (int)((q.M + BM - 1) / BM);
  a.tiles_n = (int)((q.N + BN - 1) / BN);
  const int T = a.tiles_m * a.tiles_n;
  const int grid = ((T + 7) / 8) * 8;
  hipLaunchKernelGGL((k_gemm<MODE, FA, FB, BRA, BRB>), dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int MODE, int BRA, int BRB>
hipError_t run_fmt(const GemmProblem& q, hipStream_t s) {
  if (q.fa == kE4M3 && q.fb == kE4M3) return run<MODE, kE4M3, kE4M3, BRA, BRB>(q, s);
  if (q.fa == kE5M2 && q.fb == kE4M3) return run<MODE, kE5M2, kE4M3, BRA, BRB>(q, s);
  if (q.fa == kE4M3 && q.fb == kE5M2) return run<MODE, kE4M3, kE5M2, BRA, BRB>(q, s);
  return run<MODE, kE5M2, kE5M2, BRA, BRB>(q, s);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& q, hipStream_t s) {
  if (q.M == 0 || q.N == 0) return hipSuccess;
  if (q.mode == kTensor) return run_fmt<kTensor, 1, 1>(q, s);
  if (q.mode == kMX) return run_fmt<kMX, 1, 1>(q, s);
  if (q.bra == 1 && q.brb == 128) return run_fmt<kBlock, 1, 128>(q, s);
  if (q.bra == 1 && q.brb == 1) return run_fmt<kBlock, 1, 1>(q, s);
  if (q.bra == 128 && q.brb == 1) return run_fmt<kBlock, 128, 1>(q, s);
  return run_fmt<kBlock, 128, 128>(q, s);
}

}  // namespace fp8sg
