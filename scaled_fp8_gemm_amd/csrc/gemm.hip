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
// Design (gfx950): a 256-thread workgroup (one wave per SIMD, so each wave may
// use the full 512-entry register file) computes a 256 x BN output tile in K
// steps of 128 bytes.  Operand tiles go from HBM/L2 straight into LDS with
// buffer_load_dwordx4 ... lds (no staging registers, no LDS write
// instructions); the buffer descriptor's range check zero-fills rows past the
// edge, and a K tail is zero-filled by pointing its lanes past the range.  LDS
// holds two buffers per operand (4 x 32 KB) so the load of step k+1 overlaps
// the MFMAs of step k.  16-byte chunks are XOR-swizzled by row so the 16 rows
// a fragment read touches fall in different banks.  The 4 waves form a 2 x 2
// grid; each owns a 128 (M) x WN (N) sub-tile as 8 x WN/16 blocks of
// v_mfma_f32_16x16x128_f8f6f4 (the full-rate FP8 MFMA of CDNA4: 32 cycles
// each).  Tensor and MX scaling use WN = 128 (BN = 256): 256 FP32
// accumulators per lane, which the compiler keeps in AGPRs.  Block scaling
// must rescale every 128-K partial sum with VALU FMAs, which cannot address
// AGPRs, so it uses WN = 64 (BN = 128) with the accumulators in VGPRs.  The weight side is the
// MFMA's A operand so each lane ends up holding four consecutive output
// columns of one row (8-byte BF16 stores).  Workgroups are mapped to tiles
// XCD by XCD, in groups of 8 tile rows, so neighbouring tiles share operand
// panels in the same L2.
//
// MFMA operand layout (measured on gfx950): lane l holds row l%16 of its
// operand; bytes 0..15 hold K [16g, 16g+16) and bytes 16..31 hold K
// [64+16g, 64+16g+16) of the 128-K step, with g = l/16.  The E8M0 scale of
// lane l applies to row l%16 and 32-K block l/16.  The 4 outputs of lane l are
// rows 4g..4g+3 of the A operand against column l%16 of the B operand.
#include "fp8_device.h"
#include "launch.h"

namespace fp8sg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BM = 256, BK = 128, NT = 256;

template <int MODE> struct Shape {
  static constexpr int WN = (MODE == 1) ? 64 : 128;   // wave sub-tile width (N)
  static constexpr int BN = 2 * WN;                   // workgroup tile width (N)
  static constexpr int NJ = WN / 16;                  // B fragments per wave
};

enum : int { kTensor = 0, kBlock = 1, kMX = 2 };

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

struct Args {
  const uint8_t* A;
  const uint8_t* B;
  const void* sa;
  const void* sb;
  uint16_t* C;
  int64_t M, N, K;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

typedef int v4i __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ pointer (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p);
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from rsrc + voffset into LDS
// at m0 + 16 * lane.  Issued through inline assembly so that the compiler
// neither models it as an LDS write (which would make it wait for the load
// before unrelated LDS reads of the other buffer) nor reorders it; completion
// is awaited explicitly with vmcnt before the workgroup barrier.  m0 is
// reserved by the compiler, so the sequence restores it.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, int voffset) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voffset), "s"(rsrc)
      : "memory");
}

// Operand tile loader.  A ROWS x 128-byte tile is ROWS/8 chunks of 8 rows
// (1 KB); wave w moves chunks w*L .. w*L+L-1 with L = ROWS/32.  Lane l of a
// chunk lands at LDS byte l*16 of it, i.e. row l/8 and physical 16-byte slot
// l%8, so it loads logical chunk (l%8) ^ (row & 7) of that row.  The buffer
// descriptor covers exactly the tile's valid rows, so the hardware range
// check zero-fills rows past the matrix edge; lanes whose chunk lies past K
// are pointed at the end of the range and get zeros too.
template <int ROWS>
struct TileLoader {
  static constexpr int L = ROWS / 32;
  v4i rsrc;
  uint32_t records;
  int64_t K;
  int voff[L];      // byte offset of this lane's chunk in each of its loads (k0 = 0)
  int kchunk;       // logical 16-byte chunk this lane loads

  __device__ __forceinline__ void init(const uint8_t* base, int64_t rows_left, int64_t K_) {
    K = K_;
    const int64_t rows = rows_left < ROWS ? rows_left : ROWS;
    records = __builtin_amdgcn_readfirstlane((uint32_t)(rows * K));
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    rsrc[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) & 0xffff;  // stride 0
    rsrc[2] = (int)records;
    rsrc[3] = 0x00020000;
    const int lane = threadIdx.x & 63, w = wave_id();
    kchunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int row = (w * L + i) * 8 + (lane >> 3);
      voff[i] = (int)(row * K) + kchunk * 16;
    }
  }

  __device__ __forceinline__ void load(const uint8_t* tile, int64_t k0) const {
    const int w = wave_id();
    const bool kin = k0 + kchunk * 16 < K;
    const uint32_t base = lds_addr(tile) + (uint32_t)(w * L * 1024);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int off = kin ? voff[i] + (int)k0 : (int)records;
      dma16(rsrc, base + i * 1024, off);
    }
  }
};

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

// Per-step scale operands of this lane (prefetched one step ahead).
template <int MODE, int BRA, int BRB> struct StepScales;

template <int BRA, int BRB> struct StepScales<kTensor, BRA, BRB> {
  __device__ __forceinline__ void load(const Args&, int64_t, int64_t, int, int) {}
};

template <int BRA, int BRB> struct StepScales<kMX, BRA, BRB> {
  static constexpr int NJ = Shape<kMX>::NJ;
  int a[8], b[NJ];    // E8M0 bytes: row lr of each fragment, 32-K block 4*kt + g
  __device__ __forceinline__ void load(const Args& p, int64_t m_base, int64_t n_base, int kt,
                                       int lane) {
    const int64_t kb32 = p.K / 32;
    const int64_t kblk = (int64_t)kt * 4 + (lane >> 4);
    const bool kin = kblk < kb32;
    const uint8_t* ea = static_cast<const uint8_t*>(p.sa);
    const uint8_t* eb = static_cast<const uint8_t*>(p.sb);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int64_t m = m_base + f * 16 + (lane & 15);
      a[f] = (kin && m < p.M) ? (int)ea[m * kb32 + kblk] : 127;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n = n_base + j * 16 + (lane & 15);
      b[j] = (kin && n < p.N) ? (int)eb[n * kb32 + kblk] : 127;
    }
  }
};

template <int BRA, int BRB> struct StepScales<kBlock, BRA, BRB> {
  static constexpr int NJ = Shape<kBlock>::NJ;
  float a[8];         // row scale of this lane's output row in each fragment
  float b[NJ][BRB == 1 ? 4 : 1];  // column scale(s) of this lane's 4 output columns
  __device__ __forceinline__ void load(const Args& p, int64_t m_base, int64_t n_base, int kt,
                                       int lane) {
    const int64_t kb128 = p.K / 128;
    const float* sa = static_cast<const float*>(p.sa);
    const float* sb = static_cast<const float*>(p.sb);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int64_t m = m_base + f * 16 + (lane & 15);
      const int64_t mr = (BRA == 1) ? m : (m / 128);
      a[f] = (m < p.M) ? sa[mr * kb128 + kt] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n0 = n_base + j * 16 + 4 * (lane >> 4);
      if constexpr (BRB == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) b[j][r] = (n0 + r < p.N) ? sb[(n0 + r) * kb128 + kt] : 0.f;
      } else {
        b[j][0] = (n0 < p.N) ? sb[(n0 / 128) * kb128 + kt] : 0.f;
      }
    }
  }
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

// MFMAs of one fragment row f (8 or 4 MFMAs) of this wave's sub-tile.
template <int MODE, int FA, int FB, int BRA, int BRB>
__device__ __forceinline__ void mma_row(int f, const v8i& af, const v8i (&bf)[Shape<MODE>::NJ],
                                        const StepScales<MODE, BRA, BRB>& sc,
                                        v4f (&acc)[8][Shape<MODE>::NJ]) {
  constexpr int NJ = Shape<MODE>::NJ;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if constexpr (MODE == kTensor) {
      acc[f][j] = mfma<FB, FA>(bf[j], af, acc[f][j]);
    } else if constexpr (MODE == kMX) {
      acc[f][j] = mfma_mx<FB, FA>(bf[j], af, acc[f][j], sc.b[j], sc.a[f]);
    } else {
      const v4f part = mfma<FB, FA>(bf[j], af, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[f][j][r] += (sc.a[f] * sc.b[j][BRB == 1 ? r : 0]) * part[r];
    }
  }
}

__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this lane's LDS DMA has landed
}

template <int MODE, int FA, int FB, int BRA, int BRB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm(Args p) {
  constexpr int WN = Shape<MODE>::WN, BN = Shape<MODE>::BN, NJ = Shape<MODE>::NJ;
  __shared__ __attribute__((aligned(1024))) uint8_t lA[2][BM * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[2][BN * BK];
  int tm, tn;
  if (!tile_coords(p, tm, tn)) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int wm = w >> 1, wn = w & 1;           // wave sub-tile: rows wm*128, cols wn*WN
  const int g = lane >> 4, lr = lane & 15;
  const int64_t K = p.K;
  const int nk = (int)((K + BK - 1) / BK);
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * WN;

  v4f acc[8][NJ];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  TileLoader<BM> la;
  TileLoader<BN> lb;
  la.init(p.A + m0 * K, p.M - m0, K);
  lb.init(p.B + n0 * K, p.N - n0, K);
  StepScales<MODE, BRA, BRB> sc, sc_next;

  if (nk > 0) {
    la.load(lA[0], 0);
    lb.load(lB[0], 0);
    sc.load(p, m_base, n_base, 0, lane);
  }
  wait_dma();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint8_t* As = lA[cur];
    const uint8_t* Bs = lB[cur];
    // Fragment reads for row 0 (all B fragments and A fragment 0) ...
    v8i bf[NJ], af[2];
    bf[0] = load_frag(Bs, wn * WN);
    af[0] = load_frag(As, wm * 128);
#pragma unroll
    for (int j = 1; j < NJ; ++j) bf[j] = load_frag(Bs, wn * WN + j * 16);
    // ... then the next step's tiles and scales start streaming in ...
    if (kt + 1 < nk) {
      la.load(lA[cur ^ 1], (int64_t)(kt + 1) * BK);
      lb.load(lB[cur ^ 1], (int64_t)(kt + 1) * BK);
      sc_next.load(p, m_base, n_base, kt + 1, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ... and each MFMA row runs while the next A fragment is read.
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 1 < 8) af[(f + 1) & 1] = load_frag(As, wm * 128 + (f + 1) * 16);
      __builtin_amdgcn_sched_barrier(0);
      mma_row<MODE, FA, FB, BRA, BRB>(f, af[f & 1], bf, sc, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    sc = sc_next;
    wait_dma();
    __syncthreads();
  }

  // Epilogue: scale (tensor mode), round to BF16, 8-byte stores.
  float s = 1.0f;
  if constexpr (MODE == kTensor)
    s = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sb)[0];
  const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int64_t m = m_base + f * 16 + lr;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n = n_base + j * 16 + 4 * g;
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
  constexpr int BN = Shape<MODE>::BN;
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

// ---------------------------------------------------------------------------
// Deep-pipeline kernel, used for MX scaling (K % 128 == 0).
//
// The kernel above keeps one 64 KB step in flight per CU (two LDS stages of
// 256x128 per operand), and its loads then run latency-bound: memory-side
// and MFMA time add instead of overlapping.  This kernel moves K in steps of
// 64 on v_mfma_f32_32x32x64_f8f6f4 (same FP8 rate: 64 cycles per 32x32x64),
// so a stage of the 256x256 tile is 32 KB and four stages fit in LDS: the
// loads of step k+3 are issued while step k computes.  MX scale bytes travel
// through the same LDS stages (one dword per row and step), so every global
// load of the main loop is an LDS DMA whose completion is tracked by one
// explicit vmcnt wait per step.
//
// 32x32x64 operand layout (measured): lane l holds row l%32; bytes 0..15 hold
// K [16h, 16h+16) and bytes 16..31 hold K [32+16h, 32+16h+16) of the 64-K
// step, h = l/32; the E8M0 scale of lane l applies to row l%32, 32-K block h.
// Output register r of lane l is row 8(r/4) + 4h + r%4 of the A operand
// against column l%32 of the B operand.
namespace deep {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64, NSTAGE = 4, NT = 256;
constexpr int TILE = BM * BK;          // bytes per operand per stage

// 64-byte rows, 16-byte chunks XOR-swizzled by (row >> 1) & 3: the 8 rows an
// 8-lane group of a fragment read touches land in 8 distinct 16-byte slots.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 3)) << 4);
}

__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, int voffset) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voffset), "s"(rsrc)
      : "memory");
}

__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t records) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) & 0xffff;
  r[2] = (int)__builtin_amdgcn_readfirstlane(records);
  r[3] = 0x00020000;
  return r;
}

// One operand's 256 x 64-byte stage: 16 chunks of 16 rows (1 KB); wave w
// moves chunks 4w .. 4w+3.  Lane l of a chunk lands at row l/4, physical slot
// l%4, so it loads logical chunk (l%4) ^ ((row >> 1) & 3) of that row.
struct DataLoader {
  v4i rsrc;
  uint32_t records;
  int64_t K;
  int voff[4];
  int kchunk;
  int w;            // position of the loading wave among the 4 loaders
  __device__ __forceinline__ void init(const uint8_t* base, int64_t rows_left, int64_t K_,
                                       int pos) {
    K = K_;
    w = pos;
    const int64_t rows = rows_left < BM ? rows_left : BM;
    records = (uint32_t)(rows * K);
    rsrc = make_rsrc(base, records);
    const int lane = threadIdx.x & 63;
    const int rr = lane >> 2;
    kchunk = (lane & 3) ^ ((rr >> 1) & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = (int)(((w * 4 + i) * 16 + rr) * K) + kchunk * 16;
  }
  __device__ __forceinline__ void load_one(uint32_t stage_lds, int64_t k0, int i) const {
    const int off = (k0 + kchunk * 16 < K) ? voff[i] + (int)k0 : (int)records;
    dma16(rsrc, stage_lds + (uint32_t)((w * 4 + i) * 1024), off);
  }
};

// MX scales of one operand for one stage: for each of the 256 rows the dword
// holding the E8M0 bytes of the step's two 32-K blocks (K % 128 == 0, so
// the byte offset 2*kt rounded down to even steps is dword aligned); wave w
// moves rows 64w .. 64w+63, landing at LDS byte 4*row.
struct ScaleLoader {
  v4i rsrc;
  int voff;
  int w;
  __device__ __forceinline__ void init(const uint8_t* base, int64_t rows_left, int64_t kb32,
                                       int pos) {
    w = pos;
    const int64_t rows = rows_left < BM ? rows_left : BM;
    rsrc = make_rsrc(base, (uint32_t)(rows * kb32));
    voff = (int)((w * 64 + (threadIdx.x & 63)) * kb32);
  }
  __device__ __forceinline__ void load(uint32_t stage_lds, int kt) const {
    dma4(rsrc, stage_lds + (uint32_t)(w * 256), voff + 2 * (kt & ~1));
  }
};

// vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Operand fragment of 32 rows starting at row0 of a stage tile.
__device__ __forceinline__ v8i load_frag(const uint8_t* __restrict__ s, int row0) {
  const int l = threadIdx.x & 63;
  const int r = row0 + (l & 31), h = l >> 5;
  const uint4 lo = *reinterpret_cast<const uint4*>(s + swz(r, h));
  const uint4 hi = *reinterpret_cast<const uint4*>(s + swz(r, h + 2));
  v8i o;
  o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w;
  o[4] = hi.x; o[5] = hi.y; o[6] = hi.z; o[7] = hi.w;
  return o;
}

template <bool MX, int FA, int FB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_deep(Args p) {
  constexpr int LOADS = 8 + (MX ? 2 : 0);      // DMA instructions per wave per step
  __shared__ __attribute__((aligned(1024))) uint8_t lA[NSTAGE][TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[NSTAGE][TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lSA[MX ? NSTAGE : 1][MX ? 1024 : 4];
  __shared__ __attribute__((aligned(1024))) uint8_t lSB[MX ? NSTAGE : 1][MX ? 1024 : 4];
  int tm, tn;
  if (!tile_coords(p, tm, tn)) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int wm = w >> 1, wn = w & 1;           // wave sub-tile: rows wm*128, cols wn*128
  const int h = lane >> 5, lr = lane & 31;
  const int64_t K = p.K;
  const int nk = (int)((K + BK - 1) / BK);

  v16f acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][j][r] = 0.f;

  DataLoader la, lb;
  la.init(p.A + m0 * K, p.M - m0, K, w);
  lb.init(p.B + n0 * K, p.N - n0, K, w);
  ScaleLoader sla, slb;
  if constexpr (MX) {
    const int64_t kb32 = K / 32;
    sla.init(static_cast<const uint8_t*>(p.sa) + m0 * kb32, p.M - m0, kb32, w);
    slb.init(static_cast<const uint8_t*>(p.sb) + n0 * kb32, p.N - n0, kb32, w);
  }
  uint32_t ldsA[NSTAGE], ldsB[NSTAGE], ldsSA[NSTAGE], ldsSB[NSTAGE];
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) {
    ldsA[s] = lds_addr(lA[s]);
    ldsB[s] = lds_addr(lB[s]);
    if constexpr (MX) {
      ldsSA[s] = lds_addr(lSA[s]);
      ldsSB[s] = lds_addr(lSB[s]);
    }
  }

  // All DMA of step t into stage t % NSTAGE: 4 A chunks, 4 B chunks, 2 scale rows.
  auto issue = [&](int t, int i) {
    const int st = t % NSTAGE;
    const int64_t k0 = (int64_t)t * BK;
    if (i < 4) la.load_one(ldsA[st], k0, i);
    else if (i < 8) lb.load_one(ldsB[st], k0, i - 4);
    else if constexpr (MX) {
      if (i == 8) sla.load(ldsSA[st], t);
      else slb.load(ldsSB[st], t);
    }
  };

#pragma unroll
  for (int t = 0; t < NSTAGE - 1; ++t)
    if (t < nk)
#pragma unroll
      for (int i = 0; i < LOADS; ++i) issue(t, i);

  for (int kt = 0; kt < nk; ++kt) {
    // This lane's loads of step kt are done once at most the loads of the
    // (up to two) later steps already issued are outstanding; the barrier
    // then makes every wave's part visible and frees stage (kt - 1) % 4.
    const int later = nk - 1 - kt;
    if (later >= 2) wait_vm<2 * LOADS>();
    else if (later == 1) wait_vm<LOADS>();
    else wait_vm<0>();
    __syncthreads();

    const int st = kt % NSTAGE;
    const uint8_t* As = lA[st];
    const uint8_t* Bs = lB[st];
    const bool more = kt + NSTAGE - 1 < nk;
    v8i bf[4], af[2];
    int sa[4], sb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = load_frag(Bs, wn * 128 + j * 32);
    af[0] = load_frag(As, wm * 128);
    if constexpr (MX) {
      const int sel = h + 2 * (kt & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) sb[j] = lSB[st][(wn * 128 + j * 32 + lr) * 4 + sel];
#pragma unroll
      for (int f = 0; f < 4; ++f) sa[f] = lSA[st][(wm * 128 + f * 32 + lr) * 4 + sel];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (f + 1 < 4) af[(f + 1) & 1] = load_frag(As, wm * 128 + (f + 1) * 32);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (MX)
          acc[f][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bf[j], af[f & 1], acc[f][j], FB, FA, 0, sb[j], 0, sa[f]);
        else
          acc[f][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bf[j], af[f & 1], acc[f][j], FB, FA, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // the DMA of step kt + 3, one load after each of the first MFMAs
        const int i = f * 4 + j;
        if (i < LOADS && more) {
          issue(kt + NSTAGE - 1, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // Epilogue: scale (tensor mode), BF16, four 8-byte stores per 32x32 block.
  float s = 1.0f;
  if constexpr (!MX) s = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sb)[0];
  const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t m = m0 + wm * 128 + f * 32 + lr;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 128 + j * 32 + 8 * q + 4 * h;
        if (n >= p.N) continue;
        uint16_t* dst = p.C + m * p.N + n;
        const float a0 = acc[f][j][4 * q] * s, a1 = acc[f][j][4 * q + 1] * s;
        const float a2 = acc[f][j][4 * q + 2] * s, a3 = acc[f][j][4 * q + 3] * s;
        if (vec_ok) {
          uint2 o;
          o.x = pack_bf16x2(a0, a1);
          o.y = pack_bf16x2(a2, a3);
          *reinterpret_cast<uint2*>(dst) = o;
        } else {
          const float v[4] = {a0, a1, a2, a3};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.N) dst[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xffffu);
        }
      }
    }
  }
}

template <bool MX, int FA, int FB>
hipError_t run(const GemmProblem& q, hipStream_t s) {
  Args a;
  a.A = q.A; a.B = q.B; a.sa = q.sa; a.sb = q.sb; a.C = q.C;
  a.M = q.M; a.N = q.N; a.K = q.K;
  a.tiles_m = (int)((q.M + BM - 1) / BM);
  a.tiles_n = (int)((q.N + BN - 1) / BN);
  const int T = a.tiles_m * a.tiles_n;
  const int grid = ((T + 7) / 8) * 8;
  hipLaunchKernelGGL((k_gemm_deep<MX, FA, FB>), dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <bool MX>
hipError_t run_fmt(const GemmProblem& q, hipStream_t s) {
  if (q.fa == kE4M3 && q.fb == kE4M3) return run<MX, kE4M3, kE4M3>(q, s);
  if (q.fa == kE5M2 && q.fb == kE4M3) return run<MX, kE5M2, kE4M3>(q, s);
  if (q.fa == kE4M3 && q.fb == kE5M2) return run<MX, kE4M3, kE5M2>(q, s);
  return run<MX, kE5M2, kE5M2>(q, s);
}

}  // namespace deep

}  // namespace

hipError_t launch_gemm(const GemmProblem& q, hipStream_t s) {
  if (q.M == 0 || q.N == 0) return hipSuccess;
  if (q.mode == kTensor) return run_fmt<kTensor, 1, 1>(q, s);
  if (q.mode == kMX) {
    if (q.K % 128 == 0) return deep::run_fmt<true>(q, s);
    return run_fmt<kMX, 1, 1>(q, s);   // MX with K % 128 != 0: scale rows not dword aligned
  }
  if (q.bra == 1 && q.brb == 128) return run_fmt<kBlock, 1, 128>(q, s);
  if (q.bra == 1 && q.brb == 1) return run_fmt<kBlock, 1, 1>(q, s);
  if (q.bra == 128 && q.brb == 1) return run_fmt<kBlock, 128, 1>(q, s);
  return run_fmt<kBlock, 128, 128>(q, s);
}

}  // namespace fp8sg
