// gemm_mx_k32.hip -- MXFP8 GEMM C[M][N] = sum_k a 2^ea(i,k/32) b 2^eb(j,k/32)
// (FP8 quantisation training guide, section "MXFP8 scaling": 1x32 blocks,
// E8M0 scales) for contraction lengths that are a multiple of 32 but not of
// 128.  The main kernel (gemm.hip) moves each row's E8M0 bytes of a 128-K
// step as one aligned dword through LDS, which needs K % 128 == 0; this one
// loads every lane's scale bytes from global memory instead, one step ahead.
//
// Design: a 256-thread workgroup (one wave per SIMD) computes a 256 x 256
// output tile in K steps of 128 bytes, operand tiles moved into two LDS
// stages by LDS DMA (gemm_common.h); the 4 waves form a 2 x 2 grid of 128 x 128
// sub-tiles, 8 x 8 blocks of v_mfma_scale_f32_16x16x128_f8f6f4 whose scale
// operands are the E8M0 bytes; a K tail is zero-filled by the loader and its
// scale bytes read as 127 (x1).
#include "gemm_common.h"
#include "launch.h"

namespace fp8sg {

namespace {

namespace mxk32 {

constexpr int BM = 256, BN = 256, NT = 256, WN = 128, NJ = WN / 16;

// E8M0 bytes of this lane for one step: row lr of each fragment, 32-K block
// 4*kt + g (127 past the edge or past K).
struct StepScales {
  int a[8], b[NJ];
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

template <int FA, int FB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_mx_k32(Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lA[2][BM * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[2][BN * BK];
  int tm, tn;
  if (!tile_coords(p, tm, tn)) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int wm = w >> 1, wn = w & 1;
  const int g = lane >> 4, lr = lane & 15;
  const int64_t K = p.K;
  const int nk = (int)((K + BK - 1) / BK);
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * WN;

  v4f acc[8][NJ];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  TileLoader<BM, 4> la;
  TileLoader<BN, 4> lb;
  la.init(p.A + m0 * K, p.M - m0, K, w);
  lb.init(p.B + n0 * K, p.N - n0, K, w);
  StepScales sc, sc_next;
  if (nk > 0) {
    la.load(lA[0], 0);
    lb.load(lB[0], 0);
    sc.load(p, m_base, n_base, 0, lane);
  }
  wait_vm<0>();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint8_t* As = lA[cur];
    const uint8_t* Bs = lB[cur];
    v8i bf[NJ], af[2];
    bf[0] = load_frag(Bs, wn * WN);
    af[0] = load_frag(As, wm * 128);
#pragma unroll
    for (int j = 1; j < NJ; ++j) bf[j] = load_frag(Bs, wn * WN + j * 16);
    if (kt + 1 < nk) {
      la.load(lA[cur ^ 1], (int64_t)(kt + 1) * BK);
      lb.load(lB[cur ^ 1], (int64_t)(kt + 1) * BK);
      sc_next.load(p, m_base, n_base, kt + 1, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 1 < 8) af[(f + 1) & 1] = load_frag(As, wm * 128 + (f + 1) * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[f][j] = mfma_mx<FB, FA>(bf[j], af[f & 1], acc[f][j], sc.b[j], sc.a[f]);
      __builtin_amdgcn_sched_barrier(0);
    }
    sc = sc_next;
    wait_vm<0>();
    __syncthreads();
  }

  __shared__ uint32_t red[NT / 64];
  const float qs = p.Cq != nullptr ? *p.q_scale : 1.0f;
  uint32_t mx = 0;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int64_t m = m_base + f * 16 + lr;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n = n_base + j * 16 + 4 * g;
      if (n >= p.N) continue;
      const v4f a = acc[f][j];
      store4(p, m, n, a[0], a[1], a[2], a[3], qs, mx);
    }
  }
  tile_amax<NT>(p, tm, tn, mx, red);
}

template <int FA, int FB>
hipError_t run(const GemmProblem& q, hipStream_t s) {
  Args a;
  a.A = q.A; a.B = q.B; a.sa = q.sa; a.sb = q.sb; a.C = q.C; a.out = q.out;
  a.Cq = q.Cq; a.q_scale = q.q_scale; a.q_fmt = q.q_fmt; a.part = q.part;
  a.M = q.M; a.N = q.N; a.K = q.K;
  a.tiles_m = (int)((q.M + BM - 1) / BM);
  a.tiles_n = (int)((q.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_mx_k32<FA, FB>), dim3(grid_for_tiles(a.tiles_m * a.tiles_n)),
                     dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace mxk32

}  // namespace

hipError_t launch_gemm_mx_k32(const GemmProblem& q, hipStream_t s) {
  if (q.fa == kE4M3 && q.fb == kE4M3) return mxk32::run<kE4M3, kE4M3>(q, s);
  if (q.fa == kE5M2 && q.fb == kE4M3) return mxk32::run<kE5M2, kE4M3>(q, s);
  if (q.fa == kE4M3 && q.fb == kE5M2) return mxk32::run<kE4M3, kE5M2>(q, s);
  return mxk32::run<kE5M2, kE5M2>(q, s);
}

}  // namespace fp8sg
