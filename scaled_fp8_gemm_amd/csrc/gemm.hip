// gemm.hip -- scaled FP8 GEMM C[M][N] = A[M][K] . B[N][K]^T on gfx950 MFMA,
// FP32 accumulation, BF16 output, two waves per SIMD (8 waves, 512 threads
// per workgroup).  One kernel serves fprop, dgrad and wgrad of a linear layer
// (FP8 quantisation training guide, sections "code changes", "blockwise
// scaling" and "MXFP8 scaling"; fp8+bf8 search-result snippet on the forward
// pass: output cast back to BF16 after accumulation):
//   tensor: C = (sa * sb) * sum_k a b
//   block : C = sum_b sa(i,b) sb(j,b) P_b,  P_b = sum_{k in 128-K block b} a b
//   MX    : C = sum_k a 2^ea(i,k/32) b 2^eb(j,k/32)
// with FP32 accumulation and one BF16 rounding at the end.
//
// Design.  A 256 x 256 output tile per workgroup, K steps of 128 bytes, two
// LDS stages of 64 KB: A and B tiles go from HBM/L2 straight into LDS with
// buffer_load_dwordx4 ... lds (gemm_common.h), so the load of step k+1
// overlaps the MFMAs of step k, plus the step's per-row scales.  The 8 waves form a 4 (M) x 2 (N)
// grid of 64 x 128 sub-tiles: 4 x 8 fragments of v_mfma_*_16x16x128_f8f6f4,
// 128 FP32 accumulators per lane.  That is half of what a one-wave-per-SIMD
// 128 x 128 sub-tile needs, so
//   * blockwise scaling keeps its accumulators in VGPRs, where the VALU can
//     add each 128-K partial product times its scale: the MFMAs of fragment
//     column j are issued before the scale-and-add of column j - 1, so that
//     VALU work overlaps MFMA execution, and the SIMD's second wave fills the
//     MFMA pipe while one wave waits;
//   * the two waves of a SIMD hide each other's LDS and barrier latency in
//     every mode.
// Per-step scales (FP32 block scales, or the four E8M0 bytes of a row's
// 128-K step) travel by LDS DMA with the tiles, four steps at a time: one
// 16-byte load per tile row and operand every fourth step, 64 rows per wave,
// into a double-buffered chunk.
#include "gemm_common.h"
#include "launch.h"

namespace fp8sg {

namespace {

namespace w8 {

constexpr int BM = 256, BN = 256, NT = 512, NW = 8;
constexpr int WM = 64, WN = 128;           // wave sub-tile

constexpr int NF = WM / 16, NJ = WN / 16;  // fragments per wave: 4 (M) x 8 (N)

// Blockwise promotion of fragment column j: acc[f][j] += s(f, r) * P[f], the
// 128-K partial products of this step times their FP32 scale product.
// With 128-row blocks on B (BRB == 128) the wave's 128 columns share one
// scale, already folded into s[f]; with per-row B scales (BRB == 1) the four
// columns of this lane read theirs from the step's scale words.
template <int BRB>
__device__ __forceinline__ void promote(v4f (&acc)[NF][NJ], const v4f (&P)[NF],
                                        const float (&s)[NF], const uint32_t* S, int sw, int j,
                                        int wn, int g) {
  if constexpr (BRB == 128) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[f][j][r] += s[f] * P[f][r];
  } else {
    const float* Sf = reinterpret_cast<const float*>(S);
    const int n = 256 + wn * WN + j * 16 + 4 * g;   // scale rows of this lane's 4 columns
    const float b[4] = {Sf[n * 4 + sw], Sf[(n + 1) * 4 + sw], Sf[(n + 2) * 4 + sw],
                        Sf[(n + 3) * 4 + sw]};
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[f][j][r] += (s[f] * b[r]) * P[f][r];
  }
}

// SPREAD: the next step's tile loads are issued over the first SPREAD
// fragment columns of a step (1: all at its start).  Spreading keeps the
// texture-address FIFO from filling (both waves of a SIMD would stall on it
// at once) but gives the last loads less time before the step's barrier:
// +5-8 % on the LLaMA2-7B up-projection (K = 4096), -3 to -5 % where the
// long-K operand panels come from the infinity cache or HBM (K >= 5120).
template <int MODE, int FA, int FB, int BRA, int BRB, int SPREAD = 1>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm8(Args p) {
  constexpr bool SCALED = MODE != kTensor;
  __shared__ __attribute__((aligned(1024))) uint8_t lA[2][BM * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t lB[2][BN * BK];
  // per chunk of four steps: row r's words at 4r .. 4r+3; rows 0..255 = A,
  // 256..511 = B
  __shared__ __attribute__((aligned(16))) uint32_t lS[SCALED ? 2 : 1][SCALED ? 2048 : 4];
  // where the scale DMA of a step that starts no chunk lands (zeros)
  __shared__ __attribute__((aligned(16))) uint32_t lS_idle[SCALED && SPREAD > 1 ? 256 : 4];
  int tm, tn;
  if (!tile_coords(p, tm, tn)) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int wm = w >> 1, wn = w & 1;
  const int g = lane >> 4, lr = lane & 15;
  const int64_t K = p.K;
  const int nk = (int)((K + BK - 1) / BK);
  const int64_t m_base = m0 + wm * WM, n_base = n0 + wn * WN;

  v4f acc[NF][NJ];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  TileLoader<BM, NW> la;
  TileLoader<BN, NW> lb;
  la.init(p.A + m0 * K, p.M - m0, K, w);
  lb.init(p.B + n0 * K, p.N - n0, K, w);
  ScaleRows ls;
  if constexpr (SCALED) {
    const int64_t words = K / 128;   // scale words per row: one per 128-K step
    if (w < 4)
      ls.init(p.sa, m0, p.M - m0, MODE == kBlock ? BRA : 1, words, w);
    else
      ls.init(p.sb, n0, p.N - n0, MODE == kBlock ? BRB : 1, words, w - 4);
  }
  auto issue = [&](int stage, int kt) {
    la.load(lA[stage], (int64_t)kt * BK);
    lb.load(lB[stage], (int64_t)kt * BK);
    if constexpr (SCALED)
      if ((kt & 3) == 0)
        ls.load(lds_addr(&lS[(kt >> 2) & 1][((w & 3) * 64 + (w >> 2) * 256) * 4]), kt >> 2);
  };
  // Part `part` of SPREAD of the loads of step kt into `stage`, A and B loads
  // alternating, without branches: live = false (no next step) or a step
  // that starts no scale chunk reads out of range, fetching nothing
  // (zeros land in the unused stage, or in lS_idle).
  constexpr int NLD = 2 * TileLoader<BM, NW>::L;
  auto issue_part = [&](int stage, int kt, int part, bool live) {
#pragma unroll
    for (int i = part * NLD / SPREAD; i < (part + 1) * NLD / SPREAD; ++i) {
      if (i & 1)
        lb.load_one(lB[stage], (int64_t)kt * BK, i >> 1, live);
      else
        la.load_one(lA[stage], (int64_t)kt * BK, i >> 1, live);
    }
    if constexpr (SCALED) {
      if (part == 0) {
        const bool chunk = live && (kt & 3) == 0;
        const uint32_t to = lds_addr(&lS[(kt >> 2) & 1][((w & 3) * 64 + (w >> 2) * 256) * 4]);
        const uint32_t idle = lds_addr(&lS_idle[0]);
        const uint32_t m = 0u - (uint32_t)chunk;
        ls.load((to & m) | (idle & ~m), kt >> 2, chunk);
      }
    }
  };

  if (nk > 0) issue(0, 0);
  wait_vm<0>();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint8_t* As = lA[cur];
    const uint8_t* Bs = lB[cur];
    v8i af[NF], bf[2];
#pragma unroll
    for (int f = 0; f < NF; ++f) af[f] = load_frag(As, wm * WM + f * 16);
    bf[0] = load_frag(Bs, wn * WN);
    // step scales of this lane: word sw of each row in chunk buffer sc
    const int sc = (kt >> 2) & 1, sw = kt & 3;
    float sa_f[NF];
    float sb_u = 0.f;
    int ea[NF], eb[2];
    if constexpr (MODE == kBlock) {
      const float* S = reinterpret_cast<const float*>(lS[sc]);
#pragma unroll
      for (int f = 0; f < NF; ++f) sa_f[f] = S[(wm * WM + f * 16 + lr) * 4 + sw];
      if constexpr (BRB == 128) {
        sb_u = S[(256 + wn * WN) * 4 + sw];
#pragma unroll
        for (int f = 0; f < NF; ++f) sa_f[f] *= sb_u;
      }
    } else if constexpr (MODE == kMX) {
      const uint8_t* S = reinterpret_cast<const uint8_t*>(lS[sc]);
#pragma unroll
      for (int f = 0; f < NF; ++f) ea[f] = S[((wm * WM + f * 16 + lr) * 4 + sw) * 4 + g];
      eb[0] = S[((256 + wn * WN + lr) * 4 + sw) * 4 + g];
    }
    if constexpr (SPREAD == 1) {
      if (kt + 1 < nk) issue(cur ^ 1, kt + 1);
    }
    __builtin_amdgcn_sched_barrier(0);

    v4f P[2][NF];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (SPREAD > 1)
        if (j < SPREAD) issue_part(cur ^ 1, kt + 1, j, kt + 1 < nk);
      if (j + 1 < NJ) bf[(j + 1) & 1] = load_frag(Bs, wn * WN + (j + 1) * 16);
      if constexpr (MODE == kMX) {
        // the next column's B scale byte, one column ahead like its fragment
        if (j + 1 < NJ)
          eb[(j + 1) & 1] = reinterpret_cast<const uint8_t*>(
              lS[sc])[((256 + wn * WN + (j + 1) * 16 + lr) * 4 + sw) * 4 + g];
      }
      if constexpr (MODE == kTensor) {
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f][j] = mfma<FB, FA>(bf[j & 1], af[f], acc[f][j]);
      } else if constexpr (MODE == kMX) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[f][j] = mfma_mx<FB, FA>(bf[j & 1], af[f], acc[f][j], eb[j & 1], ea[f]);
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          P[j & 1][f] = mfma<FB, FA>(bf[j & 1], af[f], v4f{0.f, 0.f, 0.f, 0.f});
        // keep column j's MFMAs ahead of column j-1's promotion: those
        // partial products are complete by now, so the VALU works while the
        // MFMAs of column j run
        __builtin_amdgcn_sched_barrier(0);
        if (j > 0) promote<BRB>(acc, P[(j - 1) & 1], sa_f, lS[sc], sw, j - 1, wn, g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == kBlock)
      promote<BRB>(acc, P[(NJ - 1) & 1], sa_f, lS[sc], sw, NJ - 1, wn, g);
    wait_vm<0>();
    __syncthreads();
  }

  // Epilogue: scale (tensor mode), then BF16 / FP32 / FP32-accumulate stores
  // (and the fused FP8 copy and amax of the BF16 output).
  __shared__ uint32_t red[NT / 64];
  const float qs = p.Cq != nullptr ? *p.q_scale : 1.0f;
  uint32_t mx = 0;
  float s = 1.0f;
  if constexpr (MODE == kTensor)
    s = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sb)[0];
  static_assert(BN * 2 == 512 && 2 * BM * BK == 128 * 512 && 2 * BN * BK == 128 * 512,
                "the output tile is staged as 256 rows of 512 bytes over lA and lB");
  if (p.out == 0 && p.Cq == nullptr && p.part == nullptr && (p.N & 7) == 0) {
    // Plain BF16 output: the tile goes through LDS (free after the main loop's
    // last barrier) so that global stores cover whole rows, 16 bytes per lane,
    // instead of 32-byte pieces of 16 rows per instruction.  256 rows of 512
    // bytes: rows 0-127 over lA, 128-255 over lB; 16-byte chunks XOR-swizzled
    // by row (two lanes per bank at most when writing, none when reading).
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const v4f a = acc[f][j];
        const int r = wm * WM + f * 16 + lr, c = wn * WN + j * 16 + 4 * g;
        uint8_t* row = r < 128 ? &lA[0][0] + r * 512 : &lB[0][0] + (r - 128) * 512;
        *reinterpret_cast<uint2*>(row + (((c >> 3) ^ (r & 31)) << 4) + ((c >> 2) & 1) * 8) =
            make_uint2(pack_bf16x2(a[0] * s, a[1] * s), pack_bf16x2(a[2] * s, a[3] * s));
      }
    __syncthreads();
    const int t = threadIdx.x, ch = t & 31;
#pragma unroll 4
    for (int k = 0; k < BM / 16; ++k) {
      const int r = k * 16 + (t >> 5);
      const int64_t m = m0 + r, n = n0 + ch * 8;
      if (m < p.M && n < p.N) {
        const uint8_t* row = r < 128 ? &lA[0][0] + r * 512 : &lB[0][0] + (r - 128) * 512;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.C) + m * p.N + n) =
            *reinterpret_cast<const uint4*>(row + ((ch ^ (r & 31)) << 4));
      }
    }
    return;
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int64_t m = m_base + f * 16 + lr;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n = n_base + j * 16 + 4 * g;
      if (n >= p.N) continue;
      const v4f a = acc[f][j];
      store4(p, m, n, a[0] * s, a[1] * s, a[2] * s, a[3] * s, qs, mx);
    }
  }
  tile_amax<NT>(p, tm, tn, mx, red);
}

template <int MODE, int FA, int FB, int BRA, int BRB, int SPREAD = 1>
hipError_t run(const GemmProblem& q, hipStream_t s) {
  Args a;
  a.A = q.A; a.B = q.B; a.sa = q.sa; a.sb = q.sb; a.C = q.C; a.out = q.out;
  a.Cq = q.Cq; a.q_scale = q.q_scale; a.q_fmt = q.q_fmt; a.part = q.part;
  a.M = q.M; a.N = q.N; a.K = q.K;
  a.tiles_m = (int)((q.M + BM - 1) / BM);
  a.tiles_n = (int)((q.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm8<MODE, FA, FB, BRA, BRB, SPREAD>), dim3(grid_for_tiles(a.tiles_m * a.tiles_n)),
                     dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int MODE, int BRA, int BRB, int SPREAD = 1>
hipError_t run_fmt(const GemmProblem& q, hipStream_t s) {
  if (q.fa == kE4M3 && q.fb == kE4M3) return run<MODE, kE4M3, kE4M3, BRA, BRB, SPREAD>(q, s);
  if (q.fa == kE5M2 && q.fb == kE4M3) return run<MODE, kE5M2, kE4M3, BRA, BRB, SPREAD>(q, s);
  if (q.fa == kE4M3 && q.fb == kE5M2) return run<MODE, kE4M3, kE5M2, BRA, BRB, SPREAD>(q, s);
  return run<MODE, kE5M2, kE5M2, BRA, BRB, SPREAD>(q, s);
}

}  // namespace w8

}  // namespace

// Blockwise needs K % 128 == 0 (checked by the ABI); MX with K % 128 != 0
// goes to the kernel of gemm_mx_k32.hip.
hipError_t launch_gemm(const GemmProblem& q0, hipStream_t s) {
  if (q0.M == 0 || q0.N == 0) {
    if (q0.amax) return launch_amax_finalize(nullptr, 0, q0.amax, s);
    return hipSuccess;
  }
  GemmProblem q = q0;
  q.part = q.amax ? q.ws : nullptr;   // per-tile maxima in the caller's workspace
  hipError_t err;
  if (q.mode == kTensor)
    err = q.K <= 4096 ? w8::run_fmt<kTensor, 1, 1, 4>(q, s) : w8::run_fmt<kTensor, 1, 1>(q, s);
  else if (q.mode == kMX)
    err = q.K % 128 != 0 ? launch_gemm_mx_k32(q, s) : w8::run_fmt<kMX, 1, 1>(q, s);
  else if (q.bra == 1 && q.brb == 128)
    err = w8::run_fmt<kBlock, 1, 128>(q, s);
  else if (q.bra == 1 && q.brb == 1)
    err = w8::run_fmt<kBlock, 1, 1>(q, s);
  else if (q.bra == 128 && q.brb == 1)
    err = w8::run_fmt<kBlock, 128, 1>(q, s);
  else
    err = w8::run_fmt<kBlock, 128, 128>(q, s);
  if (err != hipSuccess || !q.amax) return err;
  const int T = (int)(((q.M + 255) / 256) * ((q.N + 255) / 256));
  return launch_amax_finalize(q.part, T, q.amax, s);
}

}  // namespace fp8sg
