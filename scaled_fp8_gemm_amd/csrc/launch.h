// launch.h -- internal launchers of libfp8sg (host side).  Arguments have been
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8sg {

int device_cu_count();

// The caller's workspace (FP8_WORKSPACE_BYTES, 256-byte aligned), in words:
//   [0, kWorkspaceWords)            partial maxima (FP32 magnitude bits): at
//                                   most kMaxPartials per quantise launch, one
//                                   per output tile for the GEMM's fused amax
//   [kGridWordsAt, +kGridMaxWords)  grid-wide maxima of the one-launch current
//                                   scaling (two sets, one per tensor of the
//                                   paired launch; arrival masks, maxima,
//                                   flags, claims and the call's generation,
//                                   one 128-byte line each); zero before first
//                                   use, and left ready for the next call by
//                                   every launch
//   [kConfigAt, +kConfigWords)      word 0: bound on the polls of the
//                                   grid-wide wait (0 = the default)
constexpr int kWorkspaceWords = 1 << 16;
constexpr int kGridMaxWords = 260 * 32;
constexpr int kConfigWords = 32;
constexpr int kGridWordsAt = kWorkspaceWords;
constexpr int kConfigAt = kWorkspaceWords + kGridMaxWords;
constexpr int kWorkspaceTotalWords = kConfigAt + kConfigWords;
// Partial maxima of one quantise launch (its largest grid), and the words of
// one grid-wide maximum (a counter and a maximum line per group of 32
// workgroups, a flag line per group, the top counter and maximum line).
constexpr int kMaxPartials = 2048;
constexpr int kGridSetWords = (2 * (kMaxPartials / 32) + 1) * 32;
// Where one current-scaling call reduces: kMaxPartials partial maxima, one
// set of grid-wide maximum words (zero before first use, left ready), and
// the config word (the wait bound, 0 = default).
struct CurrentWs {
  uint32_t* part;
  uint32_t* grid;
  const uint32_t* cfg;
};
inline CurrentWs current_ws(uint32_t* ws) {
  return CurrentWs{ws, ws + kGridWordsAt, ws + kConfigAt};
}
// The library's static scratch on the current device (for
// fp8_quantize_tensor_current_noalloc): kScratchWords words laid out as a
// CurrentWs.  The first call on a device takes its address and clears it
// with a kernel on `s`; nothing is allocated.
constexpr int kScratchWords = kMaxPartials + kGridSetWords + kConfigWords;
hipError_t noalloc_scratch(hipStream_t s, CurrentWs* out);

// Clear a workspace for first use and set its wait bound (a fill kernel).
hipError_t launch_workspace_init(uint32_t* ws, uint32_t wait_polls, hipStream_t s);
// amax[0] = the largest of part[0 .. n-1], as an FP32 value.
hipError_t launch_amax_finalize(const uint32_t* part, int n, float* amax, hipStream_t s);

// in: 0 = BF16 input, 1 = FP32 input
// ws: the caller's workspace (may be NULL where no amax is produced)
hipError_t launch_amax(const void* x, int64_t n, int fmt, float* amax, float* scale,
                       float* scale_inv, uint32_t* ws, hipStream_t s, int in);
hipError_t launch_quantize_tensor(const void* x, int64_t rows, int64_t cols, int fmt,
                                  const float* scale, uint8_t* q, uint8_t* qT, float* amax_out,
                                  uint32_t* ws, hipStream_t s, int in);
// amax -> scale pair -> cast (current scaling): one launch when the tensor fits
// a grid the device holds at once, else two.
hipError_t launch_quantize_current(const void* x, int64_t rows, int64_t cols, int fmt,
                                   uint8_t* q, uint8_t* qT, float* amax, float* scale,
                                   float* scale_inv, const CurrentWs& ws, hipStream_t s, int in);
// One BF16 tensor under current scaling, without a transposed copy.
struct CurrentTensor {
  const void* x;
  int64_t rows, cols;
  int fmt;
  uint8_t* q;
  float* amax;
  float* scale;
  float* scale_inv;
};
// Current scaling of two tensors in one launch when the device holds both
// at once, else one launch_quantize_current each.
hipError_t launch_quantize_pair_current(const CurrentTensor& a, const CurrentTensor& b,
                                        uint32_t* ws, hipStream_t s);
hipError_t launch_history_update(float* hist, int hlen, int64_t step, const float* amax, int fmt,
                                 float* scale, float* scale_inv, hipStream_t s);
hipError_t launch_quantize_block(const void* x, int64_t rows, int64_t cols, int fmt, int br,
                                 uint8_t* q, float* scale_inv, hipStream_t s);
hipError_t launch_quantize_mx(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                              uint8_t* e8m0, hipStream_t s);
// Row-wise copy (optional) and transposed column-wise copy; kind 0: 1x128
// blocks, 1: 128x128 blocks, 2: MX 1x32 blocks.
hipError_t launch_quantize_t(const void* x, int64_t rows, int64_t cols, int fmt, int kind,
                             uint8_t* q, void* sq, uint8_t* qT, void* sqT, hipStream_t s);
hipError_t launch_convert(const float* x, int64_t n, int fmt, uint8_t* q, hipStream_t s);

// C[M][N] (BF16) = A[M][K] . B[N][K]^T with the operands' scales.
// mode: 0 tensor, 1 block (bra/brb = 1 or 128 rows per scale), 2 MX.
struct GemmProblem {
  const uint8_t* A;
  const uint8_t* B;
  const void* sa;
  const void* sb;
  void* C;
  int64_t M, N, K;
  int fa, fb;
  int mode;
  int bra, brb;
  int out;      // 0: BF16 C; 1: FP32 C; 2: FP32 C += result
  // fused epilogue (BF16 output mode): C may be NULL when Cq is given
  uint8_t* Cq;          // FP8 copy of the BF16-rounded output, or NULL
  const float* q_scale; // its scale (device float[1])
  int q_fmt;            // its format
  float* amax;          // amax of the BF16-rounded output, or NULL
  uint32_t* ws;         // the caller's workspace (needed with amax)
  uint32_t* part;       // set by launch_gemm: per-tile maxima for amax
};
hipError_t launch_gemm(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_mx_k32(const GemmProblem& p, hipStream_t s);

}  // namespace fp8sg
