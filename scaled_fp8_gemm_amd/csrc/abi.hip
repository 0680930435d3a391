// abi.hip -- the extern "C" entry points of libfp8sg (declared and documented
// in include/fp8sg.h).  Each call checks its arguments on the host, in the
// order NULL -> enum -> shape -> alignment (a NULL data pointer is accepted
// for an empty tensor, so the NULL check of data follows the shape check),
// and only then enqueues kernels on the caller's stream.  Nothing here or
// in the launchers allocates or synchronises, and the only state kept
// between calls is read-only device facts cached per device (CU count,
// occupancy-derived grid sizes): the amax-producing calls reduce through
// the caller's workspace.  The one exception is
// fp8_quantize_tensor_current_noalloc, which reduces through a static device
// array and keeps its address per device.
#include "fp8sg.h"

#include <stdint.h>

#include "launch.h"

namespace {

using fp8sg::GemmProblem;

constexpr int64_t kMaxDim = (int64_t)1 << 31;           // rows / cols limit
constexpr int64_t kMaxTileRows = (int64_t)65535 * 128;  // 2-D launch grid limit
// GEMM contraction limit: the kernels address a 256-row operand tile with
// 32-bit buffer offsets (256 * K < 2^31).
constexpr int64_t kMaxContraction = (int64_t)1 << 23;

bool fmt_ok(int32_t f) { return f == FP8_E4M3 || f == FP8_E5M2; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool dims_ok(int64_t r, int64_t c) { return r >= 0 && c >= 0 && r < kMaxDim && c < kMaxDim; }
fp8_status_t hip(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_HIP; }
hipStream_t st(void* s) { return reinterpret_cast<hipStream_t>(s); }

// A data pointer may be NULL only when the tensor it points to is empty.
bool have(const void* p, int64_t elems) { return p != nullptr || elems == 0; }

bool is_block(int32_t sc) { return sc == FP8_SCALE_BLOCK_1x128 || sc == FP8_SCALE_BLOCK_128x128; }

// The caller's workspace: FP8_WORKSPACE_BYTES of device memory, 256-byte
// aligned (the grid-wide maximum's words sit in whole 128-byte lines).
static_assert(FP8_WORKSPACE_BYTES == fp8sg::kWorkspaceTotalWords * 4, "workspace size");
uint32_t* wsp(void* ws) { return static_cast<uint32_t*>(ws); }

// C[rows_a][rows_b] = A[rows_a][kc] . B[rows_b][kc]^T with the operands' scales.
// Optional fused epilogue of the BF16 mode: the next layer's FP8 copy of the
// output (with its scale and format) and the output's amax.
struct Fused {
  uint8_t* cq = nullptr;
  const float* q_scale = nullptr;
  int q_fmt = 0;
  float* amax = nullptr;
  void* ws = nullptr;       // the caller's workspace (with amax)
};

fp8_status_t gemm(const fp8_operand_t* a, const fp8_operand_t* b, int64_t rows_a,
                  int64_t rows_b, int64_t kc, void* c, void* stream, int out = 0,
                  const Fused& fu = Fused()) {
  const bool fused = fu.cq != nullptr || fu.amax != nullptr;
  if (!a || !b) return FP8_ERR_NULL;
  if (!fmt_ok(a->fmt) || !fmt_ok(b->fmt) || (fu.cq && !fmt_ok(fu.q_fmt)))
    return FP8_ERR_UNSUPPORTED;
  if (a->scaling < FP8_SCALE_TENSOR || a->scaling > FP8_SCALE_MX_1x32 ||
      b->scaling < FP8_SCALE_TENSOR || b->scaling > FP8_SCALE_MX_1x32)
    return FP8_ERR_UNSUPPORTED;
  int mode;
  if (a->scaling == FP8_SCALE_TENSOR && b->scaling == FP8_SCALE_TENSOR)
    mode = 0;
  else if (is_block(a->scaling) && is_block(b->scaling))
    mode = 1;
  else if (a->scaling == FP8_SCALE_MX_1x32 && b->scaling == FP8_SCALE_MX_1x32)
    mode = 2;
  else
    return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows_a, kc) || !dims_ok(rows_b, kc)) return FP8_ERR_SHAPE;
  if (kc > kMaxContraction) return FP8_ERR_SHAPE;
  const int64_t nc = rows_a * rows_b;
  // the output may be NULL when it is empty, or in the fused call when the
  // FP8 copy is written instead
  const bool c_ok = have(c, nc) || fu.cq != nullptr;
  if (!have(a->data, rows_a * kc) || !have(b->data, rows_b * kc) || !c_ok ||
      !have(a->scale_inv, nc) || !have(b->scale_inv, nc) || (fu.cq && !fu.q_scale) ||
      (fu.amax && !fu.ws))
    return FP8_ERR_NULL;
  if (mode == 1) {
    if (kc % 128) return FP8_ERR_SHAPE;
    if (a->scaling == FP8_SCALE_BLOCK_128x128 && rows_a % 128) return FP8_ERR_SHAPE;
    if (b->scaling == FP8_SCALE_BLOCK_128x128 && rows_b % 128) return FP8_ERR_SHAPE;
  }
  if (mode == 2 && kc % 32) return FP8_ERR_SHAPE;
  if (fused && ((rows_a + 255) / 256) * ((rows_b + 255) / 256) > fp8sg::kWorkspaceWords)
    return FP8_ERR_SHAPE;
  if (kc % 16) return FP8_ERR_ALIGN;
  if (!aligned(a->data, 16) || !aligned(b->data, 16) || !aligned(c, 16)) return FP8_ERR_ALIGN;
  if (fused && (rows_b % 16 || !aligned(fu.cq, 16) || !aligned(fu.q_scale, 4) ||
                !aligned(fu.amax, 4) || !aligned(fu.ws, 256)))
    return FP8_ERR_ALIGN;
  if (mode != 2 && (!aligned(a->scale_inv, 4) || !aligned(b->scale_inv, 4)))
    return FP8_ERR_ALIGN;
  GemmProblem p;
  p.A = a->data;
  p.B = b->data;
  p.sa = a->scale_inv;
  p.sb = b->scale_inv;
  p.C = c;
  p.out = out;
  p.Cq = fu.cq;
  p.q_scale = fu.q_scale;
  p.q_fmt = fu.q_fmt;
  p.amax = fu.amax;
  p.ws = wsp(fu.ws);
  p.part = nullptr;
  p.M = rows_a;
  p.N = rows_b;
  p.K = kc;
  p.fa = a->fmt;
  p.fb = b->fmt;
  p.mode = mode;
  p.bra = a->scaling == FP8_SCALE_BLOCK_128x128 ? 128 : 1;
  p.brb = b->scaling == FP8_SCALE_BLOCK_128x128 ? 128 : 1;
  return hip(fp8sg::launch_gemm(p, st(stream)));
}

// amax / per-tensor cast of BF16 (in = 0) or FP32 (in = 1) input.
fp8_status_t amax_any(const void* x, int64_t rows, int64_t cols, int32_t fmt, float* amax,
                      float* scale, float* scale_inv, void* ws, void* stream, int in) {
  if (!amax || !ws) return FP8_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (!have(x, rows * cols)) return FP8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(amax, 4) || (scale && !aligned(scale, 4)) ||
      (scale_inv && !aligned(scale_inv, 4)) || !aligned(ws, 256))
    return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_amax(x, rows * cols, fmt, amax, scale, scale_inv, wsp(ws), st(stream),
                                in));
}

fp8_status_t quantize_tensor_any(const void* x, int64_t rows, int64_t cols, int32_t fmt,
                                 const float* scale, uint8_t* q, uint8_t* qT, float* amax_out,
                                 void* ws, void* stream, int in) {
  if (amax_out && !ws) return FP8_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (!have(x, rows * cols) || !have(q, rows * cols) || !have(scale, rows * cols))
    return FP8_ERR_NULL;
  if (cols % 16) return FP8_ERR_ALIGN;
  if (qT && rows % 16) return FP8_ERR_ALIGN;
  if (!aligned(x, 16) || !aligned(q, 16) || (qT && !aligned(qT, 16)) || !aligned(scale, 4) ||
      (amax_out && (!aligned(amax_out, 4) || !aligned(ws, 256))))
    return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_quantize_tensor(x, rows, cols, fmt, scale, q, qT, amax_out,
                                           amax_out ? wsp(ws) : nullptr, st(stream), in));
}

}  // namespace

extern "C" {

fp8_status_t fp8_workspace_init(void* workspace, int32_t wait_polls, void* stream) {
  if (!workspace) return FP8_ERR_NULL;
  if (wait_polls < 0) return FP8_ERR_SHAPE;
  if (!aligned(workspace, 256)) return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_workspace_init(wsp(workspace), (uint32_t)wait_polls, st(stream)));
}

fp8_status_t fp8_amax(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt, float* amax,
                      float* scale, float* scale_inv, void* workspace, void* stream) {
  return amax_any(x_bf16, rows, cols, fmt, amax, scale, scale_inv, workspace, stream, 0);
}

fp8_status_t fp8_amax_f32(const float* x_f32, int64_t rows, int64_t cols, int32_t fmt,
                          float* amax, float* scale, float* scale_inv, void* workspace,
                          void* stream) {
  return amax_any(x_f32, rows, cols, fmt, amax, scale, scale_inv, workspace, stream, 1);
}

fp8_status_t fp8_quantize_tensor(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                                 const float* scale, uint8_t* q, uint8_t* qT, float* amax_out,
                                 void* workspace, void* stream) {
  return quantize_tensor_any(x_bf16, rows, cols, fmt, scale, q, qT, amax_out, workspace, stream,
                             0);
}

fp8_status_t fp8_quantize_tensor_current(const void* x_bf16, int64_t rows, int64_t cols,
                                         int32_t fmt, uint8_t* q, uint8_t* qT, float* amax,
                                         float* scale, float* scale_inv, void* workspace,
                                         void* stream) {
  if (!amax || !scale_inv || !workspace) return FP8_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (!have(x_bf16, rows * cols) || !have(q, rows * cols)) return FP8_ERR_NULL;
  if (cols % 16) return FP8_ERR_ALIGN;
  if (qT && rows % 16) return FP8_ERR_ALIGN;
  if (!aligned(x_bf16, 16) || !aligned(q, 16) || (qT && !aligned(qT, 16)) ||
      !aligned(amax, 4) || !aligned(scale_inv, 4) || (scale && !aligned(scale, 4)) ||
      !aligned(workspace, 256))
    return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_quantize_current(x_bf16, rows, cols, fmt, q, qT, amax, scale,
                                            scale_inv, fp8sg::current_ws(wsp(workspace)),
                                            st(stream), 0));
}

fp8_status_t fp8_quantize_tensor_current_noalloc(const void* x_bf16, int64_t rows, int64_t cols,
                                                 int32_t fmt, uint8_t* q, uint8_t* qT,
                                                 float* amax, float* scale, float* scale_inv,
                                                 void* stream) {
  if (!amax || !scale_inv) return FP8_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (!have(x_bf16, rows * cols) || !have(q, rows * cols)) return FP8_ERR_NULL;
  if (cols % 16) return FP8_ERR_ALIGN;
  if (qT && rows % 16) return FP8_ERR_ALIGN;
  if (!aligned(x_bf16, 16) || !aligned(q, 16) || (qT && !aligned(qT, 16)) ||
      !aligned(amax, 4) || !aligned(scale_inv, 4) || (scale && !aligned(scale, 4)))
    return FP8_ERR_ALIGN;
  // the static scratch holds what any tensor needs: a quantise launch writes
  // at most kMaxPartials partial maxima, whatever its size
  fp8sg::CurrentWs ws;
  const hipError_t err = fp8sg::noalloc_scratch(st(stream), &ws);
  if (err != hipSuccess) return FP8_ERR_HIP;
  return hip(fp8sg::launch_quantize_current(x_bf16, rows, cols, fmt, q, qT, amax, scale,
                                            scale_inv, ws, st(stream), 0));
}

static fp8_status_t current_ok(const void* x, int64_t rows, int64_t cols, int32_t fmt,
                               const uint8_t* q, const float* amax, const float* scale,
                               const float* scale_inv) {
  if (!amax || !scale_inv) return FP8_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (!have(x, rows * cols) || !have(q, rows * cols)) return FP8_ERR_NULL;
  if (cols % 16) return FP8_ERR_ALIGN;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(amax, 4) || !aligned(scale_inv, 4) ||
      (scale && !aligned(scale, 4)))
    return FP8_ERR_ALIGN;
  return FP8_OK;
}

fp8_status_t fp8_quantize_pair_current(const void* a_bf16, int64_t a_rows, int64_t a_cols,
                                       int32_t a_fmt, uint8_t* a_q, float* a_amax,
                                       float* a_scale, float* a_scale_inv, const void* b_bf16,
                                       int64_t b_rows, int64_t b_cols, int32_t b_fmt,
                                       uint8_t* b_q, float* b_amax, float* b_scale,
                                       float* b_scale_inv, void* workspace, void* stream) {
  if (!workspace) return FP8_ERR_NULL;
  fp8_status_t e = current_ok(a_bf16, a_rows, a_cols, a_fmt, a_q, a_amax, a_scale, a_scale_inv);
  if (e != FP8_OK) return e;
  e = current_ok(b_bf16, b_rows, b_cols, b_fmt, b_q, b_amax, b_scale, b_scale_inv);
  if (e != FP8_OK) return e;
  if (!aligned(workspace, 256)) return FP8_ERR_ALIGN;
  const fp8sg::CurrentTensor ta{a_bf16, a_rows, a_cols, a_fmt, a_q, a_amax, a_scale, a_scale_inv};
  const fp8sg::CurrentTensor tb{b_bf16, b_rows, b_cols, b_fmt, b_q, b_amax, b_scale, b_scale_inv};
  return hip(fp8sg::launch_quantize_pair_current(ta, tb, wsp(workspace), st(stream)));
}

fp8_status_t fp8_quantize_tensor_f32(const float* x_f32, int64_t rows, int64_t cols, int32_t fmt,
                                     const float* scale, uint8_t* q, uint8_t* qT,
                                     float* amax_out, void* workspace, void* stream) {
  return quantize_tensor_any(x_f32, rows, cols, fmt, scale, q, qT, amax_out, workspace, stream, 1);
}

fp8_status_t fp8_amax_history_update(float* history, int32_t history_len, int64_t step,
                                     const float* amax, int32_t fmt, float* scale,
                                     float* scale_inv, void* stream) {
  if (!history || !amax || !scale || !scale_inv) return FP8_ERR_NULL;
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (history_len < 1 || history_len > 1024 || step < 0) return FP8_ERR_SHAPE;
  if (!aligned(history, 4) || !aligned(amax, 4) || !aligned(scale, 4) || !aligned(scale_inv, 4))
    return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_history_update(history, history_len, step, amax, fmt, scale,
                                          scale_inv, st(stream)));
}

fp8_status_t fp8_quantize_block(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                                int32_t block_rows, int32_t block_cols, uint8_t* q,
                                float* scale_inv, void* stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (!have(x_bf16, rows * cols) || !have(q, rows * cols) || !have(scale_inv, rows * cols))
    return FP8_ERR_NULL;
  if ((block_rows != 1 && block_rows != 128) || block_cols != 128) return FP8_ERR_UNSUPPORTED;
  if (cols % 128 || rows % block_rows) return FP8_ERR_SHAPE;
  if (block_rows == 128 && rows > kMaxTileRows) return FP8_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(scale_inv, 4)) return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_quantize_block(x_bf16, rows, cols, fmt, block_rows, q, scale_inv,
                                          st(stream)));
}

fp8_status_t fp8_quantize_block_t(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                                  int32_t block_rows, uint8_t* q, float* scale_inv, uint8_t* qT,
                                  float* scale_inv_T, void* stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (!have(x_bf16, n) || !have(qT, n) || !have(scale_inv_T, n)) return FP8_ERR_NULL;
  if ((q == nullptr) != (scale_inv == nullptr)) return FP8_ERR_NULL;
  if (block_rows != 1 && block_rows != 128) return FP8_ERR_UNSUPPORTED;
  if (rows % 128 || cols % 128) return FP8_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(qT, 16) || !aligned(scale_inv_T, 4) ||
      (q && (!aligned(q, 16) || !aligned(scale_inv, 4))))
    return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_quantize_t(x_bf16, rows, cols, fmt, block_rows == 1 ? 0 : 1, q,
                                      scale_inv, qT, scale_inv_T, st(stream)));
}

fp8_status_t fp8_quantize_mx_t(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                               uint8_t* q, uint8_t* scale_e8m0, uint8_t* qT,
                               uint8_t* scale_e8m0_T, void* stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return FP8_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (!have(x_bf16, n) || !have(qT, n) || !have(scale_e8m0_T, n)) return FP8_ERR_NULL;
  if ((q == nullptr) != (scale_e8m0 == nullptr)) return FP8_ERR_NULL;
  if (rows % 32 || cols % 32) return FP8_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(qT, 16) || (q && !aligned(q, 16))) return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_quantize_t(x_bf16, rows, cols, fmt, 2, q, scale_e8m0, qT,
                                      scale_e8m0_T, st(stream)));
}

fp8_status_t fp8_quantize_mx(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                             uint8_t* q, uint8_t* scale_e8m0, void* stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols) || cols % 32) return FP8_ERR_SHAPE;
  if (!have(x_bf16, rows * cols) || !have(q, rows * cols) || !have(scale_e8m0, rows * cols))
    return FP8_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_quantize_mx(x_bf16, rows, cols, fmt, q, scale_e8m0, st(stream)));
}

fp8_status_t fp8_gemm_fprop(const fp8_operand_t* x, const fp8_operand_t* w, int64_t M, int64_t N,
                            int64_t K, void* y_bf16, void* stream) {
  return gemm(x, w, M, N, K, y_bf16, stream);
}

fp8_status_t fp8_gemm_dgrad(const fp8_operand_t* dy, const fp8_operand_t* wT, int64_t M,
                            int64_t N, int64_t K, void* dx_bf16, void* stream) {
  return gemm(dy, wT, M, K, N, dx_bf16, stream);
}

fp8_status_t fp8_gemm_wgrad(const fp8_operand_t* dyT, const fp8_operand_t* xT, int64_t M,
                            int64_t N, int64_t K, void* dw_bf16, void* stream) {
  return gemm(dyT, xT, N, K, M, dw_bf16, stream);
}

fp8_status_t fp8_gemm_fprop_fused(const fp8_operand_t* x, const fp8_operand_t* w, int64_t M,
                                  int64_t N, int64_t K, void* y_bf16, int32_t y_fmt,
                                  const float* y_scale, uint8_t* y_q, float* y_amax,
                                  void* workspace, void* stream) {
  Fused fu;
  fu.cq = y_q;
  fu.q_scale = y_scale;
  fu.q_fmt = y_fmt;
  fu.amax = y_amax;
  fu.ws = workspace;
  if (!y_q && !y_amax) return FP8_ERR_NULL;   // use fp8_gemm_fprop
  return gemm(x, w, M, N, K, y_bf16, stream, 0, fu);
}

fp8_status_t fp8_gemm_wgrad_f32(const fp8_operand_t* dyT, const fp8_operand_t* xT, int64_t M,
                                int64_t N, int64_t K, float* dw_f32, int32_t accumulate,
                                void* stream) {
  if (accumulate != 0 && accumulate != 1) return FP8_ERR_UNSUPPORTED;
  return gemm(dyT, xT, N, K, M, dw_f32, stream, accumulate ? 2 : 1);
}

fp8_status_t fp8_convert_f32(const float* x, int64_t n, int32_t fmt, uint8_t* q, void* stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_UNSUPPORTED;
  if (n < 0) return FP8_ERR_SHAPE;
  if (!have(x, n) || !have(q, n)) return FP8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16)) return FP8_ERR_ALIGN;
  return hip(fp8sg::launch_convert(x, n, fmt, q, st(stream)));
}

const char* fp8_status_string(fp8_status_t status) {
  switch (status) {
    case FP8_OK: return "FP8_OK";
    case FP8_ERR_NULL: return "FP8_ERR_NULL: a required pointer is NULL";
    case FP8_ERR_SHAPE: return "FP8_ERR_SHAPE: size out of range or not a block multiple";
    case FP8_ERR_ALIGN: return "FP8_ERR_ALIGN: pointer or row length not aligned";
    case FP8_ERR_UNSUPPORTED: return "FP8_ERR_UNSUPPORTED: unknown enum or unsupported combination";
    case FP8_ERR_HIP: return "FP8_ERR_HIP: kernel launch failed";
  }
  return "unknown fp8_status_t";
}

}  // extern "C"
