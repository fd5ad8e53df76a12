// Host-side launch helpers shared by the kernel files and the C ABI of libfp8ds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8ds {

// Records a formatted message for fp8_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...);

// Maps a failed kernel launch to FP8DS_ELAUNCH (status -4), else 0.
int check_launch(const char* kernel_name);

int launch_ring_init(void* ring, int hist_len, int fmt, float init_scale, hipStream_t stream);
int launch_quantize(const void* x, int64_t numel, int in_type, int fmt, void* ring, void* y, int max_blocks,
                    hipStream_t stream);
}  // namespace fp8ds
struct fp8_quantize_job;
namespace fp8ds {
int launch_quantize_batch(const fp8_quantize_job* jobs, int njobs, int in_type, int fmt, hipStream_t stream);
int launch_quantize_2d(const void* x, int rows, int cols, int in_type, int fmt, bool dual, void* ring, void* y,
                       void* y_t, int max_blocks, hipStream_t stream);
int launch_amax(const void* x, int64_t numel, int in_type, int fmt, void* ring, hipStream_t stream);
size_t bias_grad_workspace(int64_t rows, int64_t cols);
int launch_bias_grad(const void* g, int rows, int cols, int g_type, const float* g_scale_inv, int out_f32, void* out,
                     void* workspace, hipStream_t stream);
// The bias gradient with its scratch in the library's own device array (no
// workspace argument, nothing allocated); FP8DS_EUNSUPPORTED past its size.
int launch_bias_grad_noalloc(const void* g, int rows, int cols, int g_type, const float* g_scale_inv, int out_f32,
                             void* out, hipStream_t stream);

struct GemmProblem {
  const uint8_t* a;
  const uint8_t* b;
  uint16_t* c;
  int fmt_a, fmt_b, layout, bias_kind;
  int m, n, k, batch;
  int64_t lda, ldb, ldc;
  int64_t stride_a, stride_b, stride_c;
  uint32_t extent_a, extent_b;   // bytes one batch entry of each operand spans, rounded up to 16
  const float* a_scale_inv;
  const float* b_scale_inv;
  const void* bias;
  const float* bias_scale_inv;   // 8-bit bias only
};

// tile_override < 0 picks the tile; max_workgroups <= 0 sizes the grid to the
// workgroups the device holds at once.
int launch_gemm(const GemmProblem& p, int tile_override, int max_workgroups, hipStream_t stream);

// Two independent problems; one launch when p0 is NN and p1 TN in the same
// formats (a layer's dX and dW), else two launches in order.
int launch_gemm_pair(const GemmProblem& p0, const GemmProblem& p1, hipStream_t stream);

// The tile launch_gemm picks for p, and the one launch_gemm_pair runs a pair
// on (-1: two launches).  Host arithmetic only.
int gemm_tile(const GemmProblem& p);
int gemm_pair_tile(const GemmProblem& p0, const GemmProblem& p1);

}  // namespace fp8ds
