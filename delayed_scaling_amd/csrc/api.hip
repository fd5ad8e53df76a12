// C ABI of libfp8ds: argument validation, dispatch to the kernels, errors.
// The declarations and their contracts are in include/fp8ds.h.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fp8ds.h"
#include "launch.h"

namespace fp8ds {

namespace {
thread_local char g_err[512] = "";
}

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* kernel_name) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(FP8DS_ELAUNCH, "%s: launch failed: %s", kernel_name, hipGetErrorString(e));
  return FP8DS_OK;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_fmt(int f) { return f == FP8DS_E4M3 || f == FP8DS_E5M2; }
bool valid_in(int t) { return t == FP8DS_IN_BF16 || t == FP8DS_IN_F16 || t == FP8DS_IN_F32; }
int64_t in_size(int t) { return t == FP8DS_IN_F32 ? 4 : 2; }
// True when the byte ranges [a, a + a_bytes) and [b, b + b_bytes) share a
// byte; an empty range overlaps nothing.
bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  if (a_bytes <= 0 || b_bytes <= 0 || !a || !b) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)b_bytes && y < x + (uintptr_t)a_bytes;
}

// Checks shared by the 1-D quantize entry points; FP8DS_OK when launchable.
int check_quantize(const char* fn, const void* x, int64_t numel, int in_type, int fmt, const void* ring,
                   const void* y, int max_blocks) {
  if (max_blocks < 0 || max_blocks > (1 << 20))
    return set_error(FP8DS_EINVAL, "%s: max_blocks %d outside [0, 2^20]", fn, max_blocks);
  if (!valid_in(in_type)) return set_error(FP8DS_EINVAL, "%s: in_type %d is not bf16 (0), fp16 (1) or fp32 (2)", fn, in_type);
  if (!valid_fmt(fmt)) return set_error(FP8DS_EINVAL, "%s: fmt %d is neither E4M3 (0) nor E5M2 (1)", fn, fmt);
  if (numel < 0) return set_error(FP8DS_EINVAL, "%s: numel %lld < 0", fn, (long long)numel);
  if (!ring) return set_error(FP8DS_EUNSUPPORTED, "%s: ring is NULL (use fp8_quantize_dynamic for dynamic scaling)", fn);
  if (!aligned16(ring)) return set_error(FP8DS_EALIGN, "%s: ring not 16-byte aligned", fn);
  if (numel == 0) return FP8DS_OK;
  if (!x || !y) return set_error(FP8DS_EINVAL, "%s: x or y is NULL", fn);
  if (!aligned16(x) || !aligned16(y)) return set_error(FP8DS_EALIGN, "%s: x or y not 16-byte aligned", fn);
  if (overlaps(x, numel * in_size(in_type), y, numel)) return set_error(FP8DS_EINVAL, "%s: x and y overlap", fn);
  return FP8DS_OK;
}
constexpr int64_t kMaxDim = 0x7FFFFFFF;

// Checks shared by the two bias-gradient entry points; FP8DS_OK with
// *nothing set when there is nothing to do (no columns).
int check_bias_grad(const char* fn, const void* g, int64_t rows, int64_t cols, int g_type, const float* g_scale_inv,
                    const void* out, bool need_workspace, const void* workspace, bool* nothing) {
  *nothing = false;
  if (g_type < FP8DS_G_BF16 || g_type > FP8DS_G_E5M2) return set_error(FP8DS_EINVAL, "%s: bad g_type %d", fn, g_type);
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim)
    return set_error(FP8DS_EINVAL, "%s: rows and cols must be in [0, 2^31)", fn);
  if (cols == 0) {
    *nothing = true;
    return FP8DS_OK;
  }
  if (!out || (need_workspace && !workspace) || (rows > 0 && !g))
    return set_error(FP8DS_EINVAL, "%s: g, out or workspace is NULL", fn);
  const bool codes = g_type == FP8DS_G_E4M3 || g_type == FP8DS_G_E5M2;
  if (codes && !g_scale_inv) return set_error(FP8DS_EINVAL, "%s: 8-bit g needs g_scale_inv", fn);
  if (cols & 7) return set_error(FP8DS_EALIGN, "%s: cols %lld is not a multiple of 8", fn, (long long)cols);
  if ((rows > 0 && !aligned16(g)) || (need_workspace && !aligned16(workspace)))
    return set_error(FP8DS_EALIGN, "%s: g or workspace not 16-byte aligned", fn);
  const int64_t esize = g_type == FP8DS_G_F32 ? 4 : codes ? 1 : 2;
  if (rows * cols * esize >= (int64_t)1 << 40) return set_error(FP8DS_EUNSUPPORTED, "%s: g too large", fn);
  return FP8DS_OK;
}


// Largest byte offset + 1 that one batch entry of a stored [rows][cols] view
// with leading dimension ld touches, rounded up to 16.
int64_t view_extent(int64_t rows, int64_t cols, int64_t ld) {
  if (rows == 0 || cols == 0) return 0;
  const int64_t e = (rows - 1) * ld + cols;
  return (e + 15) & ~int64_t(15);
}

}  // namespace
}  // namespace fp8ds

namespace fp8ds {
namespace {

// Bytes from c that a problem's output spans, and likewise its operands
// (stride 0 broadcasts span one entry) and its bias.
int64_t mm_c_bytes(const GemmProblem& p) {
  return ((int64_t)(p.batch - 1) * p.stride_c + (int64_t)(p.m - 1) * p.ldc + p.n) * 2;
}
int64_t mm_operand_bytes(uint32_t extent, const GemmProblem& p, bool is_b = false) {
  if (p.k == 0) return 0;
  return (int64_t)(p.batch - 1) * (is_b ? p.stride_b : p.stride_a) + extent;
}
int64_t mm_bias_bytes(const GemmProblem& p) {
  const int64_t e = p.bias_kind == FP8DS_BIAS_F32 ? 4 : p.bias_kind == FP8DS_BIAS_BF16 ? 2 : 1;
  return p.n * e;
}

int check_mm(const fp8_mm_args* a, GemmProblem* out, bool* empty) {
  if (!a) return set_error(FP8DS_EINVAL, "fp8_mm: args is NULL");
  if (!valid_fmt(a->fmt_a) || !valid_fmt(a->fmt_b)) return set_error(FP8DS_EINVAL, "fp8_mm: bad fmt_a/fmt_b");
  if (a->layout < FP8DS_NT || a->layout > FP8DS_TN) return set_error(FP8DS_EINVAL, "fp8_mm: bad layout %d", a->layout);
  if (a->bias_kind < FP8DS_BIAS_NONE || a->bias_kind > FP8DS_BIAS_E5M2)
    return set_error(FP8DS_EINVAL, "fp8_mm: bad bias_kind %d", a->bias_kind);
  if ((a->bias_kind == FP8DS_BIAS_E4M3 || a->bias_kind == FP8DS_BIAS_E5M2) && !a->bias_scale_inv)
    return set_error(FP8DS_EINVAL, "fp8_mm: an 8-bit bias needs bias_scale_inv");
  const int64_t m = a->m, n = a->n, k = a->k, batch = a->batch == 0 ? 1 : a->batch;
  if (m < 0 || n < 0 || k < 0 || batch < 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim || batch > kMaxDim)
    return set_error(FP8DS_EINVAL, "fp8_mm: dimensions must be in [0, 2^31)");
  if (m == 0 || n == 0) {
    *empty = true;
    return FP8DS_OK;
  }
  const bool tn = a->layout == FP8DS_TN;
  const int64_t a_rows = tn ? k : m, a_cols = tn ? m : k;
  const int64_t b_rows = a->layout == FP8DS_NT ? n : k, b_cols = a->layout == FP8DS_NT ? k : n;
  if (!a->c || !a->a_scale_inv || !a->b_scale_inv) return set_error(FP8DS_EINVAL, "fp8_mm: c or a scale pointer is NULL");
  if (k > 0 && (!a->a || !a->b)) return set_error(FP8DS_EINVAL, "fp8_mm: a or b is NULL");
  if (a->bias_kind != FP8DS_BIAS_NONE && !a->bias) return set_error(FP8DS_EINVAL, "fp8_mm: bias_kind set but bias is NULL");
  if (a->lda < (k > 0 ? a_cols : 0) || a->ldb < (k > 0 ? b_cols : 0) || a->ldc < n)
    return set_error(FP8DS_EINVAL, "fp8_mm: leading dimension smaller than the row length");
  if (a->stride_a < 0 || a->stride_b < 0 || a->stride_c < 0) return set_error(FP8DS_EINVAL, "fp8_mm: negative stride");
  if (batch > 1 && a->stride_c < m * a->ldc) return set_error(FP8DS_EINVAL, "fp8_mm: stride_c smaller than one output");
  if ((k > 0 && (!aligned16(a->a) || !aligned16(a->b))) || !aligned16(a->c) ||
      (a->bias_kind != FP8DS_BIAS_NONE && !aligned16(a->bias)))
    return set_error(FP8DS_EALIGN, "fp8_mm: a, b, c and bias must be 16-byte aligned");
  if ((a->lda & 15) || (a->ldb & 15) || (a->ldc & 7) || (a->stride_a & 15) || (a->stride_b & 15) ||
      (a->stride_c & 7))
    return set_error(FP8DS_EALIGN, "fp8_mm: lda, ldb, strides of a/b must be multiples of 16, ldc and stride_c of 8");
  const int64_t ext_a = k > 0 ? view_extent(a_rows, a_cols, a->lda) : 0;
  const int64_t ext_b = k > 0 ? view_extent(b_rows, b_cols, a->ldb) : 0;
  if (ext_a >= 0x80000000LL || ext_b >= 0x80000000LL)
    return set_error(FP8DS_EUNSUPPORTED, "fp8_mm: one batch entry of an operand spans 2 GiB or more");
  GemmProblem p{};
  p.a = static_cast<const uint8_t*>(a->a);
  p.b = static_cast<const uint8_t*>(a->b);
  p.c = static_cast<uint16_t*>(a->c);
  p.fmt_a = a->fmt_a;
  p.fmt_b = a->fmt_b;
  p.layout = a->layout;
  p.bias_kind = a->bias_kind;
  p.m = (int)m;
  p.n = (int)n;
  p.k = (int)k;
  p.batch = (int)batch;
  p.lda = a->lda;
  p.ldb = a->ldb;
  p.ldc = a->ldc;
  p.stride_a = a->stride_a;
  p.stride_b = a->stride_b;
  p.stride_c = a->stride_c;
  p.extent_a = (uint32_t)ext_a;
  p.extent_b = (uint32_t)ext_b;
  p.a_scale_inv = a->a_scale_inv;
  p.b_scale_inv = a->b_scale_inv;
  p.bias = a->bias;
  p.bias_scale_inv = a->bias_scale_inv;
  // The output is written while the operands and the bias are still read.
  const int64_t c_bytes = mm_c_bytes(p);
  if (overlaps(p.c, c_bytes, p.a, mm_operand_bytes(p.extent_a, p)) ||
      overlaps(p.c, c_bytes, p.b, mm_operand_bytes(p.extent_b, p, true)) ||
      (p.bias_kind != FP8DS_BIAS_NONE && overlaps(p.c, c_bytes, p.bias, mm_bias_bytes(p))))
    return set_error(FP8DS_EINVAL, "fp8_mm: c overlaps a, b or bias");
  *out = p;
  return FP8DS_OK;
}

}  // namespace
}  // namespace fp8ds

using namespace fp8ds;

extern "C" {

const char* fp8_last_error(void) { return g_err; }

size_t fp8_scale_ring_bytes(int hist_len) {
  if (hist_len < 1 || hist_len > FP8DS_RING_MAX_HIST) return 0;
  return (size_t)FP8DS_RING_HIST_OFFSET + (((size_t)hist_len * 4 + 15) & ~(size_t)15);
}

const float* fp8_ring_scale_inv(const void* ring) {
  return ring ? reinterpret_cast<const float*>(static_cast<const char*>(ring) + 4) : nullptr;
}

int scale_ring_init(void* ring, int hist_len, int fmt, float init_scale, void* stream) {
  if (!ring) return set_error(FP8DS_EINVAL, "scale_ring_init: ring is NULL");
  if (!aligned16(ring)) return set_error(FP8DS_EALIGN, "scale_ring_init: ring not 16-byte aligned");
  if (hist_len < 1 || hist_len > FP8DS_RING_MAX_HIST)
    return set_error(FP8DS_EINVAL, "scale_ring_init: hist_len %d outside [1, %d]", hist_len, FP8DS_RING_MAX_HIST);
  if (!valid_fmt(fmt)) return set_error(FP8DS_EINVAL, "scale_ring_init: fmt %d is neither E4M3 (0) nor E5M2 (1)", fmt);
  if (!(init_scale > 0.0f) || !(init_scale < __builtin_inff()))
    return set_error(FP8DS_EINVAL, "scale_ring_init: init_scale must be finite and > 0");
  return launch_ring_init(ring, hist_len, fmt, init_scale, static_cast<hipStream_t>(stream));
}

int fp8_quantize(const void* x_bf16, int64_t numel, int fmt, void* ring, void* y_fp8, void* stream) {
  return fp8_quantize_with_grid(x_bf16, numel, fmt, ring, y_fp8, 0, stream);
}

int fp8_quantize_with_grid(const void* x_bf16, int64_t numel, int fmt, void* ring, void* y_fp8, int max_blocks,
                           void* stream) {
  const int st = check_quantize("fp8_quantize", x_bf16, numel, FP8DS_IN_BF16, fmt, ring, y_fp8, max_blocks);
  if (st != FP8DS_OK || numel == 0) return st;
  return launch_quantize(x_bf16, numel, FP8DS_IN_BF16, fmt, ring, y_fp8, max_blocks, static_cast<hipStream_t>(stream));
}

int fp8_quantize_ex(const void* x, int64_t numel, int in_type, int fmt, void* ring, void* y_fp8, void* stream) {
  const int st = check_quantize("fp8_quantize_ex", x, numel, in_type, fmt, ring, y_fp8, 0);
  if (st != FP8DS_OK || numel == 0) return st;
  return launch_quantize(x, numel, in_type, fmt, ring, y_fp8, 0, static_cast<hipStream_t>(stream));
}

int fp8_quantize_batch(const fp8_quantize_job* jobs, int njobs, int in_type, int fmt, void* stream) {
  const char* fn = "fp8_quantize_batch";
  if (!jobs) return set_error(FP8DS_EINVAL, "%s: jobs is NULL", fn);
  if (njobs < 1 || njobs > FP8DS_MAX_BATCH)
    return set_error(FP8DS_EINVAL, "%s: njobs %d outside [1, %d]", fn, njobs, FP8DS_MAX_BATCH);
  for (int i = 0; i < njobs; ++i) {
    const fp8_quantize_job& j = jobs[i];
    const int st = check_quantize(fn, j.x, j.numel, in_type, fmt, j.ring, j.y, 0);
    if (st != FP8DS_OK) return st;
    if ((reinterpret_cast<uintptr_t>(j.scale_inv_out) & 3u) != 0)
      return set_error(FP8DS_EALIGN, "%s: job %d scale_inv_out not 4-byte aligned", fn, i);
  }
  for (int i = 0; i < njobs; ++i) {
    for (int k = i + 1; k < njobs; ++k) {
      const fp8_quantize_job &a = jobs[i], &b = jobs[k];
      if (a.ring == b.ring) return set_error(FP8DS_EINVAL, "%s: jobs %d and %d share a ring", fn, i, k);
      if (a.numel == 0 || b.numel == 0) continue;
      if (overlaps(a.y, a.numel, b.y, b.numel) || overlaps(a.y, a.numel, b.x, b.numel * in_size(in_type)) ||
          overlaps(b.y, b.numel, a.x, a.numel * in_size(in_type)))
        return set_error(FP8DS_EINVAL, "%s: the output of job %d or %d overlaps the other job's input or output", fn,
                         i, k);
    }
  }
  return launch_quantize_batch(jobs, njobs, in_type, fmt, static_cast<hipStream_t>(stream));
}

int fp8_quantize_dynamic(const void* x, int64_t numel, int in_type, int fmt, void* ring, void* y_fp8, void* stream) {
  const int st = check_quantize("fp8_quantize_dynamic", x, numel, in_type, fmt, ring, y_fp8, 0);
  if (st != FP8DS_OK || numel == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int a = launch_amax(x, numel, in_type, fmt, ring, s);
  if (a != FP8DS_OK) return a;
  return launch_quantize(x, numel, in_type, fmt, ring, y_fp8, 0, s);
}

int fp8_quantize_2d(const void* x, int64_t rows, int64_t cols, int in_type, int fmt, int layout, void* ring, void* y,
                    void* y_t, void* stream) {
  const char* fn = "fp8_quantize_2d";
  if (layout < FP8DS_ROWWISE || layout > FP8DS_DUAL) return set_error(FP8DS_EINVAL, "%s: bad layout %d", fn, layout);
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim)
    return set_error(FP8DS_EINVAL, "%s: rows and cols must be in [0, 2^31)", fn);
  const int64_t numel = rows * cols;
  if (layout == FP8DS_ROWWISE) {
    const int st = check_quantize(fn, x, numel, in_type, fmt, ring, y, 0);
    if (st != FP8DS_OK || numel == 0) return st;
    return launch_quantize(x, numel, in_type, fmt, ring, y, 0, static_cast<hipStream_t>(stream));
  }
  const bool dual = layout == FP8DS_DUAL;
  const int st = check_quantize(fn, x, numel, in_type, fmt, ring, y_t, 0);
  if (st != FP8DS_OK || numel == 0) return st;
  if ((rows & 15) || (cols & 15))
    return set_error(FP8DS_EALIGN, "%s: transposed forms need rows and cols multiples of 16 (got %lld x %lld)", fn,
                     (long long)rows, (long long)cols);
  if (dual) {
    if (!y) return set_error(FP8DS_EINVAL, "%s: DUAL needs y", fn);
    if (!aligned16(y)) return set_error(FP8DS_EALIGN, "%s: y not 16-byte aligned", fn);
    if (overlaps(x, numel * in_size(in_type), y, numel) || overlaps(y, numel, y_t, numel))
      return set_error(FP8DS_EINVAL, "%s: y overlaps x or y_t", fn);
  }
  return launch_quantize_2d(x, (int)rows, (int)cols, in_type, fmt, dual, ring, y, y_t, 0,
                            static_cast<hipStream_t>(stream));
}

size_t fp8_bias_grad_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0 || rows > kMaxDim || cols > kMaxDim) return 0;
  return bias_grad_workspace(rows, cols);
}

int fp8_bias_grad(const void* g, int64_t rows, int64_t cols, int g_type, const float* g_scale_inv, int out_f32,
                  void* out, void* workspace, void* stream) {
  bool nothing = false;
  if (const int st = check_bias_grad("fp8_bias_grad", g, rows, cols, g_type, g_scale_inv, out, true, workspace,
                                     &nothing))
    return st;
  if (nothing) return FP8DS_OK;
  return launch_bias_grad(g, (int)rows, (int)cols, g_type, g_scale_inv, out_f32 != 0, out, workspace,
                          static_cast<hipStream_t>(stream));
}

int fp8_bias_grad_noalloc(const void* g, int64_t rows, int64_t cols, int g_type, const float* g_scale_inv,
                          int out_f32, void* out, void* stream) {
  bool nothing = false;
  if (const int st = check_bias_grad("fp8_bias_grad_noalloc", g, rows, cols, g_type, g_scale_inv, out, false,
                                     nullptr, &nothing))
    return st;
  if (nothing) return FP8DS_OK;
  return launch_bias_grad_noalloc(g, (int)rows, (int)cols, g_type, g_scale_inv, out_f32 != 0, out,
                                  static_cast<hipStream_t>(stream));
}

int fp8_mm(const fp8_mm_args* a, void* stream) { return fp8_mm_with_grid(a, -1, 0, stream); }

int fp8_mm_with_tile(const fp8_mm_args* a, int tile, void* stream) { return fp8_mm_with_grid(a, tile, 0, stream); }

int fp8_mm_with_grid(const fp8_mm_args* a, int tile, int max_workgroups, void* stream) {
  if (max_workgroups < 0) return set_error(FP8DS_EINVAL, "fp8_mm: max_workgroups %d < 0", max_workgroups);
  GemmProblem p{};
  bool empty = false;
  if (const int st = check_mm(a, &p, &empty)) return st;
  if (empty) return FP8DS_OK;
  return launch_gemm(p, tile, max_workgroups, static_cast<hipStream_t>(stream));
}

int fp8_mm_pair(const fp8_mm_args* first, const fp8_mm_args* second, void* stream) {
  GemmProblem p[2]{};
  bool empty[2] = {false, false};
  if (const int st = check_mm(first, &p[0], &empty[0])) return st;
  if (const int st = check_mm(second, &p[1], &empty[1])) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (empty[0] || empty[1]) {
    if (!empty[0]) return launch_gemm(p[0], -1, 0, s);
    if (!empty[1]) return launch_gemm(p[1], -1, 0, s);
    return FP8DS_OK;
  }
  // Each output may be written while the other problem reads its operands.
  for (int i = 0; i < 2; ++i) {
    const GemmProblem &w = p[i], &r = p[1 - i];
    const int64_t c_bytes = mm_c_bytes(w);
    if (overlaps(w.c, c_bytes, r.c, mm_c_bytes(r)) || overlaps(w.c, c_bytes, r.a, mm_operand_bytes(r.extent_a, r)) ||
        overlaps(w.c, c_bytes, r.b, mm_operand_bytes(r.extent_b, r, true)) ||
        (r.bias_kind != FP8DS_BIAS_NONE && overlaps(w.c, c_bytes, r.bias, mm_bias_bytes(r))))
      return set_error(FP8DS_EINVAL, "fp8_mm_pair: the output of one problem overlaps an input or the output of the other");
  }
  return launch_gemm_pair(p[0], p[1], s);
}

int fp8_mm_tile(const fp8_mm_args* a) {
  GemmProblem p{};
  bool empty = false;
  if (const int st = check_mm(a, &p, &empty)) return st;
  return empty ? FP8DS_TILE_NONE : gemm_tile(p);
}

int fp8_mm_pair_tile(const fp8_mm_args* first, const fp8_mm_args* second) {
  GemmProblem p[2]{};
  bool empty[2] = {false, false};
  if (const int st = check_mm(first, &p[0], &empty[0])) return st;
  if (const int st = check_mm(second, &p[1], &empty[1])) return st;
  if (empty[0] && empty[1]) return FP8DS_TILE_NONE;
  if (empty[0] || empty[1]) return FP8DS_TILE_SEPARATE;
  const int t = gemm_pair_tile(p[0], p[1]);
  return t < 0 ? FP8DS_TILE_SEPARATE : t;
}

}  // extern "C"
