/*
 * fp8ds: delayed-scaling FP8 quantize and scaled FP8 GEMM for AMD MI355X (gfx950).
 *
 * Plain C ABI: no C++ types, no exceptions, no allocation.  Every pointer
 * argument named "device" is device memory owned by the caller; the library
 * keeps no device state of its own.  All calls are asynchronous on the given
 * HIP stream (a hipStream_t passed as void*; NULL = the default stream) and
 * never synchronise with the host.  A call returns FP8DS_OK after launching,
 * or a negative status having launched nothing; fp8_last_error() then holds a
 * message for the calling thread.
 *
 * Page citations name the AstrAI commit-history page and the entry on it.
 */
#ifndef FP8DS_H
#define FP8DS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 8-bit formats: OCP E4M3FN (max 448, no infinities) for forward operands and
 * OCP E5M2 (max 57344) for gradients (fp8.py history @4dc5e923: the grad ring
 * is kept apart from x/w; the format enum is validated at the binding,
 * fp8.py history @f4c44ebf, quantize split entry). */
typedef enum { FP8DS_E4M3 = 0, FP8DS_E5M2 = 1 } fp8ds_fmt;

/* Operand storage of C[M,N] = A[M,K] * B[K,N], all row-major views:
 *   NT: A stored [M,K], B stored [N,K]  (both K-contiguous: linear forward)
 *   NN: A stored [M,K], B stored [K,N]  (B crosswise: dX = G * W)
 *   TN: A stored [K,M], B stored [K,N]  (A and B crosswise: dW = G^T * X)
 * (gemm.cuh history @5e76fbd1: RowMajor/ColMajor layout tags; crosswise-A
 * and crosswise-B entries.) */
typedef enum { FP8DS_NT = 0, FP8DS_NN = 1, FP8DS_TN = 2 } fp8ds_layout;

/* Bias storage (bias-fusion entry, fp8.py history @f4c44ebf): none, bf16[N]
 * or fp32[N], or 8-bit codes[N] dequantized as dec(code) * bias_scale_inv
 * (history of test_fp8_mma.py, bias_scale entry); the sum acc * alpha + bias
 * is formed in fp32 and rounded to bf16 once. */
typedef enum {
  FP8DS_BIAS_NONE = 0,
  FP8DS_BIAS_BF16 = 1,
  FP8DS_BIAS_F32 = 2,
  FP8DS_BIAS_E4M3 = 3,
  FP8DS_BIAS_E5M2 = 4
} fp8ds_bias_kind;

/* Element type a quantize reads (fp8.py history @f4c44ebf, entry templating
 * the quantize on its input type). */
typedef enum { FP8DS_IN_BF16 = 0, FP8DS_IN_F16 = 1, FP8DS_IN_F32 = 2 } fp8ds_in_type;

/* Orientation of a 2-D quantize (history of `tests`, entry splitting the
 * quantize into quantize / quantize_dual with a layout enum). */
typedef enum { FP8DS_ROWWISE = 0, FP8DS_TRANSPOSED = 1, FP8DS_DUAL = 2 } fp8ds_quant_layout;

/* Element type of a gradient summed by fp8_bias_grad: raw bf16 / fp16 / fp32,
 * or 8-bit codes dequantized with a scale (fp8.py history @f4c44ebf,
 * pre-quantized g entry). */
typedef enum {
  FP8DS_G_BF16 = 0,
  FP8DS_G_F16 = 1,
  FP8DS_G_F32 = 2,
  FP8DS_G_E4M3 = 3,
  FP8DS_G_E5M2 = 4
} fp8ds_grad_type;

enum {
  FP8DS_OK = 0,
  FP8DS_EINVAL = -1,      /* null pointer, bad enum, negative or oversized dimension  */
  FP8DS_EALIGN = -2,      /* base pointer or leading dimension not 16-byte aligned    */
  FP8DS_EUNSUPPORTED = -3,/* valid request the library does not implement             */
  FP8DS_ELAUNCH = -4      /* the HIP runtime rejected the kernel launch               */
};

/* ---------------------------------------------------------------------------
 * Scale ring: the per-operand delayed-scaling state (fp8.py history
 * @4dc5e923: one buffer packing the history, the scale and a counter; one
 * ring per operand x, w, g).  Caller-owned device memory of
 * fp8_scale_ring_bytes(hist_len) bytes, 16-byte aligned, laid out as:
 *
 *   offset  type     field
 *   0       float    scale           multiplier the next quantize applies
 *   4       float    scale_inv_used  1 / (scale the last quantize applied): the
 *                                    GEMM's dequantization multiplier (scale
 *                                    snapshot entry, fp8.py history @f4c44ebf)
 *   8       float    amax_last       amax of the last quantized tensor
 *   12      int32    idx             next history slot to write
 *   16      int32    hist_len        window length H, 1..1024
 *   20      int32    fmt             fp8ds_fmt the ring serves
 *   24      uint32   status          sticky device-side error bits (see below)
 *   28      uint32   (reserved, 0)
 *   32      uint32   amax_bits       scratch: running max of |x| bits, 0 between calls
 *   36      uint32   ticket          scratch: finished-group counter, 0 between calls
 *   40..63           (reserved, 0)
 *   64      32 x 64 B                scratch: per block-group {uint32 amax_bits,
 *                                    uint32 ticket, 56 B pad}, 0 between calls
 *   2112    float    hist[H]         amax history window
 *
 * The ring is the only state of the method: copying its bytes out and back
 * checkpoints and restores it.  Calls that use one ring must be ordered on
 * one stream; concurrent use of one ring is undefined.
 * status bits: 1 = fp8_quantize fmt differed from the ring's fmt,
 *              2 = ring header invalid (hist_len or idx out of range).
 * A call that sets a status bit leaves the ring's scale, history and index
 * unchanged; its output bytes are unspecified.
 * ------------------------------------------------------------------------- */
#define FP8DS_RING_HEADER_BYTES 64
#define FP8DS_RING_HIST_OFFSET 2112
#define FP8DS_RING_MAX_HIST 1024

/* Bytes of a ring with hist_len slots: 2112 + 4 * hist_len rounded up to 16;
 * 0 if hist_len is outside [1, 1024]. */
size_t fp8_scale_ring_bytes(int hist_len);

/* Device address of a ring's scale_inv_used field (ring + 4), for
 * fp8_mm_args.a_scale_inv / b_scale_inv. */
const float* fp8_ring_scale_inv(const void* ring);

/* Initialise a ring on `stream`: zero history, idx 0, scale = init_scale,
 * scale_inv_used = 1/init_scale (IEEE binary32), scratch and status zero.
 * ring: device, fp8_scale_ring_bytes(hist_len) bytes, 16-byte aligned.
 * init_scale must be finite and > 0 (the pages' "seed" of a ring, fp8.py
 * history @4dc5e923, FP8TensorMeta entry). */
int scale_ring_init(void* ring, int hist_len, int fmt, float init_scale, void* stream);

/* Delayed-scaling quantize (fp8.py history @4dc5e923, ring-finalize entry;
 * @f4c44ebf, quantize split and amax entries):
 *   y[i] = saturate_round_nearest_even_fmt(fl32(x[i]) * scale)   for i < numel
 * with scale = ring->scale read at launch, NaN -> 0x7F | sign.  In the same
 * launch (last-block epilogue, no extra kernel) the ring is advanced:
 *   a = max_i |x[i]| (fp32, before the cast); hist[idx] = a; idx = (idx+1) % H;
 *   w = max(hist); if w finite and > 0 and FMAX/w finite: scale = FMAX/w;
 *   scale_inv_used = 1/scale_used; amax_last = a.
 * x: device bf16[numel], 16-byte aligned.  y: device uint8[numel] (fp8
 * codes), 16-byte aligned, must not overlap x.  ring: an initialised ring of
 * format fmt.  numel == 0 launches nothing and leaves the ring unchanged.
 * ring == NULL (dynamic scaling) returns FP8DS_EUNSUPPORTED. */
int fp8_quantize(const void* x_bf16, int64_t numel, int fmt, void* ring, void* y_fp8, void* stream);

/* fp8_quantize with the grid capped at max_blocks workgroups of 256 threads
 * (0 = the default cap); same results bit for bit, for tuning sweeps. */
int fp8_quantize_with_grid(const void* x_bf16, int64_t numel, int fmt, void* ring, void* y_fp8, int max_blocks,
                           void* stream);

/* fp8_quantize of an input of any fp8ds_in_type (fp8.py history @f4c44ebf,
 * input-type entry): the element is widened to fp32 exactly, then as above;
 * amax is max |fl32(x)|.  x: device, numel elements of in_type, 16-byte
 * aligned.  Same errors as fp8_quantize; in_type outside the enum is
 * FP8DS_EINVAL. */
int fp8_quantize_ex(const void* x, int64_t numel, int in_type, int fmt, void* ring, void* y_fp8, void* stream);

/* Up to FP8DS_MAX_BATCH independent fp8_quantize_ex calls in one launch:
 * each job is exactly fp8_quantize_ex on its own tensor and ring (fp8.py
 * history @4dc5e923, ring-finalize entry, applied per job: each job's blocks
 * elect their own last block).  Meant for the small tensors of one layer
 * (X and W of a linear), where a launch is mostly fixed latency.
 * All jobs share in_type and fmt.  Per job: x, numel, ring and y as in
 * fp8_quantize_ex; scale_inv_out, if not NULL, a 4-byte aligned device fp32
 * that receives fl32(1 / scale applied), the value the job's ring holds in
 * scale_inv_used after the call, so the caller keeps the forward's
 * dequantization scale without a copy.  Jobs with numel == 0 are skipped.
 * jobs: host array of njobs entries (1 <= njobs <= FP8DS_MAX_BATCH), read
 * before the call returns.  The rings must be distinct, and no job's y may
 * overlap another job's x or y (FP8DS_EINVAL); per-job errors as
 * fp8_quantize_ex, reported before anything is launched. */
#define FP8DS_MAX_BATCH 8
typedef struct fp8_quantize_job {
  const void* x;
  int64_t numel;
  void* ring;
  void* y;
  float* scale_inv_out;
} fp8_quantize_job;
int fp8_quantize_batch(const fp8_quantize_job* jobs, int njobs, int in_type, int fmt, void* stream);

/* Quantize of a rows x cols row-major tensor in one or two orientations
 * (history of `tests`: quantize / quantize_dual, orientations byte-equal to
 * the plain quantize):
 *   ROWWISE:    y[r][c]   = code of x[r][c]          (y: rows x cols)
 *   TRANSPOSED: y_t[c][r] = code of x[r][c]          (y_t: cols x rows)
 *   DUAL:       both, from one read of x.
 * The codes and the ring update are exactly those of fp8_quantize_ex on the
 * same elements (one amax fold per call).  x: device, 16-byte aligned; y and
 * y_t: device, 16-byte aligned, unused ones may be NULL; neither may overlap
 * x.  TRANSPOSED and DUAL need rows and cols to be multiples of 16
 * (FP8DS_EALIGN otherwise) and rows, cols < 2^31.  rows == 0 or cols == 0
 * launches nothing. */
int fp8_quantize_2d(const void* x, int64_t rows, int64_t cols, int in_type, int fmt, int layout, void* ring, void* y,
                    void* y_t, void* stream);

/* Dynamic-scaling quantize: the tensor's own amax sets its scale
 * (fp8.py history @4dc5e923, dynamic-path entry; history of `tests`, recipe
 * with a dynamic flag).  Two launches on `stream`: a read of x that leaves in
 * ring hist[0] = a = max |fl32(x)| and scale = FMAX / a (1 if a is zero,
 * infinite or NaN or the quotient overflows), then fp8_quantize_ex with that
 * scale, after which scale_inv_used = 1 / scale and amax_last = a.
 * ring: an initialised ring with hist_len 1 and format fmt (status bit 2 is
 * set otherwise, and the ring and y are then unspecified).  Other arguments
 * and errors as fp8_quantize_ex. */
int fp8_quantize_dynamic(const void* x, int64_t numel, int in_type, int fmt, void* ring, void* y_fp8, void* stream);

/* Bias gradient (fp8.py history @f4c44ebf: the column sum of the output
 * gradient, run only when the bias needs a gradient; a pre-quantized g is
 * dequantized before the sum; gradients are bf16):
 *   out[c] = sum_r g[r][c]   accumulated in fp32, rounded once to bf16
 *                            (out_f32 == 0) or stored as fp32 (out_f32 != 0)
 * g: device, rows x cols row-major of g_type; 8-bit codes are dequantized as
 * fl32(dec(code) * g_scale_inv[0]) (g_scale_inv: device fp32, unused for the
 * other types).  cols must be a multiple of 8 and g 16-byte aligned.
 * The summation order depends only on (rows, cols): results are the same
 * bits run to run.  workspace: device, at least
 * fp8_bias_grad_workspace_bytes(rows, cols) bytes, 16-byte aligned,
 * zero-filled before its first use; every call leaves it all zero again, so
 * one workspace serves calls of any shape whose size it covers (calls sharing
 * a workspace must be ordered on one stream).  cols == 0 launches nothing;
 * rows == 0 writes zeros. */
size_t fp8_bias_grad_workspace_bytes(int64_t rows, int64_t cols);
int fp8_bias_grad(const void* g, int64_t rows, int64_t cols, int g_type, const float* g_scale_inv, int out_f32,
                  void* out, void* workspace, void* stream);

/* fp8_bias_grad for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results (bit for bit) and errors
 * as fp8_bias_grad, without `workspace`: the tickets and partial sums live in
 * a device array of the library, FP8DS_BIAS_GRAD_NOALLOC_MAX_BYTES bytes per
 * GPU, held from the first call on that GPU until the process ends.  A shape
 * whose fp8_bias_grad_workspace_bytes exceeds that size is
 * FP8DS_EUNSUPPORTED (with 1 MiB: any rows with cols up to 2^17, or cols up
 * to about 2.6e5 with few rows).  Nothing is allocated and nothing
 * synchronizes.  All calls on one GPU share the array: calls that may overlap
 * on one GPU (other streams, other threads) race and give undefined results;
 * order them on one stream.  The first call on a GPU also clears the array's
 * ticket words (one small kernel on `stream`; repeated while the stream is
 * capturing, so a captured graph clears them too); every call leaves the
 * array zero again. */
#define FP8DS_BIAS_GRAD_NOALLOC_MAX_BYTES (1 << 20)
int fp8_bias_grad_noalloc(const void* g, int64_t rows, int64_t cols, int g_type, const float* g_scale_inv,
                          int out_f32, void* out, void* stream);

/* Scaled FP8 GEMM arguments.  Zero-initialise and set what you use: a
 * zeroed field means "absent" (gemm.cuh history @5e76fbd1, null-default
 * params entry). */
typedef struct fp8_mm_args {
  const void* a;            /* device fp8 codes, layout per `layout`                 */
  const void* b;            /* device fp8 codes                                      */
  void* c;                  /* device bf16 [batch][M][ldc] output                    */
  int fmt_a, fmt_b;         /* fp8ds_fmt of each operand                             */
  int layout;               /* fp8ds_layout                                          */
  int bias_kind;            /* fp8ds_bias_kind                                       */
  int64_t m, n, k;          /* problem size; each 0 .. 2^31-1                        */
  int64_t batch;            /* number of products; 0 is treated as 1                 */
  int64_t lda, ldb, ldc;    /* leading dimension of each stored view, in elements    */
  int64_t stride_a, stride_b, stride_c; /* batch strides in elements; 0 broadcasts a/b */
  const float* a_scale_inv; /* device fp32 scalar, e.g. fp8_ring_scale_inv(ring_a)   */
  const float* b_scale_inv; /* device fp32 scalar                                    */
  const void* bias;         /* device bf16[N], fp32[N] or codes[N], broadcast over rows, batch */
  const float* bias_scale_inv; /* device fp32 scalar for an 8-bit bias, else unused  */
} fp8_mm_args;

/* Scaled FP8 GEMM (gemm.cuh history @5e76fbd1; fp8.py history @f4c44ebf,
 * bias-fusion and 3-D operand entries):
 *   C[b][m][n] = bf16_rne( sum_k A_b[m,k] * B_b[k,n]  (fp32 accumulate)
 *                          * (a_scale_inv * b_scale_inv) + fl32(bias[n]) )
 * Alignment: a, b, c, bias 16-byte aligned; lda, ldb multiples of 16 and
 * ldc a multiple of 8; batch strides multiples of 16 (a, b) and 8 (c).
 * Each stored operand of one batch entry must span < 2^31 bytes.
 * lda >= K (NT/NN) or >= M (TN); ldb >= K (NT) or >= N (NN/TN); ldc >= N.
 * m == 0 or n == 0 launches nothing; k == 0 writes bf16(bias) (or 0).
 * c must not overlap a, b or bias (checked over the bytes each spans;
 * FP8DS_EINVAL). */
int fp8_mm(const fp8_mm_args* args, void* stream);

/* fp8_mm with the workgroup tile forced: tile = index into the tile family
 * (M x N: 0: 256x256, 1: 128x128, 2: 64x64, 3: 256x128, 4: 128x256, 5 and 6:
 * 256x256 with eight waves, 7 and 8: 128x128 and 64x64 on 128-byte K units),
 * -1 or any index outside 0..8 = the automatic choice.  Every tile accumulates each output over K in the same order, so
 * all tiles give the same bits; for tests and tuning sweeps. */
int fp8_mm_with_tile(const fp8_mm_args* args, int tile, void* stream);

/* fp8_mm_with_tile with the grid bounded: at most max_workgroups workgroups,
 * each running every G-th output tile in turn (G = the grid size); 0 = as
 * many as the device holds at once (what fp8_mm uses).  Results are the
 * same bits as fp8_mm_with_tile with the same tile; for tests that need one
 * workgroup to run several tiles on small problems, and for tuning.
 * max_workgroups < 0 or > 2^31-1 is FP8DS_EINVAL. */
int fp8_mm_with_grid(const fp8_mm_args* args, int tile, int max_workgroups, void* stream);

/* Two independent fp8_mm calls, each exactly as fp8_mm on its own arguments
 * (its output bits included), issued together: a layer's dX = G.W (NN) and
 * dW = G^T.X (TN) on the forward's codes (fp8.py history @f4c44ebf,
 * forward-carries-scale entry: the backward's two GEMMs).  When `first` is
 * NN and `second` is TN with the same fmt_a and fmt_b, both run in one launch
 * whose workgroups are split between them, so small GEMMs that each leave
 * most of the chip idle share it, unless one of them is big enough for the
 * four-wave 256x256 tile on its own; any other pair runs as two launches in
 * order.  Each argument set is validated as fp8_mm validates it, and neither
 * output may overlap the other problem's operands, bias or output
 * (FP8DS_EINVAL); nothing is launched on an error.  An empty problem (m or n
 * zero) is skipped. */
int fp8_mm_pair(const fp8_mm_args* first, const fp8_mm_args* second, void* stream);

/* The tile fp8_mm would run these arguments on (an index of the tile family,
 * as fp8_mm_with_tile takes it), FP8DS_TILE_NONE when it would launch nothing
 * (m or n is 0), or the negative status fp8_mm would return for them.  Host
 * arithmetic only: no device is needed and nothing is launched; the pointers
 * are checked as fp8_mm checks them but never read.  For tests of the
 * automatic tile choice and for tuning (not a step of the method). */
#define FP8DS_TILE_NONE 64
#define FP8DS_TILE_SEPARATE 65
int fp8_mm_tile(const fp8_mm_args* args);

/* The same for fp8_mm_pair: the tile of the one launch that runs both
 * problems, FP8DS_TILE_SEPARATE when they go out as separate fp8_mm launches
 * (each on the tile fp8_mm_tile reports for it; also when exactly one is
 * empty), FP8DS_TILE_NONE when both are empty, or the negative status of the
 * first invalid argument set (the pair's overlap checks are not made). */
int fp8_mm_pair_tile(const fp8_mm_args* first, const fp8_mm_args* second);

/* The library's own error report (not a step of the method): a message
 * describing the last non-zero status returned on the calling thread, kept in
 * thread-local storage until that thread's next failing call.  The pointer is
 * owned by the library; never NULL (an empty string before any failure). */
const char* fp8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8DS_H */
