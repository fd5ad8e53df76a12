// Scaled FP8 x FP8 GEMM, host side: the tile family, the choice of tile and
// grid, and the launches of the kernels in gemm_kernel.h (instantiated by the
// gemm_*.hip picker files).
//
// Pages: AstrAI commit history of csrc/kernels/fp8/gemm.cuh (@5e76fbd1) and
// of astrai/extension/fp8.py (@f4c44ebf): a small-tile family for small
// problems, dispatch thresholds by problem size, grouped rasterization.
#include <atomic>

#include "gemm_kernel.h"
#include "launch.h"

namespace fp8ds {

namespace {

// ---------------------------------------------------------------------------
// Host side: tile family and dispatch.

struct TileCfg {
  int bm, bn, waves;
};
// Tile family (index = the tile argument of fp8_mm_with_tile).  256x256 with
// four waves runs one workgroup per CU (4 LDS stages, 128 KiB), each wave a
// 128x128 block: the large-problem tile, as it reads the fewest LDS bytes per
// MFMA; the eight-wave 256x256 tiles give every SIMD two waves of a 128x64 /
// 64x128 block (the large tile of a GEMM with a bias); 256x128 / 128x256 run two
// workgroups per CU (3 stages, 72 KiB each);
// 128x128 and 64x64 serve problems too small to fill the chip; the 128x128
// and 64x64 tiles on 128-byte K units (five 16 / 8 KiB slots, two / four
// workgroups per CU) are the ones the automatic choice takes, the general
// kernel's stay for tests.
constexpr TileCfg kTiles[] = {{256, 256, 4}, {128, 128, 4}, {64, 64, 4}, {256, 128, 4},
                              {128, 256, 4}, {256, 256, 8}, {256, 256, 8}, {128, 128, 4}, {64, 64, 4}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// The kernel of one tile, layout and format pair, from its picker file.
GemmFn kernel_for(int tile, int layout, int fa, int fb) {
  const bool large = tile == 0 || tile == 5 || tile == 6;
  if (layout == 0) return large ? gemm_fn_nt_large(tile, fa, fb) : gemm_fn_nt_small(tile, fa, fb);
  if (layout == 1) return large ? gemm_fn_nn_large(tile, fa, fb) : gemm_fn_nn_small(tile, fa, fb);
  return large ? gemm_fn_tn_large(tile, fa, fb) : gemm_fn_tn_small(tile, fa, fb);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile choice by grid size, from per-shape timings on 256 CUs:
//  * a 256x256 tile when its grid fills at least three quarters of the CUs,
//    except when K <= 1024 and its last round of tiles is partial: there
//    the 128x128 tile on 128-byte K units, two workgroups per CU, ends
//    sooner (4096x3072x1024, 192 tiles: 15.2 against 17.8 us;
//    8192x3072x1024, 384 tiles: 25.5 against 30.9 us; with a bias 16.7 and
//    28.9 against 20.6 and 34.9 us), while on whole rounds the two are level
//    and with K = 4096 the 256x256 tile is clearly faster (4096^3: 50 against
//    62 us); with K <= 512 the 128x128 unit tile wins on whole rounds too
//    (64 x 512^3 batched: 12.6 against 14.3 us);
//  * else the 128x128 tile on 128-byte units when its grid fills the CUs, or
//    half-fills them with K >= 2048 (a half-empty chip of 128x128 tiles
//    beats a full one of 64x64 tiles once the K loop is long enough to
//    amortize their higher per-tile rate); the unit tile ran 0-25 % faster
//    than the general kernel's 128x128 tile on every layer shape measured
//    (8192x1024x4096 NT: 29.4 against 39.0 us), with the same bits;
//  * else 64x64 on 128-byte units, the most tiles (against the general
//    kernel's 64x64 tile, same bits: 1024x1024x4096 NT 12.9 -> 10.8 us,
//    1024x1536x2048 NN 10.3 -> 9.0 us, TN level).
int64_t tile_count(const GemmProblem& p, int t) {
  return cdiv(p.m, kTiles[t].bm) * cdiv(p.n, kTiles[t].bn) * p.batch;
}

// The rule over a launch's total tile count and (shortest) K.
int tile_for(int64_t (*count)(const GemmProblem*, int), const GemmProblem* ps, int64_t k, int big) {
  constexpr int64_t kCUs = 256;
  const int64_t tb = count(ps, big);
  if (4 * tb >= 3 * kCUs && !(k <= 512 || (k <= 1024 && tb % kCUs != 0))) return big;
  const int64_t t1 = count(ps, 7);
  if (t1 >= kCUs || (2 * t1 >= kCUs && k >= 2048)) return 7;
  return 8;
}

// Large launches take the four-wave 256x256 tile without a bias and the
// eight-wave one, which stages its bias epilogue through LDS, with one.
int choose_tile(const GemmProblem& p) {
  return tile_for([](const GemmProblem* q, int t) { return tile_count(*q, t); }, &p, p.k, p.bias_kind == 0 ? 0 : 6);
}

// For a fused pair: the same rule over both problems' tiles and the shorter K
// (its 256x256 answer, the eight-wave tile, sends the two out as separate
// launches: gemm_pair_tile below).  The partial-round
// exception holds for pairs too: the 12-layer step at 2048 tokens (whose MLP
// down-projection pair has 192 tiles of 256x256 and K = 1024) went from
// 2.58-2.59 to 2.50-2.52 ms, at 4096 tokens (that pair, 320 tiles, then runs
// as one launch instead of two) from 3.53-3.59 to 3.50-3.52 ms.
int choose_pair_tile(const GemmProblem (&pp)[2]) {
  return tile_for([](const GemmProblem* q, int t) { return tile_count(q[0], t) + tile_count(q[1], t); }, pp,
                  pp[0].k < pp[1].k ? pp[0].k : pp[1].k, 6);
}

// Workgroups of one kernel that fit on the device at once (CUs x occupancy),
// cached per device and kernel.
int resident_workgroups(const void* fn, int slot, int threads) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][kNumTiles * 16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int hit = cache[dev][slot].load(std::memory_order_relaxed);
  if (hit > 0) return hit;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) !=
          hipSuccess)
    return 0;
  const int r = cus * per_cu;
  if (r > 0) cache[dev][slot].store(r, std::memory_order_relaxed);
  return r;
}

}  // namespace

namespace {

GemmKArgs make_kargs(const GemmProblem& p, int t) {
  GemmKArgs k{};
  k.a = p.a;
  k.b = p.b;
  k.c = p.c;
  k.m = p.m;
  k.n = p.n;
  k.k = p.k;
  k.tiles_m = (int)cdiv(p.m, kTiles[t].bm);
  k.tiles_n = (int)cdiv(p.n, kTiles[t].bn);
  k.batch = p.batch;
  k.group_m = 4;
  k.lda = (uint32_t)p.lda;
  k.ldb = (uint32_t)p.ldb;
  k.ldc = p.ldc;
  k.stride_a = p.stride_a;
  k.stride_b = p.stride_b;
  k.stride_c = p.stride_c;
  k.extent_a = p.extent_a;
  k.extent_b = p.extent_b;
  k.a_scale_inv = p.a_scale_inv;
  k.b_scale_inv = p.b_scale_inv;
  k.bias = p.bias;
  k.bias_scale_inv = p.bias_scale_inv;
  k.bias_kind = p.bias_kind;
  k.ldc_small = p.ldc * 256 < 0x80000000LL;
  return k;
}

// Workgroups for `total` tiles given `g` resident slots: one per slot, each
// running every G-th tile; G a multiple of 8 keeps tile v on XCD v mod 8.
int64_t grid_for(int64_t total, int64_t g) {
  if (g <= 0) g = total;
  if (g < total && g >= 8) g &= ~int64_t(7);
  return g > total ? total : g;
}

int check_counts(int64_t total, int64_t g, int k) {
  if (total > 0x7FFFFFFF) return set_error(-3, "fp8_mm: %lld tiles exceed the grid limit", (long long)total);
  if (cdiv(total, g) * cdiv(k, 64) > 0x7FFFFFFF)
    return set_error(-3, "fp8_mm: %lld K stages per workgroup exceed the kernel's counter",
                     (long long)(cdiv(total, g) * cdiv(k, 64)));
  return 0;
}

}  // namespace

int launch_gemm(const GemmProblem& p, int tile_override, int max_workgroups, hipStream_t stream) {
  const int t = (tile_override >= 0 && tile_override < kNumTiles) ? tile_override : choose_tile(p);
  const GemmKArgs k = make_kargs(p, t);
  const int64_t total = (int64_t)k.tiles_m * k.tiles_n * k.batch;
  if (total > 0x7FFFFFFF) return set_error(-3, "fp8_mm: %lld tiles exceed the grid limit", (long long)total);
  GemmFn fn = kernel_for(t, p.layout, p.fmt_a, p.fmt_b);
  const int threads = 64 * kTiles[t].waves;
  const int64_t g = grid_for(total, max_workgroups > 0
                                        ? max_workgroups
                                        : resident_workgroups(reinterpret_cast<const void*>(fn),
                                                              t * 16 + p.layout * 4 + p.fmt_a * 2 + p.fmt_b, threads));
  if (const int st = check_counts(total, g, p.k)) return st;
  hipLaunchKernelGGL(fn, dim3((unsigned)g), dim3(threads), 0, stream, k);
  return check_launch("gemm_kernel");
}

int gemm_tile(const GemmProblem& p) { return choose_tile(p); }

int gemm_pair_tile(const GemmProblem& p0, const GemmProblem& p1) {
  if (!(p0.layout == 1 && p1.layout == 2 && p0.fmt_a == p1.fmt_a && p0.fmt_b == p1.fmt_b)) return -1;
  const GemmProblem pp[2] = {p0, p1};
  const int t = choose_pair_tile(pp);
  // A pair big enough for the eight-wave 256x256 tile runs faster as two
  // launches, each on its own tile (graph-replayed, one box: dX 8192x1024x4096
  // + dW 4096x1024x8192 69-76 us as two, 78-88 us as one; at 11264 tokens
  // 97-99 against 109-112 us), so only the unit tiles run pairs.  Every tile
  // gives the same bits, so the outputs do not depend on the choice.
  if (t == 6) return -1;
  return t;
}

int launch_gemm_pair(const GemmProblem& p0, const GemmProblem& p1, hipStream_t stream) {
  const int t = gemm_pair_tile(p0, p1);
  if (t < 0) {
    const int st = launch_gemm(p0, -1, 0, stream);
    return st ? st : launch_gemm(p1, -1, 0, stream);
  }
  const GemmKArgs k0 = make_kargs(p0, t), k1 = make_kargs(p1, t);
  const int64_t n0 = (int64_t)k0.tiles_m * k0.tiles_n * k0.batch, n1 = (int64_t)k1.tiles_m * k1.tiles_n * k1.batch;
  if (n0 > 0x7FFFFFFF || n1 > 0x7FFFFFFF) return set_error(-3, "fp8_mm_pair: tiles exceed the grid limit");
  GemmPairFn fn = gemm_pair_fn(t, p0.fmt_a, p0.fmt_b);
  const int threads = 64 * kTiles[t].waves;
  const int64_t res = resident_workgroups(reinterpret_cast<const void*>(fn), t * 16 + 12 + p0.fmt_a * 2 + p0.fmt_b,
                                          threads);
  // Both problems' tiles at once when the device holds them all; otherwise the
  // resident slots split in proportion to each problem's MFMA work.
  int64_t g0 = n0, g1 = n1;
  if (res > 0 && n0 + n1 > res) {
    const double w0 = (double)n0 * (p0.k > 0 ? p0.k : 1), w1 = (double)n1 * (p1.k > 0 ? p1.k : 1);
    int64_t s0 = (int64_t)((double)res * w0 / (w0 + w1) + 0.5);
    if (s0 < 1) s0 = 1;
    if (s0 > res - 1) s0 = res - 1;
    g0 = grid_for(n0, s0);
    g1 = grid_for(n1, res - g0);
  }
  if (const int st = check_counts(n0, g0, p0.k)) return st;
  if (const int st = check_counts(n1, g1, p1.k)) return st;
  hipLaunchKernelGGL(fn, dim3((unsigned)(g0 + g1)), dim3(threads), 0, stream, k0, k1, (int)g0);
  return check_launch("gemm_pair_kernel");
}

}  // namespace fp8ds
