// Scaled FP8 x FP8 GEMM with fp32 accumulation, per-operand dequantization,
// fused fp32 bias and one bf16 rounding, on gfx950 FP8 MFMA.
//
// Pages: AstrAI commit history of csrc/kernels/fp8/gemm.cuh (@5e76fbd1) and
// of astrai/extension/fp8.py (@f4c44ebf): bf16-only output, bias added in
// fp32 before the single rounding with exact N tails, batched operands with
// stride-0 broadcast, congruous (NT) forward and crosswise dX / dW operands,
// grouped rasterization, a small-tile family for small problems.  Their CUDA
// tiling (cp.async staging, ldmatrix, PRMT transposes) is prior art only.
//
// gfx950 design:
//  * 4 waves per workgroup in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2)
//    block of C made of 32 x 32 tiles of v_mfma_f32_32x32x64_f8f6f4.  The
//    instruction's first source is the B fragment and its second the A
//    fragment, so each lane ends up holding four consecutive n of one row m:
//    8-byte bf16 stores and 4-wide bias loads in the epilogue.  The per-operand
//    format selectors of the instruction take E4M3 x E4M3 and E5M2 x E4M3
//    (dX, dW) alike.
//  * Operand tiles go global -> LDS with buffer_load ... lds (no VGPR round
//    trip), 128 K-bytes per stage, two stages.  Loads outside the operand or
//    past K are given an offset beyond the buffer's size and land as zeros.
//  * K-contiguous tiles are [rows][128 B] and are read with ds_read_b128;
//    MN-contiguous (crosswise) tiles are [128 k][BM or BN bytes] and are read
//    with ds_read_b64_tr_b8, which transposes 8 x 8-byte blocks across 16
//    lanes, so crosswise operands need no transpose pass.  16-byte chunks are
//    XOR-swizzled per row so both read kinds are free of bank conflicts.
//  * The workgroup -> tile map gives each of the 8 XCDs (workgroups are dealt
//    to XCDs round-robin) a contiguous run of tiles in grouped order, so the
//    tiles sharing A rows and B columns meet in one XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace fp8ds {

namespace {

constexpr int kBK = 64;           // K bytes (= elements) per pipeline stage
constexpr uint32_t kOOB = 0x80000000u;  // offset past every buffer: loads give zero

struct GemmKArgs {
  const uint8_t* a;
  const uint8_t* b;
  uint16_t* c;
  int m, n, k;
  int tiles_m, tiles_n, batch, group_m;
  uint32_t lda, ldb;
  int64_t ldc;
  int64_t stride_a, stride_b, stride_c;
  uint32_t extent_a, extent_b;
  const float* a_scale_inv;
  const float* b_scale_inv;
  const void* bias;
  int bias_kind;
};

// K-contiguous tile [rows][64 B]: 16-byte chunk c of row r sits at chunk
// c ^ swz_k(r).  A fragment read (32 consecutive rows, lanes l and l+32
// taking adjacent chunk pairs of one row) is then free of LDS bank conflicts;
// the choice was measured on gfx950 (SQ_LDS_BANK_CONFLICT = 0), where the
// xor of (r >> 1) ^ (r >> 3) still left 4 conflict cycles per ds_read_b128.
__device__ __forceinline__ int swz_k(int r) { return (r >> 2) & 3; }

// MN-contiguous tile [64 k][R chunks]: chunk c of row k sits at c ^ swz_mn(k).
// A transpose read touches 8 consecutive rows x 2 adjacent chunks; the
// swizzle spreads them over distinct bank groups.
template <int R>
__device__ __forceinline__ int swz_mn(int k) {
  if constexpr (R == 16) return ((k & 7) << 1) | ((k >> 2) & 1);
  else if constexpr (R == 8) return k & 7;
  else return ((k >> 2) & 1) << 1;
}

// Workgroup -> (batch, tile row, tile column).
__device__ __forceinline__ void map_tile(const GemmKArgs& p, int& bt, int& tm, int& tn) {
  const int total = p.tiles_m * p.tiles_n * p.batch;
  const int w = blockIdx.x;
  const int q = total >> 3, r = total & 7;
  const int xcd = w & 7, j = w >> 3;
  const int t = xcd < r ? xcd * (q + 1) + j : r * (q + 1) + (xcd - r) * q + j;
  const int per_batch = p.tiles_m * p.tiles_n;
  bt = t / per_batch;
  const int u = t - bt * per_batch;
  const int in_group = p.group_m * p.tiles_n;
  const int g = u / in_group;
  const int first_m = g * p.group_m;
  const int gsize = min(p.tiles_m - first_m, p.group_m);
  const int v = u - g * in_group;
  tm = first_m + v % gsize;
  tn = v / gsize;
}

// 32 rows x 64 k of a K-contiguous tile: lane l gets row base + l%32,
// k = 32*(l/32) + [0, 32).
__device__ __forceinline__ v8i frag_k(const lds_char_t* tile, int base, int lane) {
  const int row = base + (lane & 31);
  const int c0 = 2 * (lane >> 5);
  const int sw = swz_k(row);
  const v4i lo = *(const lds_v4i_t*)(tile + row * kBK + ((c0 ^ sw) << 4));
  const v4i hi = *(const lds_v4i_t*)(tile + row * kBK + (((c0 + 1) ^ sw) << 4));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The same fragment from an MN-contiguous tile [64 k][R*16 B] through four
// transpose reads: read t hands lane l the bytes k = 32*(l/32) + 8*t + [0, 8)
// of column base + l%32.  Within each 16-lane group, the even lanes address
// rows k..k+7 at the group's first 8 columns and the odd lanes the next 8.
template <int R>
__device__ __forceinline__ v8i frag_mn(const lds_char_t* tile, int base, int lane) {
  const int q = lane & 15;
  const int cl = (base >> 4) + ((lane >> 4) & 1);
  v2i part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kr = 32 * (lane >> 5) + 8 * t + (q >> 1);
    const int addr = kr * (R * 16) + ((cl ^ swz_mn<R>(kr)) << 4) + 8 * (q & 1);
    part[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(tile + addr));
  }
  return v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
}

template <bool KC, int ROWS>
__device__ __forceinline__ v8i load_frag(const lds_char_t* tile, int base, int lane) {
  if constexpr (KC) return frag_k(tile, base, lane);
  else return frag_mn<ROWS / 16>(tile, base, lane);
}

// Per-lane byte offset of load slot `slot` of an operand tile, for k0 = 0;
// kOOB for rows / columns outside the operand.  kpos receives the slot's K
// position inside the stage (checked against K only in the last stage).
template <bool KC, int ROWS>
__device__ __forceinline__ uint32_t slot_offset(int slot, int mn0, int mn_lim, uint32_t ld, int& kpos) {
  if constexpr (KC) {
    const int row = slot >> 2, pch = slot & 3, lch = pch ^ swz_k(row);
    kpos = lch << 4;
    return mn0 + row < mn_lim ? (uint32_t)row * ld + (uint32_t)(lch << 4) : kOOB;
  } else {
    constexpr int R = ROWS / 16;
    const int kr = slot / R, pch = slot % R, lch = pch ^ swz_mn<R>(kr);
    kpos = kr;
    return mn0 + (lch << 4) < mn_lim ? (uint32_t)kr * ld + (uint32_t)(lch << 4) : kOOB;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most `stages` stages of LPS loads each are still in flight.
template <int LPS, int STAGES>
__device__ __forceinline__ void wait_stages(int stages) {
  static_assert(LPS * (STAGES - 1) <= 63, "vmcnt holds at most 63");
  if (stages >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * LPS));
  else if (stages == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS));
  else if (stages == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Workgroup barrier ordering LDS only: outstanding global->LDS prefetches of
// later stages stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int BM, int BN, int WGM, int WGN, int kStages, bool A_KC, bool B_KC, int FA, int FB, int OCC>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void gemm_kernel(GemmKArgs p) {
  constexpr int NW = WGM * WGN, kThreads = 64 * NW;   // waves in a WGM x WGN grid
  constexpr int WM = BM / WGM, WN = BN / WGN;          // C block of one wave
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * kBK, B_BYTES = BN * kBK, STAGE = A_BYTES + B_BYTES;
  constexpr int A_LOADS = A_BYTES / 1024 / NW, B_LOADS = B_BYTES / 1024 / NW;
  constexpr int LPS = A_LOADS + B_LOADS;
  static_assert(TM >= 1 && TN >= 1 && A_LOADS >= 1 && B_LOADS >= 1, "tile too small");
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStages * STAGE];
  lds_char_t* smem = (lds_char_t*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  int bt, tmi, tni;
  map_tile(p, bt, tmi, tni);
  const int m0 = tmi * BM, n0 = tni * BN;

  const uint32_t a_tile_off = A_KC ? (uint32_t)m0 * p.lda : (uint32_t)m0;
  const uint32_t b_tile_off = B_KC ? (uint32_t)n0 * p.ldb : (uint32_t)n0;
  const uint8_t* a_tile = p.a + bt * p.stride_a + a_tile_off;
  const uint8_t* b_tile = p.b + bt * p.stride_b + b_tile_off;
  const uint32_t a_rem = p.extent_a - a_tile_off;
  const uint32_t b_rem = p.extent_b - b_tile_off;

  uint32_t a_voff[A_LOADS], b_voff[B_LOADS];
  int a_kpos[A_LOADS], b_kpos[B_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j)
    a_voff[j] = slot_offset<A_KC, BM>((j * NW + wave) * 64 + lane, m0, p.m, p.lda, a_kpos[j]);
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j)
    b_voff[j] = slot_offset<B_KC, BN>((j * NW + wave) * 64 + lane, n0, p.n, p.ldb, b_kpos[j]);

  // Global -> LDS loads of K stage kt into LDS buffer kt % kStages: the
  // scalar part (descriptors, LDS bases) once per stage, then one
  // buffer_load ... lds per call of issue_one.
  struct LoadCtx {
    v4i ra, rb;
    uint32_t la, lb;
    int klim;
    bool tail;
  };
  auto load_ctx = [&](int kt, bool tail) __attribute__((always_inline)) {
    const int k0 = kt * kBK;
    const uint32_t a_adv = A_KC ? (uint32_t)k0 : (uint32_t)k0 * p.lda;
    const uint32_t b_adv = B_KC ? (uint32_t)k0 : (uint32_t)k0 * p.ldb;
    LoadCtx c;
    c.ra = rsrc_words(a_tile + a_adv, a_rem > a_adv ? a_rem - a_adv : 0u);
    c.rb = rsrc_words(b_tile + b_adv, b_rem > b_adv ? b_rem - b_adv : 0u);
    c.la = lds_address(smem + (kt % kStages) * STAGE) + wave * 1024;
    c.lb = c.la + A_BYTES;
    c.klim = p.k - k0;
    c.tail = tail;
    return c;
  };
  auto issue_one = [&](const LoadCtx& c, int j) __attribute__((always_inline)) {
    if (j < A_LOADS)
      load_lds16(c.ra, c.la + j * NW * 1024, (c.tail && a_kpos[j] >= c.klim) ? kOOB : a_voff[j]);
    else
      load_lds16(c.rb, c.lb + (j - A_LOADS) * NW * 1024,
                 (c.tail && b_kpos[j - A_LOADS] >= c.klim) ? kOOB : b_voff[j - A_LOADS]);
  };
  auto issue = [&](int kt, bool tail) __attribute__((always_inline)) {
    const LoadCtx c = load_ctx(kt, tail);
#pragma unroll
    for (int j = 0; j < LPS; ++j) issue_one(c, j);
  };

  // The chunk holding K's last bytes also holds the row's padding; zero the
  // bytes at or past K in the K-contiguous tiles of the last stage (one row
  // per thread, at most 15 bytes each).
  auto zero_k_padding = [&](int kt) __attribute__((always_inline)) {
    const int kin = p.k - kt * kBK;
    const int c_lo = kin & ~15;
    lds_char_t* sa = smem + (kt % kStages) * STAGE;
    constexpr int ROWS = (A_KC ? BM : 0) + (B_KC ? BN : 0);
    for (int r = threadIdx.x; r < ROWS; r += kThreads) {
      const bool in_a = A_KC && r < BM;
      const int row = in_a || !A_KC ? r : r - BM;
      lds_char_t* rp = sa + (in_a ? 0 : A_BYTES) + row * kBK + (((c_lo >> 4) ^ swz_k(row)) << 4) - c_lo;
#pragma nounroll
      for (int b = kin; b < c_lo + 16; ++b) rp[b] = 0;
    }
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};

  // Fragments of two consecutive stages live in registers: while the MFMAs
  // of stage kt run, the LDS reads of stage kt+1 and the global loads of
  // stage kt+kStages are in flight.
  v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  auto read_frags = [&](int kt, v8i (&fa)[TM], v8i (&fb)[TN]) __attribute__((always_inline)) {
    const lds_char_t* sa = smem + (kt % kStages) * STAGE;
    const lds_char_t* sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = load_frag<A_KC, BM>(sa, wm * WM + i * 32, lane);
#pragma unroll
    for (int i = 0; i < TN; ++i) fb[i] = load_frag<B_KC, BN>(sb, wn * WN + i * 32, lane);
  };
  auto mfmas = [&](const v8i (&fa)[TM], const v8i (&fb)[TN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], FB, FA, 0, 0, 0, 0);
  };

  const int kt_total = (p.k + kBK - 1) / kBK;
  const int kt_full = p.k / kBK;
  const bool kfix = (p.k & 15) != 0;
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < kt_total) issue(s, s >= kt_full);
  if (kt_total > 0) {
    wait_stages<LPS, kStages>(min(kStages, kt_total) - 1);
    lds_barrier();
    if (kfix && kt_full == 0) {
      zero_k_padding(0);
      lds_barrier();
    }
    read_frags(0, fa0, fb0);
  }

  // Steady state, two stages per trip with no conditions: make stage kt+1
  // visible, then issue stage kt's MFMAs one by one, each followed by its
  // share of the global loads of stage kt+kStages (into the buffer stage kt
  // freed) and of the LDS reads of stage kt+1's fragments.  Scheduling
  // barriers keep that interleave: bursts of loads or LDS reads right after
  // the barrier left the matrix cores idle.  The wave runs at raised priority
  // while it issues the MFMA stream.
  constexpr int NM = TM * TN, NF = TM + TN;
  auto steady = [&](int kt, const v8i (&fa)[TM], const v8i (&fb)[TN], v8i (&na)[TM], v8i (&nb)[TN])
                    __attribute__((always_inline)) {
    wait_stages<LPS, kStages>(kStages - 2);
    lds_barrier();
    const LoadCtx c = load_ctx(kt + kStages, kt + kStages >= kt_full);
    const lds_char_t* sa = smem + ((kt + 1) % kStages) * STAGE;
    const lds_char_t* sb = sa + A_BYTES;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int i = q / TM, j = q % TM;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[i], fa[j], acc[i][j], FB, FA, 0, 0, 0, 0);
#pragma unroll
      for (int l = q * LPS / NM; l < (q + 1) * LPS / NM; ++l) issue_one(c, l);
#pragma unroll
      for (int f = q * NF / NM; f < (q + 1) * NF / NM; ++f) {
        if (f < TM) na[f] = load_frag<A_KC, BM>(sa, wm * WM + f * 32, lane);
        else nb[f - TM] = load_frag<B_KC, BN>(sb, wn * WN + (f - TM) * 32, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // The last stages: the same with the prefetch and the next reads guarded.
  auto drain = [&](int kt, const v8i (&fa)[TM], const v8i (&fb)[TN], v8i (&na)[TM], v8i (&nb)[TN])
                   __attribute__((always_inline)) {
    if (kt + 1 < kt_total) {
      wait_stages<LPS, kStages>(min(kt + kStages - 1, kt_total - 1) - (kt + 1));
      lds_barrier();
      if (kfix && kt + 1 == kt_full) {
        zero_k_padding(kt + 1);
        lds_barrier();
      }
      if (kt + kStages < kt_total) issue(kt + kStages, kt + kStages >= kt_full);
      read_frags(kt + 1, na, nb);
    }
    mfmas(fa, fb);
  };
  int kt = 0;
  for (; kt + kStages + 1 < kt_total; kt += 2) {
    steady(kt, fa0, fb0, fa1, fb1);
    steady(kt + 1, fa1, fb1, fa0, fb0);
  }
  for (; kt < kt_total; kt += 2) {
    drain(kt, fa0, fb0, fa1, fb1);
    if (kt + 1 < kt_total) drain(kt + 1, fa1, fb1, fa0, fb0);
  }

  // Epilogue: y = acc * (sa_inv * sb_inv) + bias[n], one bf16 rounding.
  const float alpha = p.a_scale_inv[0] * p.b_scale_inv[0];
  uint16_t* cb = p.c + bt * p.stride_c;
#pragma unroll
  for (int i = 0; i < TN; ++i) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int n = n0 + wn * WN + i * 32 + 8 * rq + 4 * (lane >> 5);
      if (n >= p.n) continue;
      float bias4[4] = {0.f, 0.f, 0.f, 0.f};
      const bool full4 = n + 3 < p.n;
      if (p.bias_kind == 1) {
        const uint16_t* bp = static_cast<const uint16_t*>(p.bias) + n;
        if (full4) {
          const uint2 w = *reinterpret_cast<const uint2*>(bp);
          bias4[0] = __uint_as_float(w.x << 16);
          bias4[1] = __uint_as_float(w.x & 0xFFFF0000u);
          bias4[2] = __uint_as_float(w.y << 16);
          bias4[3] = __uint_as_float(w.y & 0xFFFF0000u);
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < p.n) bias4[e] = __uint_as_float((uint32_t)bp[e] << 16);
        }
      } else if (p.bias_kind == 2) {
        const float* bp = static_cast<const float*>(p.bias) + n;
        if (full4) {
          const float4 w = *reinterpret_cast<const float4*>(bp);
          bias4[0] = w.x; bias4[1] = w.y; bias4[2] = w.z; bias4[3] = w.w;
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < p.n) bias4[e] = bp[e];
        }
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + wm * WM + j * 32 + (lane & 31);
        if (m >= p.m) continue;
        const float y0 = __builtin_fmaf(acc[i][j][4 * rq + 0], alpha, bias4[0]);
        const float y1 = __builtin_fmaf(acc[i][j][4 * rq + 1], alpha, bias4[1]);
        const float y2 = __builtin_fmaf(acc[i][j][4 * rq + 2], alpha, bias4[2]);
        const float y3 = __builtin_fmaf(acc[i][j][4 * rq + 3], alpha, bias4[3]);
        uint16_t* dst = cb + (int64_t)m * p.ldc + n;
        if (full4) {
          *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        } else {
          const uint32_t lo = pack_bf16x2(y0, y1), hi = pack_bf16x2(y2, y3);
          const uint16_t v[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
          for (int e = 0; e < 4; ++e)
            if (n + e < p.n) dst[e] = v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: tile family and dispatch.

struct TileCfg {
  int bm, bn, waves;
};
// Tile family (index = the tile argument of fp8_mm_with_tile).  256x256 with
// four waves runs one workgroup per CU (4 LDS stages, 128 KiB), each wave a
// 128x128 block; the eight-wave 256x256 tiles give every SIMD two waves of a
// 128x64 / 64x128 block so one wave's memory stalls hide behind the other's
// MFMAs; 256x128 / 128x256 run two workgroups per CU (3 stages, 72 KiB
// each); 128x128 and 64x64 serve problems too small to fill the chip.
constexpr TileCfg kTiles[] = {{256, 256, 4}, {128, 128, 4}, {64, 64, 4}, {256, 128, 4},
                              {128, 256, 4}, {256, 256, 8}, {256, 256, 8}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

typedef void (*GemmFn)(GemmKArgs);

template <int BM, int BN, int WGM, int WGN, int ST, int OCC>
GemmFn pick_kernel(int layout, int fa, int fb) {
#define FP8DS_FMT_CASES(AKC, BKC)                                                              \
  if (fa == 0 && fb == 0) return gemm_kernel<BM, BN, WGM, WGN, ST, AKC, BKC, 0, 0, OCC>;       \
  if (fa == 1 && fb == 0) return gemm_kernel<BM, BN, WGM, WGN, ST, AKC, BKC, 1, 0, OCC>;       \
  if (fa == 0 && fb == 1) return gemm_kernel<BM, BN, WGM, WGN, ST, AKC, BKC, 0, 1, OCC>;       \
  return gemm_kernel<BM, BN, WGM, WGN, ST, AKC, BKC, 1, 1, OCC>;
  if (layout == 0) { FP8DS_FMT_CASES(true, true) }
  if (layout == 1) { FP8DS_FMT_CASES(true, false) }
  FP8DS_FMT_CASES(false, false)
#undef FP8DS_FMT_CASES
}

GemmFn kernel_for(int tile, int layout, int fa, int fb) {
  switch (tile) {
    case 0: return pick_kernel<256, 256, 2, 2, 4, 1>(layout, fa, fb);
    case 1: return pick_kernel<128, 128, 2, 2, 4, 2>(layout, fa, fb);
    case 2: return pick_kernel<64, 64, 2, 2, 4, 4>(layout, fa, fb);
    case 3: return pick_kernel<256, 128, 2, 2, 3, 2>(layout, fa, fb);
    case 4: return pick_kernel<128, 256, 2, 2, 3, 2>(layout, fa, fb);
    case 5: return pick_kernel<256, 256, 2, 4, 4, 1>(layout, fa, fb);
    default: return pick_kernel<256, 256, 4, 2, 4, 1>(layout, fa, fb);
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest tile whose grid still fills the 256 CUs; else the one with most tiles.
int choose_tile(const GemmProblem& p) {
  // Largest tile whose grid still fills the 256 CUs, else the one with most
  // tiles.  For the 256x256 size the eight-wave variant measured faster.
  constexpr int64_t kCUs = 256;
  constexpr int order[] = {6, 1, 2};
  for (int t : order) {
    const int64_t tiles = cdiv(p.m, kTiles[t].bm) * cdiv(p.n, kTiles[t].bn) * p.batch;
    if (tiles >= kCUs) return t;
  }
  return 2;
}

}  // namespace

int launch_gemm(const GemmProblem& p, int tile_override, hipStream_t stream) {
  const int t = (tile_override >= 0 && tile_override < kNumTiles) ? tile_override : choose_tile(p);
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
  k.bias_kind = p.bias_kind;
  const int64_t total = (int64_t)k.tiles_m * k.tiles_n * k.batch;
  if (total > 0x7FFFFFFF) return set_error(-3, "fp8_mm: %lld tiles exceed the grid limit", (long long)total);
  GemmFn fn = kernel_for(t, p.layout, p.fmt_a, p.fmt_b);
  hipLaunchKernelGGL(fn, dim3((unsigned)total), dim3(64 * kTiles[t].waves), 0, stream, k);
  return check_launch("gemm_kernel");
}

}  // namespace fp8ds
