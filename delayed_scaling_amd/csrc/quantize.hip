// Delayed-scaling FP8 quantize with a fused amax and an in-kernel scale-ring
// update, its transposed / dual form, the dynamic recipe's amax pass and the
// bias-gradient column sum.
//
// Pages (AstrAI commit histories):
//  * astrai/extension/fp8.py @4dc5e923, ring-finalize entry: the history
//    update and the next scale are computed inside the quantize launch, by
//    whichever block completes last, rather than by a launch of their own;
//  * fp8.py @f4c44ebf: the quantize is templated on its input type (bf16,
//    fp16, fp32); the bias gradient is a column sum taken only when needed,
//    over a dequantized gradient when the gradient is pre-quantized;
//  * history of `tests`: quantize and quantize_dual with a layout enum, the
//    two orientations byte-equal to the plain one;
//  * fp8.py @4dc5e923: the dynamic recipe measures its scale inline.
//
// Each quantize launch streams x once (16-byte loads), so the kernels are
// bound by HBM.  Each block reduces max|x| over its elements and climbs a
// completion tree kept in the ring's scratch lines (a per-group max + ticket,
// then a top-level ticket; a one-block launch skips it); the block holding
// the last top-level ticket finalizes the ring and every scratch word is back
// at zero for the next call on the same stream.
#include <atomic>

#include "device_common.h"
#include "fp8ds.h"
#include "launch.h"

namespace fp8ds {

namespace {

constexpr int kQBlock = 256;     // threads per block
constexpr int kQUnroll = 4;      // 16-byte chunks in flight per thread
constexpr int kDefaultBlocks = 1024;  // grid cap: 4 blocks per CU; larger inputs loop
constexpr int kFlatTree = 64;         // launches of at most this many blocks skip the group level
constexpr int k2dBlocks = 1024;       // grid cap of the transposed / dual quantize

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Element types.  mag() is a bit pattern of |x| that orders like |x| (NaN
// above infinity); mag_f32() turns the largest one into float32 bits.

template <int IN>
struct In;
template <>
struct In<kInBf16> {
  static constexpr int kBits = 16;
  static constexpr uint32_t kInfMag = 0x7F80u;
  __device__ static float f(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static uint32_t mag(uint32_t b) { return b & 0x7FFFu; }
  __device__ static uint32_t mag_f32(uint32_t m) { return m << 16; }
  __device__ static uint32_t sign(uint32_t b) { return (b >> 8) & 0x80u; }
};
template <>
struct In<kInF16> {
  static constexpr int kBits = 16;
  static constexpr uint32_t kInfMag = 0x7C00u;
  __device__ static float f(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }
  __device__ static uint32_t mag(uint32_t b) { return b & 0x7FFFu; }
  // Widened exactly, NaN payloads included: infinity and NaN move their
  // mantissa bits up unchanged (a signalling NaN stays signalling, where the
  // hardware convert would quiet it); finite values convert exactly.
  __device__ static uint32_t mag_f32(uint32_t m) {
    return m >= kInfMag ? 0x7F800000u | ((m & 0x3FFu) << 13) : __float_as_uint(f(m));
  }
  __device__ static uint32_t sign(uint32_t b) { return (b >> 8) & 0x80u; }
};
template <>
struct In<kInF32> {
  static constexpr int kBits = 32;
  static constexpr uint32_t kInfMag = 0x7F800000u;
  __device__ static float f(uint32_t b) { return __uint_as_float(b); }
  __device__ static uint32_t mag(uint32_t b) { return b & 0x7FFFFFFFu; }
  __device__ static uint32_t mag_f32(uint32_t m) { return m; }
  __device__ static uint32_t sign(uint32_t b) { return (b >> 24) & 0x80u; }
};

// Casts two products to the format's codes in the low or high half-word of
// `word`.  Products are clamped to +-FMAX first because the hardware convert
// is nearest-even but does not saturate; NaN is repaired by the caller.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b, uint32_t word) {
  if constexpr (FMT == kE4M3)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)word, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)word, HI);
}

template <int FMT>
__device__ __forceinline__ float clamp_fmax(float v) {
  constexpr float m = FmtTraits<FMT>::kMax;
  return fminf(fmaxf(v, -m), m);
}

// Four elements (raw bits) to four codes packed in one word; NaN elements
// come out as whatever the convert makes of the clamped value (nan_fix4
// repairs them).
template <int FMT, int IN>
__device__ __forceinline__ uint32_t cvt4(const uint32_t (&e)[4], float scale) {
  using T = In<IN>;
  const uint32_t out =
      cvt_pair<FMT, false>(clamp_fmax<FMT>(T::f(e[0]) * scale), clamp_fmax<FMT>(T::f(e[1]) * scale), 0u);
  return cvt_pair<FMT, true>(clamp_fmax<FMT>(T::f(e[2]) * scale), clamp_fmax<FMT>(T::f(e[3]) * scale), out);
}

// A NaN element encodes as 0x7F with its sign.
template <int IN>
__device__ __forceinline__ uint32_t nan_fix4(const uint32_t (&e)[4], uint32_t out) {
  using T = In<IN>;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (T::mag(e[i]) > T::kInfMag) out = (out & ~(0xFFu << (8 * i))) | ((0x7Fu | T::sign(e[i])) << (8 * i));
  return out;
}

// Four elements (raw bits) to four codes packed in one word, NaN included.
// amag collects max mag().
template <int FMT, int IN>
__device__ __forceinline__ uint32_t quant4(const uint32_t (&e)[4], float scale, uint32_t& amag) {
  using T = In<IN>;
  const uint32_t m = max(max(T::mag(e[0]), T::mag(e[1])), max(T::mag(e[2]), T::mag(e[3])));
  amag = max(amag, m);
  const uint32_t out = cvt4<FMT, IN>(e, scale);
  return m > T::kInfMag ? nan_fix4<IN>(e, out) : out;
}

// 16 input bytes -> codes: 8 elements -> 2 words for 16-bit types, 4
// elements -> 1 word for fp32.
template <int FMT, int IN>
__device__ __forceinline__ void quant16(v4u v, float scale, uint32_t (&out)[2], uint32_t& amag) {
  if constexpr (In<IN>::kBits == 16) {
    const uint32_t e0[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
    const uint32_t e1[4] = {v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
    out[0] = quant4<FMT, IN>(e0, scale, amag);
    out[1] = quant4<FMT, IN>(e1, scale, amag);
  } else {
    const uint32_t e[4] = {v.x, v.y, v.z, v.w};
    out[0] = quant4<FMT, IN>(e, scale, amag);
  }
}

// Elements (raw bits) of 16 input bytes: 8 for 16-bit types (e[0..7]), 4 for
// fp32 (e[0..3]).
template <int IN>
__device__ __forceinline__ void split16(v4u v, uint32_t (&e0)[4], uint32_t (&e1)[4]) {
  if constexpr (In<IN>::kBits == 16) {
    e0[0] = v.x & 0xFFFFu; e0[1] = v.x >> 16; e0[2] = v.y & 0xFFFFu; e0[3] = v.y >> 16;
    e1[0] = v.z & 0xFFFFu; e1[1] = v.z >> 16; e1[2] = v.w & 0xFFFFu; e1[3] = v.w >> 16;
  } else {
    e0[0] = v.x; e0[1] = v.y; e0[2] = v.z; e0[3] = v.w;
    e1[0] = e1[1] = e1[2] = e1[3] = 0u;
  }
}

// Running max of mag() over whole 16-byte chunks.  16-bit types keep one
// maximum per half-word (packed u16 max, one instruction per input word);
// fp32 keeps one per word.
template <int IN>
struct MagMax {
  uint32_t m = 0;   // two u16 maxima for 16-bit types, one u32 for fp32
  __device__ __forceinline__ void add(v4u v) {
    if constexpr (In<IN>::kBits == 16) {
      u16x2 a = __builtin_bit_cast(u16x2, m);
      a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu));
      a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
      a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu));
      a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
      m = __builtin_bit_cast(uint32_t, a);
    } else {
      m = max(max(m, v.x & 0x7FFFFFFFu), max(v.y & 0x7FFFFFFFu, max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
    }
  }
  // The largest mag() seen, as one value.
  __device__ __forceinline__ uint32_t get() const {
    if constexpr (In<IN>::kBits == 16) return max(m & 0xFFFFu, m >> 16);
    else return m;
  }
};

// U whole 16-byte chunks to codes (o[u][0..1] for 16-bit types, o[u][0] for
// fp32), NaN included, their max mag() folded into amag.  The NaN repair is
// one wave-uniform test per group: it runs only when some lane's group holds
// a NaN.
template <int FMT, int IN, int U>
__device__ __forceinline__ void quant_group(const v4u (&v)[U], float scale, uint32_t (&o)[U][2], uint32_t& amag) {
  using T = In<IN>;
  MagMax<IN> g;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    g.add(v[u]);
    uint32_t e0[4], e1[4];
    split16<IN>(v[u], e0, e1);
    o[u][0] = cvt4<FMT, IN>(e0, scale);
    o[u][1] = T::kBits == 16 ? cvt4<FMT, IN>(e1, scale) : 0u;
  }
  const uint32_t m = g.get();
  amag = max(amag, m);
  const bool nan = m > T::kInfMag;
  if (__builtin_amdgcn_ballot_w64(nan) != 0 && nan) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t e0[4], e1[4];
      split16<IN>(v[u], e0, e1);
      o[u][0] = nan_fix4<IN>(e0, o[u][0]);
      if constexpr (T::kBits == 16) o[u][1] = nan_fix4<IN>(e1, o[u][1]);
    }
  }
}

// Waits until every vector-memory operation of this wave has completed,
// the returning atomic that produced v included, before anything after it
// is issued.  The completion tree orders its atomics this way rather than by
// release/acquire fences (an agent-scope fence writes back the whole L2).
__device__ __forceinline__ void wait_returned(uint32_t v) {
  asm volatile("s_waitcnt vmcnt(0)" : : "v"(v) : "memory");
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Block-wide max, read by every thread after one barrier.  Each kernel calls
// it once, at its end, so `red` needs no barrier before it is written.
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kQBlock / 64; ++i) r = max(r, red[i]);
  return r;
}

// Completion tree, called by thread 0 of every block with the block's max
// |x| as float32 bits; G blocks take part, this one is number b.  All words
// are device-scope atomics, performed where every XCD sees them, and a ticket
// is taken only after the max (or ticket) it covers has been performed (its
// returned value is waited for).  No release/acquire fence is needed: the
// only data handed between blocks are the atomic words themselves.
//  * At most kFlatTree blocks: each block takes the top-level max, then the
//    top-level ticket.  Returns kTopMax in the block drawing the last ticket:
//    the top-level max then covers every block.
//  * More: block b belongs to group b % kRingGroups, whose 64-byte line
//    holds a running max and a ticket; each block takes its group's max, then
//    the group's ticket, and the block drawing a group's last ticket takes a
//    top-level ticket.  Returns kGroupMax in the block drawing the last
//    top-level ticket: every group's max is then final (each of its members
//    took it before its group ticket, and the group's last member took the
//    top-level ticket after all of those), so the launch's max is the max of
//    the group words.  Four dependent round trips on the last block's path.
constexpr int kNotLast = 0, kTopMax = 1, kGroupMax = 2;
__device__ int climb_tree(RingHeader* ring, uint32_t bmax, int G, int b) {
  if (G <= kFlatTree) {
    const uint32_t prev = __hip_atomic_fetch_max(&ring->amax_bits, bmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_returned(prev);
    const uint32_t t = __hip_atomic_fetch_add(&ring->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_returned(t);
    return t == (uint32_t)G - 1 ? kTopMax : kNotLast;
  }
  static_assert(kFlatTree >= kRingGroups, "a two-level launch fills every group");
  const int g = b % kRingGroups;
  const uint32_t members = (uint32_t)((G - g + kRingGroups - 1) / kRingGroups);
  RingGroup* grp = ring_groups(ring) + g;
  const uint32_t prev = __hip_atomic_fetch_max(&grp->amax_bits, bmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_returned(prev);
  const uint32_t t = __hip_atomic_fetch_add(&grp->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_returned(t);
  if (t != members - 1) return kNotLast;
  const uint32_t t2 = __hip_atomic_fetch_add(&ring->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_returned(t2);
  return t2 == (uint32_t)kRingGroups - 1 ? kGroupMax : kNotLast;
}

// Called by every thread at the end of a launch of G blocks (this one number
// b).  Reduces the block's max, climbs the tree and returns true in wave 0 of
// the one block that finishes last, with *a = max |x| of the launch (float32
// bits, the same in every lane).  Other waves, and other blocks, return false
// and are done; the caller finalizes the ring with wave 0.
__device__ __forceinline__ bool fold_amax(RingHeader* ring, uint32_t amag_f32, uint32_t* red, int G, int b,
                                          uint32_t* a) {
  const uint32_t bmax = block_max(amag_f32, red);
  if (threadIdx.x >= 64) return false;
  if (G == 1) {
    // The only block: its max is the launch's, and the tree's words are
    // never touched (they stay zero), which saves three dependent round
    // trips to the device-scope atomics on small tensors.
    *a = __builtin_amdgcn_readfirstlane(bmax);
    return true;
  }
  int kind = kNotLast;
  if (threadIdx.x == 0) kind = climb_tree(ring, bmax, G, b);
  kind = __builtin_amdgcn_readfirstlane(kind);
  if (kind == kNotLast) return false;
  uint32_t v = 0u;
  if (kind == kTopMax) {
    if (threadIdx.x == 0) {
      v = __hip_atomic_load(&ring->amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_returned(v);
    }
    v = __builtin_amdgcn_readfirstlane(v);
  } else {
    // Lane g reads group g's max, then clears the group's line: no other
    // block touches it again in this launch.  (Plain atomic loads and
    // stores: an exchange whose returned value shared a register with its
    // data was measured returning the new value on this target.)
    RingGroup* grp = ring_groups(ring) + threadIdx.x;
    if (threadIdx.x < kRingGroups) {
      v = __hip_atomic_load(&grp->amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_returned(v);
      __hip_atomic_store(&grp->amax_bits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&grp->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    v = __builtin_amdgcn_readfirstlane(wave_max(v));
  }
  *a = v;
  return true;
}

__device__ __forceinline__ void clear_top(RingHeader* ring) {
  __hip_atomic_store(&ring->amax_bits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&ring->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The ring as a launch finds it, read once at kernel start: the scale it
// applies, the header, and in wave 0 the first 64 history entries other than
// slot idx (lane j holds entry j, float32 bits, 0 for idx and past the end).
// Nothing else writes the ring until the launch's last block finalizes it, so
// that block needs no further loads for windows of up to 64 entries.
struct RingPre {
  float scale;
  int hist_len, idx, fmt;
  uint32_t win;
};

__device__ __forceinline__ bool header_ok(int H, int idx) {
  return H >= 1 && H <= FP8DS_RING_MAX_HIST && idx >= 0 && idx < H;
}

__device__ __forceinline__ RingPre read_ring(RingHeader* ring) {
  RingPre p;
  p.scale = ring->scale;
  p.hist_len = ring->hist_len;
  p.idx = ring->idx;
  p.fmt = ring->fmt;
  p.win = 0u;
  const int lane = (int)threadIdx.x;
  if (lane < 64 && header_ok(p.hist_len, p.idx) && lane < p.hist_len && lane != p.idx)
    p.win = __float_as_uint(ring_hist(ring)[lane]);
  return p;
}

// The delayed-scaling ring update, run by wave 0 of the last block with the
// launch's amax a: hist[idx] = a, idx advances, the next scale is FMAX over
// the window's max when that is finite and positive and the quotient finite,
// scale_inv_used = 1/scale (the scale this launch applied), amax_last = a.
// scale_inv_out, when given, also receives 1/scale.
template <int FMT>
__device__ void finalize_ring(RingHeader* ring, const RingPre& p, uint32_t a, float* scale_inv_out) {
  const bool bad_header = !header_ok(p.hist_len, p.idx);
  const bool fmt_mismatch = p.fmt != FMT;
  float* hist = ring_hist(ring);
  uint32_t w = max(p.win, a);
  if (!bad_header) {
    for (int j = 64 + (int)threadIdx.x; j < p.hist_len; j += 64)
      if (j != p.idx) w = max(w, __float_as_uint(hist[j]));
  }
  w = wave_max(w);
  if (threadIdx.x == 0) {
    if (bad_header || fmt_mismatch) {
      ring->status |= (bad_header ? kStatusBadHeader : 0u) | (fmt_mismatch ? kStatusFmtMismatch : 0u);
    } else {
      hist[p.idx] = __uint_as_float(a);
      ring->idx = p.idx + 1 == p.hist_len ? 0 : p.idx + 1;
      float next = p.scale;
      if (w > 0u && w < 0x7F800000u) {
        const float t = FmtTraits<FMT>::kMax / __uint_as_float(w);
        if (__float_as_uint(t) < 0x7F800000u) next = t;
      }
      ring->scale = next;
      ring->scale_inv_used = 1.0f / p.scale;
      ring->amax_last = __uint_as_float(a);
    }
    if (scale_inv_out != nullptr) *scale_inv_out = 1.0f / p.scale;
    clear_top(ring);
  }
}

// ---------------------------------------------------------------------------
// Row-wise quantize: x is a flat array of numel elements, nchunk whole 16-byte
// chunks and `tail` elements after them.  One launch serves one tensor
// (quantize_kernel) or up to kMaxBatch tensors with their own rings
// (quantize_batch_kernel: consecutive runs of blocks per tensor, each run a
// launch of its own as far as the tree is concerned).

struct QuantJob {
  const v4u* x;
  uint8_t* y;
  int64_t nchunk;
  const uint8_t* x_tail;
  uint8_t* y_tail;
  int32_t tail;
  int32_t blocks;            // blocks of this job (its grid)
  RingHeader* ring;
  float* scale_inv_out;      // optional copy of the applied 1/scale
};

constexpr int kMaxBatch = FP8DS_MAX_BATCH;
struct QuantBatch {
  QuantJob job[kMaxBatch];
  int32_t njobs;
};

// Block b of a G-block grid over job j.
template <int FMT, int IN>
__device__ __forceinline__ void quantize_rows(const QuantJob& j, int G, int b, uint32_t* red) {
  using T = In<IN>;
  constexpr int kOut = T::kBits == 16 ? 8 : 4;   // codes per 16 input bytes
  const RingPre pre = read_ring(j.ring);
  const float scale = pre.scale;
  const v4u* __restrict__ x = j.x;
  uint8_t* __restrict__ y = j.y;
  const int64_t nchunk = j.nchunk;
  uint32_t amag = 0;

  // Streaming stores on every path (the compiler may merge the paths'
  // stores; a plain store there measured 12 % slower on the whole pass).
  auto put = [&](int64_t c, const uint32_t (&o)[2]) __attribute__((always_inline)) {
    if constexpr (kOut == 8)
      __builtin_nontemporal_store(v2u{o[0], o[1]}, reinterpret_cast<v2u*>(y) + c);
    else
      __builtin_nontemporal_store(o[0], reinterpret_cast<uint32_t*>(y) + c);
  };
  const int64_t step = (int64_t)G * kQBlock * kQUnroll;
  for (int64_t base = (int64_t)b * kQBlock * kQUnroll + threadIdx.x; base < nchunk; base += step) {
    if (base + (kQUnroll - 1) * kQBlock < nchunk) {
      v4u v[kQUnroll];
#pragma unroll
      for (int u = 0; u < kQUnroll; ++u) v[u] = __builtin_nontemporal_load(x + base + u * kQBlock);
      uint32_t o[kQUnroll][2];
      quant_group<FMT, IN, kQUnroll>(v, scale, o, amag);
#pragma unroll
      for (int u = 0; u < kQUnroll; ++u) put(base + u * kQBlock, o[u]);
    } else {
      for (int u = 0; u < kQUnroll; ++u) {
        const int64_t c = base + u * kQBlock;
        if (c < nchunk) {
          uint32_t o[2];
          quant16<FMT, IN>(x[c], scale, o, amag);
          put(c, o);
        }
      }
    }
  }
  // Elements past the last whole 16-byte chunk.
  if (j.tail > 0 && b == 0 && threadIdx.x == 0) {
    for (int i = 0; i < j.tail; ++i) {
      uint32_t e[4] = {0u, 0u, 0u, 0u};
      if constexpr (T::kBits == 16) e[0] = reinterpret_cast<const uint16_t*>(j.x_tail)[i];
      else e[0] = reinterpret_cast<const uint32_t*>(j.x_tail)[i];
      j.y_tail[i] = (uint8_t)(quant4<FMT, IN>(e, scale, amag) & 0xFFu);
    }
  }

  uint32_t a;
  if (!fold_amax(j.ring, T::mag_f32(amag), red, G, b, &a)) return;
  finalize_ring<FMT>(j.ring, pre, a, j.scale_inv_out);
}

template <int FMT, int IN>
__global__ __launch_bounds__(kQBlock) void quantize_kernel(QuantJob job) {
  __shared__ uint32_t red[kQBlock / 64];
  quantize_rows<FMT, IN>(job, (int)gridDim.x, (int)blockIdx.x, red);
}

template <int FMT, int IN>
__global__ __launch_bounds__(kQBlock) void quantize_batch_kernel(QuantBatch batch) {
  __shared__ uint32_t red[kQBlock / 64];
  int b = (int)blockIdx.x, j = 0;
  while (j + 1 < batch.njobs && b >= batch.job[j].blocks) {
    b -= batch.job[j].blocks;
    ++j;
  }
  quantize_rows<FMT, IN>(batch.job[j], batch.job[j].blocks, b, red);
}

// ---------------------------------------------------------------------------
// Transposed / dual quantize of an R x C row-major tensor, R and C multiples
// of 16.  A block takes a 128-row x 128-column tile:
//  1. threads quantize 16-byte pieces of the tile's rows, consecutive threads
//     on consecutive pieces (and, for the dual form, store those codes), and
//     write the codes to an LDS tile [128 rows][128 codes] whose 16-byte
//     chunks are XOR-swizzled per row;
//  2. transpose reads (ds_read_b64_tr_b8) hand each lane 64 consecutive rows
//     of one column, which it writes to a second LDS tile [128 columns][128
//     rows] (rows padded to 144 bytes against bank conflicts);
//  3. eight lanes per column then store 16 bytes each: every store
//     instruction writes whole 128-byte lines of the transposed output.
// Each tile row reads 256 contiguous input bytes (bf16): on this part the
// mix of row reads and transposed 128-byte writes measured 6-10 % faster
// with 256-byte than with 128-byte read segments (a probe that only moves
// the bytes), and the 64-column tile of the first version left the kernel
// at 0.56 of the HBM nameplate.

constexpr int kTileR = 128, kTileC = 128, kTStride = kTileR + 16;

// Chunk c of codes-tile row r sits at c ^ tile_swz(r): the 8 rows of a
// transpose read (one 16-byte chunk each, 128-byte rows) then fall on 8
// distinct 16-byte bank slots.
__device__ __forceinline__ int tile_swz(int r) { return (r >> 1) & 7; }

template <int FMT, int IN, bool DUAL>
__global__ __launch_bounds__(kQBlock) void quantize_2d_kernel(const uint8_t* __restrict__ x, uint8_t* __restrict__ y,
                                                              uint8_t* __restrict__ y_t, int rows, int cols,
                                                              int tiles_c, RingHeader* __restrict__ ring) {
  using T = In<IN>;
  constexpr int kElemBytes = T::kBits / 8;
  __shared__ __attribute__((aligned(16))) char codes_lds[kTileR * kTileC];
  __shared__ __attribute__((aligned(16))) char trans_lds[kTileC * kTStride];
  __shared__ uint32_t red[kQBlock / 64];
  const RingPre pre = read_ring(ring);
  const float scale = pre.scale;
  uint32_t amag = 0;
  lds_char_t* tile = (lds_char_t*)codes_lds;
  lds_char_t* ttile = (lds_char_t*)trans_lds;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = ((rows + kTileR - 1) / kTileR) * tiles_c;
  // Loads: 16 bytes each, kPer elements; kLoads per tile row, consecutive
  // threads on consecutive pieces of a row, so each load instruction reads
  // whole 128-byte lines.
  constexpr int kPer = 16 / kElemBytes, kLoads = kTileC / kPer, kIters = kTileR * kLoads / kQBlock;
  constexpr int kWords = kPer / 4;                            // code words per load
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int r0 = (t / tiles_c) * kTileR, c0 = (t % tiles_c) * kTileC;
    v4u cur[kIters];
#pragma unroll
    for (int j = 0; j < kIters; ++j) {
      const int item = threadIdx.x + j * kQBlock;
      const int r = r0 + item / kLoads, c = c0 + (item % kLoads) * kPer;
      cur[j] = v4u{0u, 0u, 0u, 0u};                          // cols % 16 == 0: a load is wholly in or out
      if (r < rows && c < cols)
        cur[j] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + ((int64_t)r * cols + c) * kElemBytes));
    }
    uint32_t w[kIters][2];
    quant_group<FMT, IN, kIters>(cur, scale, w, amag);
    if constexpr (DUAL) {
#pragma unroll
      for (int j = 0; j < kIters; ++j) {
        const int item = threadIdx.x + j * kQBlock;
        const int r = r0 + item / kLoads, c = c0 + (item % kLoads) * kPer;
        if (r < rows && c < cols) {
          if constexpr (kWords == 2)
            __builtin_nontemporal_store(v2u{w[j][0], w[j][1]}, reinterpret_cast<v2u*>(y + (int64_t)r * cols + c));
          else
            __builtin_nontemporal_store(w[j][0], reinterpret_cast<uint32_t*>(y + (int64_t)r * cols + c));
        }
      }
    }
    __syncthreads();   // the previous tile's reads of both LDS tiles are done
#pragma unroll
    for (int j = 0; j < kIters; ++j) {
      const int item = threadIdx.x + j * kQBlock;
      const int tr = item / kLoads, piece = item % kLoads;
      const int byte = piece * kPer;                          // code byte in the row
      lds_char_t* p = tile + tr * kTileC + (((byte >> 4) ^ tile_swz(tr)) << 4) + (byte & 15);
      if constexpr (kWords == 2) *(lds_v2i_t*)p = v2i{(int)w[j][0], (int)w[j][1]};
      else *(__attribute__((address_space(3))) int*)p = (int)w[j][0];
    }
    __syncthreads();
    {
      // Lane l of wave w takes column 32*w + l%32 and tile rows 64*(l/32) +
      // [0, 64).  Within each 16-lane group, the even lanes address rows
      // k..k+7 of the group's 16-column chunk and the odd lanes the other 8
      // bytes of those rows; each read hands a lane 8 consecutive rows of its
      // column.
      const int col = 32 * wave + (lane & 31);
      const int rbase = 64 * (lane >> 5);
      const int q = lane & 15;
      const int chunk = 2 * wave + ((lane >> 4) & 1);
      v2i part[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const int kr = rbase + 8 * h + (q >> 1);
        const int addr = kr * kTileC + ((chunk ^ tile_swz(kr)) << 4) + 8 * (q & 1);
        part[h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(tile + addr));
      }
      lds_char_t* dst = ttile + col * kTStride + rbase;
#pragma unroll
      for (int h = 0; h < 8; h += 2)
        *(lds_v4i_t*)(dst + 8 * h) = v4i{part[h][0], part[h][1], part[h + 1][0], part[h + 1][1]};
    }
    __syncthreads();
    // Eight lanes per column, 16 bytes each: column t/8 + 32*j, rows
    // 16*(t%8) + [0, 16) of the tile.  (A plain store: streaming stores of
    // the transposed output measured 7 % slower here.)
#pragma unroll
    for (int j = 0; j < kTileC / 32; ++j) {
      const int col = (threadIdx.x >> 3) + 32 * j, piece = threadIdx.x & 7;
      const int oc = c0 + col, orow = r0 + 16 * piece;
      const v4i v = *(const lds_v4i_t*)(ttile + col * kTStride + 16 * piece);
      if (oc < cols && orow < rows) *reinterpret_cast<v4i*>(y_t + (int64_t)oc * rows + orow) = v;
    }
  }

  uint32_t a;
  if (!fold_amax(ring, T::mag_f32(amag), red, (int)gridDim.x, (int)blockIdx.x, &a)) return;
  finalize_ring<FMT>(ring, pre, a, nullptr);
}

// ---------------------------------------------------------------------------
// Dynamic recipe, pass 1: max |x| over the tensor into a length-1 ring,
// publishing scale = FMAX / amax (1 when amax is zero, infinite or NaN or the
// quotient overflows).  The quantize pass that follows applies that scale and
// folds the same amax again, which leaves the same scale and records
// scale_inv_used = 1 / scale.

template <int FMT, int IN>
__global__ __launch_bounds__(kQBlock) void amax_kernel(const v4u* __restrict__ x, int64_t nchunk,
                                                       const uint8_t* __restrict__ x_tail, int tail,
                                                       RingHeader* __restrict__ ring) {
  using T = In<IN>;
  __shared__ uint32_t red[kQBlock / 64];
  const RingPre pre = read_ring(ring);
  uint32_t amag = 0;
  auto take = [&](v4u v) __attribute__((always_inline)) {
    if constexpr (T::kBits == 16) {
      amag = max(amag, max(max(T::mag(v.x & 0xFFFFu), T::mag(v.x >> 16)), max(T::mag(v.y & 0xFFFFu), T::mag(v.y >> 16))));
      amag = max(amag, max(max(T::mag(v.z & 0xFFFFu), T::mag(v.z >> 16)), max(T::mag(v.w & 0xFFFFu), T::mag(v.w >> 16))));
    } else {
      amag = max(amag, max(max(T::mag(v.x), T::mag(v.y)), max(T::mag(v.z), T::mag(v.w))));
    }
  };
  const int64_t step = (int64_t)gridDim.x * kQBlock * kQUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kQBlock * kQUnroll + threadIdx.x; base < nchunk; base += step) {
    if (base + (kQUnroll - 1) * kQBlock < nchunk) {
      v4u v[kQUnroll];
#pragma unroll
      for (int u = 0; u < kQUnroll; ++u) v[u] = __builtin_nontemporal_load(x + base + u * kQBlock);
#pragma unroll
      for (int u = 0; u < kQUnroll; ++u) take(v[u]);
    } else {
      for (int u = 0; u < kQUnroll; ++u)
        if (base + u * kQBlock < nchunk) take(x[base + u * kQBlock]);
    }
  }
  if (tail > 0 && blockIdx.x == 0 && threadIdx.x == 0) {
    for (int i = 0; i < tail; ++i) {
      const uint32_t e = T::kBits == 16 ? reinterpret_cast<const uint16_t*>(x_tail)[i]
                                        : reinterpret_cast<const uint32_t*>(x_tail)[i];
      amag = max(amag, T::mag(e));
    }
  }
  uint32_t a;
  if (!fold_amax(ring, T::mag_f32(amag), red, (int)gridDim.x, (int)blockIdx.x, &a)) return;
  if (threadIdx.x == 0) {
    const bool bad = pre.hist_len != 1 || pre.idx != 0;
    if (bad || pre.fmt != FMT) {
      ring->status |= (bad ? kStatusBadHeader : 0u) | (pre.fmt != FMT ? kStatusFmtMismatch : 0u);
    } else {
      float s = 1.0f;
      if (a > 0u && a < 0x7F800000u) {
        const float t = FmtTraits<FMT>::kMax / __uint_as_float(a);
        if (__float_as_uint(t) < 0x7F800000u) s = t;
      }
      ring_hist(ring)[0] = __uint_as_float(a);
      ring->scale = s;
      ring->amax_last = __uint_as_float(a);
    }
    clear_top(ring);
  }
}

// ---------------------------------------------------------------------------
// Bias gradient: out[c] = sum_r g[r][c] in fp32, g bf16 / fp16 / fp32 or 8-bit
// codes dequantized as dec(code) * s_inv.  A block takes 128 columns (256
// bytes of a bf16 row: 128-byte row pieces measured 8 % slower) and a slice
// of the rows; thread t sums columns 8*(t%16) .. +7 over rows t/16,
// t/16 + 16, ... of its slice, the 16 row lanes are added in a fixed order in
// LDS, and the slice's 128 sums go to the workspace.  Consecutive blocks take
// consecutive strips of one slice, so the blocks running together read whole
// rows.  The last block of a column strip (a ticket per strip, as in the
// ring's completion tree) adds the slices in order, its loads of them issued
// sixteen at a time, so the result does not depend on timing.  Partial sums
// travel as device-scope atomic stores and loads, so they are seen across
// XCDs without writing back any cache.  The last block clears what it read
// and its ticket: the whole workspace is zero again after every call, so one
// workspace serves calls of any shape up to its size.

constexpr int kGBf16 = 0, kGF16 = 1, kGF32 = 2, kGE4M3 = 3, kGE5M2 = 4;

template <int GT>
__device__ __forceinline__ void load8(const uint8_t* row, int col, float s_inv, float (&v)[8]) {
  if constexpr (GT == kGBf16 || GT == kGF16) {
    const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(row + col * 2));
    const uint32_t e[8] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16,
                           w.z & 0xFFFFu, w.z >> 16, w.w & 0xFFFFu, w.w >> 16};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = GT == kGBf16 ? In<kInBf16>::f(e[i]) : In<kInF16>::f(e[i]);
  } else if constexpr (GT == kGF32) {
    const v4u w0 = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(row + col * 4));
    const v4u w1 = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(row + col * 4 + 16));
    const uint32_t e[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(e[i]);
  } else {
    const v2u w = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(row + col));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = (int)((i < 4 ? w.x : w.y) >> (8 * (i & 3)));
      const float d = GT == kGE4M3 ? __builtin_amdgcn_cvt_f32_fp8(c, 0) : __builtin_amdgcn_cvt_f32_bf8(c, 0);
      v[i] = d * s_inv;
    }
  }
}

constexpr int kGradCols = 128;                      // columns per strip (256 bytes of a bf16 row)
constexpr int kGradGroups = kGradCols / 8;          // 8-column groups, one per thread of a row lane
constexpr int kGradRowLanes = kQBlock / kGradGroups;

template <int GT>
__global__ __launch_bounds__(kQBlock) void bias_grad_kernel(const uint8_t* __restrict__ g, int rows, int cols,
                                                            int slices, int rows_per_slice,
                                                            const float* __restrict__ g_scale_inv, int out_f32,
                                                            void* __restrict__ out, float* __restrict__ partial,
                                                            uint32_t* __restrict__ tickets) {
  constexpr int kElem = GT == kGF32 ? 4 : (GT == kGBf16 || GT == kGF16) ? 2 : 1;
  __shared__ float sums[kGradRowLanes][kGradCols + 1];
  __shared__ int s_last;
  const int strips = (int)gridDim.x / slices, strip = blockIdx.x % strips, slice = blockIdx.x / strips;
  const int c0 = strip * kGradCols;
  const int cg = threadIdx.x % kGradGroups, rl = threadIdx.x / kGradGroups;   // 8-column group, row lane
  const int col = c0 + 8 * cg;
  const float s_inv = (GT == kGE4M3 || GT == kGE5M2) ? g_scale_inv[0] : 1.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int r_begin = slice * rows_per_slice;
  const int r_end = min(rows, r_begin + rows_per_slice);
  if (col < cols) {
    // Rows r, r + kGradRowLanes, ... added in that order; eight rows' loads
    // go out together.
    constexpr int kRowsInFlight = 8, kStep = kGradRowLanes;
    int r = r_begin + rl;
    for (; r + kStep * (kRowsInFlight - 1) < r_end; r += kStep * kRowsInFlight) {
      float v[kRowsInFlight][8];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) load8<GT>(g + (int64_t)(r + kStep * u) * cols * kElem, col, s_inv, v[u]);
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[u][i];
    }
    for (; r < r_end; r += kStep) {
      float v[8];
      load8<GT>(g + (int64_t)r * cols * kElem, col, s_inv, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sums[rl][8 * cg + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < kGradCols) {
    float s = 0.f;
    for (int j = 0; j < kGradRowLanes; ++j) s += sums[j][threadIdx.x];
    if (c0 + threadIdx.x < cols)
      __hip_atomic_store(partial + (int64_t)slice * cols + c0 + threadIdx.x, s, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(tickets + strip, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_returned(t);
    s_last = t == (uint32_t)slices - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x < kGradCols && c0 + (int)threadIdx.x < cols) {
    // The slices' sums in slice order; each group of 16 loads goes out
    // together, and every slot is cleared once all are read.
    float s = 0.f;
    float* const p0 = partial + c0 + threadIdx.x;
    for (int j0 = 0; j0 < slices; j0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        v[u] = j0 + u < slices ? __hip_atomic_load(p0 + (int64_t)(j0 + u) * cols, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (j0 + u < slices) s += v[u];
    }
    for (int j = 0; j < slices; ++j)
      __hip_atomic_store(p0 + (int64_t)j * cols, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (out_f32) static_cast<float*>(out)[c0 + threadIdx.x] = s;
    else static_cast<uint16_t*>(out)[c0 + threadIdx.x] = __builtin_bit_cast(uint16_t, (__bf16)s);
  }
  if (threadIdx.x == 0) __hip_atomic_store(tickets + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void ring_init_kernel(RingHeader* ring, int hist_len, int fmt, float init_scale) {
  float* hist = ring_hist(ring);
  for (int j = threadIdx.x; j < hist_len; j += blockDim.x) hist[j] = 0.0f;
  uint32_t* scratch = reinterpret_cast<uint32_t*>(ring_groups(ring));
  for (int j = threadIdx.x; j < kRingGroups * 16; j += blockDim.x) scratch[j] = 0u;
  if (threadIdx.x == 0) {
    ring->scale = init_scale;
    ring->scale_inv_used = 1.0f / init_scale;
    ring->amax_last = 0.0f;
    ring->idx = 0;
    ring->hist_len = hist_len;
    ring->fmt = fmt;
    ring->status = 0u;
    ring->reserved0 = 0u;
    ring->amax_bits = 0u;
    ring->ticket = 0u;
    for (int i = 0; i < 6; ++i) ring->reserved1[i] = 0u;
  }
}

typedef void (*QuantFn)(QuantJob);
typedef void (*QuantBatchFn)(QuantBatch);
typedef void (*AmaxFn)(const v4u*, int64_t, const uint8_t*, int, RingHeader*);
typedef void (*Quant2dFn)(const uint8_t*, uint8_t*, uint8_t*, int, int, int, RingHeader*);

template <int FMT>
QuantFn quant_fn(int in) {
  return in == kInBf16 ? quantize_kernel<FMT, kInBf16> : in == kInF16 ? quantize_kernel<FMT, kInF16>
                                                                       : quantize_kernel<FMT, kInF32>;
}
template <int FMT>
QuantBatchFn quant_batch_fn(int in) {
  return in == kInBf16 ? quantize_batch_kernel<FMT, kInBf16>
         : in == kInF16 ? quantize_batch_kernel<FMT, kInF16>
                        : quantize_batch_kernel<FMT, kInF32>;
}
template <int FMT>
AmaxFn amax_fn(int in) {
  return in == kInBf16 ? amax_kernel<FMT, kInBf16> : in == kInF16 ? amax_kernel<FMT, kInF16> : amax_kernel<FMT, kInF32>;
}
template <int FMT, bool DUAL>
Quant2dFn quant2d_fn(int in) {
  return in == kInBf16 ? quantize_2d_kernel<FMT, kInBf16, DUAL>
         : in == kInF16 ? quantize_2d_kernel<FMT, kInF16, DUAL>
                        : quantize_2d_kernel<FMT, kInF32, DUAL>;
}

int in_bytes(int in) { return in == kInF32 ? 4 : 2; }

// Grid of a streaming launch over numel elements of the input type.
int64_t stream_blocks(int64_t nchunk, int max_blocks) {
  const int64_t per_block = (int64_t)kQBlock * kQUnroll;
  int64_t blocks = (nchunk + per_block - 1) / per_block;
  if (blocks < 1) blocks = 1;
  if (max_blocks <= 0) max_blocks = kDefaultBlocks;
  return blocks > max_blocks ? max_blocks : blocks;
}

}  // namespace

int launch_ring_init(void* ring, int hist_len, int fmt, float init_scale, hipStream_t stream) {
  hipLaunchKernelGGL(ring_init_kernel, dim3(1), dim3(256), 0, stream, static_cast<RingHeader*>(ring), hist_len,
                     fmt, init_scale);
  return check_launch("ring_init_kernel");
}

namespace {

// The job of one tensor on a grid of at most max_blocks blocks.
QuantJob make_job(const void* x, int64_t numel, int in_type, void* ring, void* y, float* scale_inv_out,
                  int max_blocks) {
  const int per16 = 16 / in_bytes(in_type);
  QuantJob j{};
  j.nchunk = numel / per16;
  j.tail = (int)(numel % per16);
  j.blocks = (int)stream_blocks(j.nchunk, max_blocks);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* yb = static_cast<uint8_t*>(y);
  j.x = reinterpret_cast<const v4u*>(xb);
  j.y = yb;
  j.x_tail = xb + j.nchunk * 16;
  j.y_tail = yb + j.nchunk * per16;
  j.ring = static_cast<RingHeader*>(ring);
  j.scale_inv_out = scale_inv_out;
  return j;
}

}  // namespace

int launch_quantize(const void* x, int64_t numel, int in_type, int fmt, void* ring, void* y, int max_blocks,
                    hipStream_t stream) {
  const QuantJob j = make_job(x, numel, in_type, ring, y, nullptr, max_blocks);
  QuantFn fn = fmt == kE4M3 ? quant_fn<kE4M3>(in_type) : quant_fn<kE5M2>(in_type);
  hipLaunchKernelGGL(fn, dim3((unsigned)j.blocks), dim3(kQBlock), 0, stream, j);
  return check_launch("quantize_kernel");
}

int launch_quantize_batch(const fp8_quantize_job* jobs, int njobs, int in_type, int fmt, hipStream_t stream) {
  QuantBatch b{};
  int64_t total = 0, chunks = 0;
  for (int i = 0; i < njobs; ++i) {
    if (jobs[i].numel == 0) continue;
    b.job[b.njobs] = make_job(jobs[i].x, jobs[i].numel, in_type, jobs[i].ring, jobs[i].y, jobs[i].scale_inv_out, 0);
    total += b.job[b.njobs].blocks;
    chunks += b.job[b.njobs].nchunk;
    ++b.njobs;
  }
  if (b.njobs == 0) return 0;
  // Past the grid cap of a single launch, the jobs share that cap in
  // proportion to their size (two 8192^2 tensors: 512 blocks each ran 6 %
  // faster than 1024 each).
  if (total > kDefaultBlocks) {
    total = 0;
    for (int i = 0; i < b.njobs; ++i) {
      const int64_t share = (int64_t)kDefaultBlocks * b.job[i].nchunk / chunks;
      b.job[i].blocks = (int)(share < 1 ? 1 : share < b.job[i].blocks ? share : b.job[i].blocks);
      total += b.job[i].blocks;
    }
  }
  QuantBatchFn fn = fmt == kE4M3 ? quant_batch_fn<kE4M3>(in_type) : quant_batch_fn<kE5M2>(in_type);
  hipLaunchKernelGGL(fn, dim3((unsigned)total), dim3(kQBlock), 0, stream, b);
  return check_launch("quantize_batch_kernel");
}

int launch_quantize_2d(const void* x, int rows, int cols, int in_type, int fmt, bool dual, void* ring, void* y,
                       void* y_t, int max_blocks, hipStream_t stream) {
  const int tiles_c = (cols + kTileC - 1) / kTileC;
  const int64_t ntiles = (int64_t)((rows + kTileR - 1) / kTileR) * tiles_c;
  int64_t blocks = ntiles < 1 ? 1 : ntiles;
  if (max_blocks <= 0) max_blocks = k2dBlocks;
  if (blocks > max_blocks) blocks = max_blocks;
  Quant2dFn fn = fmt == kE4M3 ? (dual ? quant2d_fn<kE4M3, true>(in_type) : quant2d_fn<kE4M3, false>(in_type))
                              : (dual ? quant2d_fn<kE5M2, true>(in_type) : quant2d_fn<kE5M2, false>(in_type));
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kQBlock), 0, stream, static_cast<const uint8_t*>(x),
                     static_cast<uint8_t*>(y), static_cast<uint8_t*>(y_t), rows, cols, tiles_c,
                     static_cast<RingHeader*>(ring));
  return check_launch("quantize_2d_kernel");
}

int launch_amax(const void* x, int64_t numel, int in_type, int fmt, void* ring, hipStream_t stream) {
  const int eb = in_bytes(in_type);
  const int per16 = 16 / eb;
  const int64_t nchunk = numel / per16;
  const int tail = (int)(numel % per16);
  const int64_t blocks = stream_blocks(nchunk, 0);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  AmaxFn fn = fmt == kE4M3 ? amax_fn<kE4M3>(in_type) : amax_fn<kE5M2>(in_type);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kQBlock), 0, stream, reinterpret_cast<const v4u*>(xb), nchunk,
                     xb + nchunk * 16, tail, static_cast<RingHeader*>(ring));
  return check_launch("amax_kernel");
}

// Row slices per column strip: enough blocks to cover the CUs four times
// over, each slice at least 32 rows.  A function of the shape only, so the
// summation order (and the result) is fixed for a shape.
int bias_grad_slices(int64_t rows, int64_t cols) {
  const int64_t strips = (cols + kGradCols - 1) / kGradCols;
  int64_t s = (1024 + strips - 1) / strips;
  const int64_t max_s = (rows + 31) / 32;
  if (s > max_s) s = max_s;
  if (s > 256) s = 256;
  return (int)(s < 1 ? 1 : s);
}

// Workspace: one ticket per column strip, then the slices' partial sums.
size_t bias_grad_tickets_bytes(int64_t cols) {
  const int64_t strips = (cols + kGradCols - 1) / kGradCols;
  return ((size_t)strips * 4 + 255) & ~(size_t)255;
}

size_t bias_grad_workspace(int64_t rows, int64_t cols) {
  return bias_grad_tickets_bytes(cols) + (size_t)bias_grad_slices(rows, cols) * (size_t)cols * 4;
}

int launch_bias_grad(const void* g, int rows, int cols, int g_type, const float* g_scale_inv, int out_f32, void* out,
                     void* workspace, hipStream_t stream) {
  const int slices = bias_grad_slices(rows, cols);
  const int rps = (rows + slices - 1) / slices;
  const int strips = (cols + kGradCols - 1) / kGradCols;
  uint32_t* tickets = static_cast<uint32_t*>(workspace);
  float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + bias_grad_tickets_bytes(cols));
  typedef void (*Fn)(const uint8_t*, int, int, int, int, const float*, int, void*, float*, uint32_t*);
  const Fn fns[] = {bias_grad_kernel<kGBf16>, bias_grad_kernel<kGF16>, bias_grad_kernel<kGF32>,
                    bias_grad_kernel<kGE4M3>, bias_grad_kernel<kGE5M2>};
  hipLaunchKernelGGL(fns[g_type], dim3((unsigned)(strips * slices)), dim3(kQBlock), 0, stream,
                     static_cast<const uint8_t*>(g), rows, cols, slices, rps, g_scale_inv, out_f32, out, partial,
                     tickets);
  return check_launch("bias_grad_kernel");
}


// ---------------------------------------------------------------------------
// The bias gradient without a caller workspace, for callers that cannot
// allocate: its tickets and partial sums live in `scratch`, a device array of
// this file that every GPU the library runs on holds until the process ends.
// Host code never passes the array's name to a kernel (on the host that name
// is only a stand-in): each device's address is looked up once with
// hipGetSymbolAddress, with that device current, and kept per device.

static __device__ __align__(256) uint8_t scratch[FP8DS_BIAS_GRAD_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::atomic<bool> g_scratch_clear[kMaxDevices];

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// The current device's copy of `scratch`, or nullptr (with the error set).
void* scratch_address(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error(FP8DS_ELAUNCH, "fp8_bias_grad_noalloc: no usable current device");
    return nullptr;
  }
  *dev_out = dev;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    set_error(FP8DS_ELAUNCH, "fp8_bias_grad_noalloc: hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

int launch_bias_grad_noalloc(const void* g, int rows, int cols, int g_type, const float* g_scale_inv, int out_f32,
                             void* out, hipStream_t stream) {
  const size_t need = bias_grad_workspace(rows, cols);
  if (need > (size_t)FP8DS_BIAS_GRAD_NOALLOC_MAX_BYTES)
    return set_error(FP8DS_EUNSUPPORTED,
                     "fp8_bias_grad_noalloc: a %d x %d gradient needs %zu bytes of scratch, more than the %d the "
                     "library holds (use fp8_bias_grad with a workspace)",
                     rows, cols, need, FP8DS_BIAS_GRAD_NOALLOC_MAX_BYTES);
  int dev = 0;
  void* ws = scratch_address(&dev);
  if (!ws) return FP8DS_ELAUNCH;
  // The kernel leaves its scratch all zero after every call; the first call
  // on a device zeroes the ticket words (a fill kernel on the caller's stream,
  // so it can be captured).  While the stream is capturing, the clear goes
  // into the graph and the next call clears again.
  if (!g_scratch_clear[dev].load(std::memory_order_acquire)) {
    const int words = (int)(bias_grad_tickets_bytes(cols) / 4);
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), words);
    if (const int st = check_launch("clear_words_kernel")) return st;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
      g_scratch_clear[dev].store(true, std::memory_order_release);
  }
  return launch_bias_grad(g, rows, cols, g_type, g_scale_inv, out_f32, out, ws, stream);
}

}  // namespace fp8ds
