// Device-side definitions shared by the quantize and GEMM kernels of libfp8ds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8ds {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v2i lds_v2i_t;
typedef __attribute__((address_space(3))) v4i lds_v4i_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

// Quantize input element types (fp8ds_in_type).
constexpr int kInBf16 = 0;
constexpr int kInF16 = 1;
constexpr int kInF32 = 2;

// Byte layout of the scale ring (documented in include/fp8ds.h).
struct RingHeader {
  float scale;
  float scale_inv_used;
  float amax_last;
  int32_t idx;
  int32_t hist_len;
  int32_t fmt;
  uint32_t status;
  uint32_t reserved0;
  uint32_t amax_bits;
  uint32_t ticket;
  uint32_t reserved1[6];
};
static_assert(sizeof(RingHeader) == 64, "ring header is 64 bytes");

// Completion-tree scratch of the ring: one 64-byte line per block group, so
// the per-block atomics of a quantize launch spread over kRingGroups lines
// instead of queueing on one address.  Zero between calls.
constexpr int kRingGroups = 32;
struct RingGroup {
  uint32_t amax_bits;
  uint32_t ticket;
  uint32_t pad[14];
};
static_assert(sizeof(RingGroup) == 64, "one group per 64-byte line");
constexpr int kRingHistOffset = 64 + kRingGroups * 64;   // 2112

__device__ __forceinline__ RingGroup* ring_groups(RingHeader* r) { return reinterpret_cast<RingGroup*>(r + 1); }
__device__ __forceinline__ float* ring_hist(RingHeader* r) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(r) + kRingHistOffset);
}

constexpr uint32_t kStatusFmtMismatch = 1u;
constexpr uint32_t kStatusBadHeader = 2u;

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<kE4M3> {
  static constexpr float kMax = 448.0f;       // 1.75 * 2^8
  static constexpr uint32_t kMaxCode = 0x7E;
};
template <>
struct FmtTraits<kE5M2> {
  static constexpr float kMax = 57344.0f;     // 1.75 * 2^15
  static constexpr uint32_t kMaxCode = 0x7B;
};

// Raw buffer resource over `bytes` bytes from `base`; loads at offsets at or
// beyond `bytes` return zero (the word-3 constant selects 32-bit raw access).
// Both arguments must be uniform across the wave: they are moved to scalar
// registers explicitly, so the descriptor never needs a per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// The four words of a raw buffer descriptor in scalar registers, for the
// inline-asm LDS loads below (base, stride 0, size in bytes, 32-bit raw format).
__device__ __forceinline__ v4i rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return v4i{(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
             (int)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xFFFFu),
             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// One buffer_load_dwordx4 ... lds: each lane's 16 bytes at byte soff + voff
// of the buffer land at LDS byte lds_base + 16 * lane (lds_base and soff
// wave-uniform).  Callers keep soff + voff below 2^32 and the buffer size at
// least soff + voff for every load meant to read memory; a load whose voff is
// at or past the buffer size lands as zeros.  Written as inline asm so the
// compiler does not guard every later LDS read with a wait for all
// outstanding loads: callers count these loads themselves (vmcnt) and order
// LDS through barriers.  The instruction writes no VGPR.
__device__ __forceinline__ void load_lds16(v4i rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
#pragma clang diagnostic pop
}

__device__ __forceinline__ uint32_t lds_address(const lds_char_t* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

}  // namespace fp8ds
