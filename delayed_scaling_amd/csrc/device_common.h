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
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace fp8ds
