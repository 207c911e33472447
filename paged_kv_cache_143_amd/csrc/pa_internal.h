// Internal helpers shared by the libpa HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kWave = 64;         // CDNA wavefront width

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Bytes per stored element, and per element of the 16-bit-or-wider inputs
// (k_new, v_new, q): bf16 for FP8 pools.
inline int elem_bytes(pa_dtype t) { return t == PA_F32 ? 4 : t == PA_FP8_E4M3 ? 1 : 2; }
inline int input_bytes(pa_dtype t) { return t == PA_F32 ? 4 : 2; }

inline bool dtype_ok(pa_dtype t) {
  return t == PA_F32 || t == PA_F16 || t == PA_BF16 || t == PA_FP8_E4M3;
}

// Host-side validation of a pool descriptor.  Returns PA_OK or the status.
inline pa_status check_pool(const pa_pool_desc* p) {
  if (!p) return PA_ERR_INVALID_ARG;
  if (p->num_blocks < 1 || p->block_size < 1 || p->num_kv_heads < 1 || p->head_dim < 1)
    return PA_ERR_INVALID_ARG;
  if (!dtype_ok(p->dtype)) return PA_ERR_UNSUPPORTED;
  if (p->dtype == PA_FP8_E4M3 && (!p->k_scales || !p->v_scales)) return PA_ERR_INVALID_ARG;
  if (p->block_size != 8 && p->block_size != 16 && p->block_size != 32) return PA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return PA_ERR_UNSUPPORTED;
  // Flat slot indices are int32.
  if ((int64_t)p->num_blocks * p->block_size > INT32_MAX) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Elements in one (block, KV head) tile and in one block across heads.
inline int64_t tile_elems(const pa_pool_desc* p) { return (int64_t)p->block_size * p->head_dim; }

inline pa_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// E4M3 code of x / scale: the quotient in fp32 (IEEE division), clamped to
// +-448 so that the conversion cannot overflow, rounded to nearest even by
// the hardware conversion; NaN gives 0x7F.
__device__ inline uint32_t fp8_code(float x, float scale) {
  float y = x / scale;
  if (y != y) return 0x7Fu;
  y = y > 448.f ? 448.f : (y < -448.f ? -448.f : y);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFFu;
}
__device__ inline float bf16_bits_to_float(uint32_t b16) { return __builtin_bit_cast(float, b16 << 16); }

// Byte offset of K elements d .. d+7 (d a multiple of 8) of token t inside one
// 16-bit (block, KV head) tile of b tokens and D dims: sub-tiles of
// R = min(b, 16) tokens, each [D/32][R][4][8 elements] -- a matrix-core load
// of 16 rows then reads 1 KiB contiguous.
__device__ inline int k16_offset(int t, int d, int b, int D) {
  const int R = b < 16 ? b : 16;
  const int s = t / R, tl = t - s * R;
  return (s * R * D + (d >> 5) * (R * 32) + tl * 32 + (d & 31)) * 2;
}

// Byte offsets of (token t, dim d) inside one FP8 (block, KV head) tile of b
// tokens and D dims: sub-tiles of R = min(b, 16) tokens, each
//   K: [g < 4][h < D/64][row < R][16 bytes], dim d = g*D/4 + 16h + byte;
//   V: [tg < R/4][h < D/64][r < 16][4 dims][4 tokens], dim d = r*D/16 + 4h + e.
__device__ inline int fp8_k_offset(int t, int d, int b, int D) {
  const int R = b < 16 ? b : 16;
  const int s = t / R, tl = t - s * R;
  const int g = d / (D / 4), w = d - g * (D / 4);
  return s * R * D + g * (R * D / 4) + (w >> 4) * (R * 16) + tl * 16 + (w & 15);
}
__device__ inline int fp8_v_offset(int t, int d, int b, int D) {
  const int R = b < 16 ? b : 16;
  const int s = t / R, tl = t - s * R;
  const int r = d / (D / 16), w = d - r * (D / 16);
  return s * R * D + (tl >> 2) * (4 * D) + (w >> 2) * 256 + r * 16 + (w & 3) * 4 + (tl & 3);
}

}  // namespace pa
