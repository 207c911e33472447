// Matrix-core tile code shared by the decode and prefill kernels (gfx950):
// MFMA wrappers, the per-sub-tile K/V register fragments read straight from
// the pool layout, the query fragment, and one online-softmax step over a
// 16-token sub-tile.
//
// Roles (v_mfma_f32_16x16x32_{bf16,f16}; fp32 pools: 16x16x4_f32):
//   S^T = K q^T: A = K sub-tile (16 tokens as rows), B = q (16 query columns),
//   C = 16 tokens x 16 columns, lane (c + 16 g) holding tokens 4g..4g+3 of
//   column c -- which is exactly the B-operand layout of
//   O^T += V^T P^T, so P never moves between lanes.
#pragma once

#include "pa_internal.h"

namespace pa {

constexpr int kRows = 16;           // tokens per matrix-core row tile (sub-tile)

struct TagF32 {};
struct TagF16 {};
struct TagBF16 {};
struct TagFP8 {};       // E4M3 storage, dequantized to bf16 in registers

template <class Tag> struct Is16 { static constexpr bool value = true; };
template <> struct Is16<TagF32> { static constexpr bool value = false; };

// ---- matrix-core wrappers -------------------------------------------------
template <class Tag> __device__ inline f32x4 mma32(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ inline f32x4 mma32<TagBF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ inline f32x4 mma32<TagFP8>(u32x4 a, u32x4 b, f32x4 c) {
  return mma32<TagBF16>(a, b, c);
}
template <> __device__ inline f32x4 mma32<TagF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even narrowing of p to 16 bits, and the residual.
template <class Tag> __device__ inline uint32_t narrow16(float x);
template <> __device__ inline uint32_t narrow16<TagBF16>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
template <> __device__ inline uint32_t narrow16<TagF16>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <> __device__ inline uint32_t narrow16<TagFP8>(float x) { return narrow16<TagBF16>(x); }
template <class Tag> __device__ inline float widen16(uint32_t bits);
template <> __device__ inline float widen16<TagBF16>(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}
template <> __device__ inline float widen16<TagFP8>(uint32_t bits) { return widen16<TagBF16>(bits); }
template <> __device__ inline float widen16<TagF16>(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ inline float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// ---- per-block register fragments ------------------------------------------
// 16-bit: K sub-tile [d/32][R][4][8] -> load m gives lane (t = lane%16) the
// 8 dims 8*(4m + lane/16) .. of its token (16 bytes; each instruction reads
// 1 KiB contiguous); V tile [b/4][d][4] -> load n gives lane
// (d = 16n + lane%16) the 4 tokens 4*(lane/16) .. of that dim (8 bytes; each
// instruction reads four full 128-byte lines).
template <class Tag, int D, bool H = Is16<Tag>::value> struct Frag;

// Each tile is read through its own buffer resource (base = tile address,
// size = tile bytes); a resource of size 0 makes every lane's access out of
// range, which returns zeros without touching memory -- the one-block-ahead
// prefetch uses that past a wavefront's last block, so its wait counts stay
// static without a spare read of real data.  Decode reads each tile once per
// call: streaming (non-temporal) loads; prefill re-reads tiles across query
// tiles: ordinary cached loads.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;         // raw (untyped) buffer, gfx9 family
#ifndef PA_TEMPORAL_KV
#define PA_TEMPORAL_KV 0
#endif
constexpr int kPolicyCached = 0;
constexpr int kPolicyStream = 2;               // nt
constexpr int kKvCachePolicy = PA_TEMPORAL_KV ? kPolicyCached : kPolicyStream;

__device__ inline rsrc_t tile_rsrc(const char* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, bytes, kRsrcWord3);
}
template <int Pol = kKvCachePolicy> __device__ inline u32x4 buf_load16(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, Pol);
}
template <int Pol = kKvCachePolicy> __device__ inline u32x2 buf_load8(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, Pol);
}
template <int Pol = kKvCachePolicy> __device__ inline uint32_t buf_load4(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, Pol);
}

// Two E4M3 codes (bytes 2*hi, 2*hi+1 of w) -> two bf16 (exact: every E4M3
// value is a bf16 value).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <bool Hi> __device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, Hi));
}

template <class Tag, int D> struct Frag<Tag, D, true> {
  static constexpr int NK = D / 32;
  static constexpr int NV = D / 16;
  u32x4 k[NK];
  u32x2 v[NV];
  template <int Pol = kKvCachePolicy>
  __device__ inline void load(rsrc_t rk, rsrc_t rv, int lane, int rows = kRows) {
    const int kr = (lane & 15) * 64 + (lane >> 4) * 16;
#pragma unroll
    for (int m = 0; m < NK; ++m) k[m] = buf_load16<Pol>(rk, kr + m * rows * 64);
    const int vr = (lane >> 4) * (D * 8) + (lane & 15) * 8;
#pragma unroll
    for (int n = 0; n < NV; ++n) v[n] = buf_load8<Pol>(rv, vr + n * 128);
  }
};

// FP8 storage.  The memory system here is bound by requests (cache-line
// pieces per instruction), not bytes, so the FP8 tile layout makes every
// load instruction cover whole 128-byte lines, and the lane roles permute
// dimensions to match (a dot product and an output row do not care about
// the order of dimensions).  Per sub-tile of R rows (R = min(b, 16)):
//   K: [g < 4][h < D/64][t < R][16 bytes]: lane (t, g) holds dims
//      g*D/4 .. g*D/4 + D/4 - 1 of row t, 16 per load; k-step m of the
//      score product uses dims g*D/4 + 8m .. +7 (the q fragment matches);
//   V: [tg < R/4][h < D/64][r < 16][4 dims][4 tokens]: lane (r, tg) holds
//      dims r*D/16 .. +D/16 - 1 of tokens 4tg .. 4tg+3; dim tile n of the
//      P.V product is dim r*D/16 + n of row r (outputs permuted alike).
// Rows past R read past the sub-tile's resource (zeros) or alias other rows;
// either way they are masked.  Codes are converted to the bf16 registers of
// Frag<TagBF16> just before use.
template <int D> struct Frag<TagFP8, D, true> {
  u32x2 k[D / 32];
  uint32_t v[D / 16];
  template <int Pol = kKvCachePolicy>
  __device__ inline void load(rsrc_t rk, rsrc_t rv, int lane, int rows = kRows) {
    const int t = lane & 15, g = lane >> 4;
    const int kb = g * (rows * D / 4) + t * 16;
    const int vb = g * (4 * D) + t * 16;
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
      const u32x4 a = buf_load16<Pol>(rk, kb + h * rows * 16);
      k[2 * h] = u32x2{a[0], a[1]};
      k[2 * h + 1] = u32x2{a[2], a[3]};
      const u32x4 b = buf_load16<Pol>(rv, vb + h * 256);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * h + e] = b[e];
    }
  }
  __device__ inline Frag<TagBF16, D, true> bf16() const {
    Frag<TagBF16, D, true> f;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
      f.k[m] = u32x4{fp8x2_to_bf16x2<false>(k[m][0]), fp8x2_to_bf16x2<true>(k[m][0]),
                     fp8x2_to_bf16x2<false>(k[m][1]), fp8x2_to_bf16x2<true>(k[m][1])};
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
      f.v[n] = u32x2{fp8x2_to_bf16x2<false>(v[n]), fp8x2_to_bf16x2<true>(v[n])};
    return f;
  }
};

// The tag the matrix-core code runs in, and the registers it reads: FP8
// fragments convert to bf16 ones, the others are used as loaded.
template <class Tag> struct ComputeTag { using type = Tag; };
template <> struct ComputeTag<TagFP8> { using type = TagBF16; };
template <class Tag> struct IsFP8 { static constexpr bool value = false; };
template <> struct IsFP8<TagFP8> { static constexpr bool value = true; };
template <class Tag, int D> __device__ inline Frag<Tag, D> compute_regs(const Frag<Tag, D>& f) {
  return f;
}
template <int D> __device__ inline Frag<TagBF16, D> compute_regs(const Frag<TagFP8, D>& f) {
  return f.bf16();
}

// fp32: K tile [16][d] -> load j gives lane (t = lane%16) dims
// 4*(4j + lane/16) ..; V tile [16/4][d][4] -> load n gives lane
// (d = 16n + lane%16) the 4 tokens 4*(lane/16) ...
template <class Tag, int D> struct Frag<Tag, D, false> {
  static constexpr int NK = D / 16;
  static constexpr int NV = D / 16;
  f32x4 k[NK];
  f32x4 v[NV];
  template <int Pol = kKvCachePolicy>
  __device__ inline void load(rsrc_t rk, rsrc_t rv, int lane, int = kRows) {
    const int kr = (lane & 15) * (D * 4) + (lane >> 4) * 16;
#pragma unroll
    for (int j = 0; j < NK; ++j) k[j] = __builtin_bit_cast(f32x4, buf_load16<Pol>(rk, kr + j * 64));
    const int vr = (lane >> 4) * (D * 16) + (lane & 15) * 16;
#pragma unroll
    for (int n = 0; n < NV; ++n) v[n] = __builtin_bit_cast(f32x4, buf_load16<Pol>(rv, vr + n * 256));
  }
};

// Query fragment: the B operand of S = K q^T for head (lane % 16) of the group.
template <class Tag, int D, bool H = Is16<Tag>::value> struct QFrag;
template <class Tag, int D> struct QFrag<Tag, D, true> {
  u32x4 q[D / 32];
  __device__ inline void load(const char* qrow, bool valid, int lane) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const int dim0 = 8 * (4 * m + (lane >> 4));
      q[m] = valid ? *reinterpret_cast<const u32x4*>(qrow + dim0 * 2) : u32x4{0, 0, 0, 0};
    }
  }
};
// FP8: k-step m of lane group g uses dims g*D/4 + 8m .. +7 (the K layout above).
template <int D> struct QFrag<TagFP8, D, true> : QFrag<TagBF16, D, true> {
  __device__ inline void load(const char* qrow, bool valid, int lane) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const int dim0 = (lane >> 4) * (D / 4) + 8 * m;
      this->q[m] = valid ? *reinterpret_cast<const u32x4*>(qrow + dim0 * 2) : u32x4{0, 0, 0, 0};
    }
  }
};
template <class Tag, int D> struct QFrag<Tag, D, false> {
  f32x4 q[D / 16];
  __device__ inline void load(const char* qrow, bool valid, int lane) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const int dim0 = 4 * (4 * j + (lane >> 4));
      q[j] = valid ? *reinterpret_cast<const f32x4*>(qrow + dim0 * 4) : f32x4{0, 0, 0, 0};
    }
  }
};

// Running softmax state of one wavefront: lane (h + 16 q) owns head h;
// acc[n][r] is output dim 16n + 4q + r of that head (the MFMA C layout).
template <int D> struct State {
  float m;      // exponent base of l and acc (log2 domain), identical across
                // the head's lanes: the running max, moved only when a score
                // exceeds it by more than kRescaleLog2
  float l;      // this lane's share of the running sum
  f32x4 acc[D / 16];
};

// Scores may exceed the exponent base by up to this much (p <= 2^8) before
// the base moves; exp2(s - m) then never overflows and the softmax is the
// same for any base.
constexpr float kRescaleLog2 = 8.f;

// One sub-tile: S = K q^T, online-softmax update of (m, l), acc += V^T P.
// n_valid: stored tokens in the sub-tile (rows past it may hold anything).
// A column may see none of the sub-tile's rows while its state is still
// empty (m = -inf, e.g. under a causal limit); its exponent base then falls
// back to 0 so that -inf - -inf never occurs.  `qk()` returns the scores,
// lane (h + 16q) holding tokens 4q..4q+3 of head h; `pv(p, t0)` adds
// V^T P for this lane's four probabilities p of tokens t0 .. t0 + 3.
template <int D, bool SkipWhole = false, class QK, class PV>
__device__ inline void attend_core(QK qk, PV pv, State<D>& st, int n_valid, float qk_scale,
                                   int lane, int lim) {
  f32x4 s = qk();
  const int t0 = 4 * (lane >> 4);
  // select, never multiply: tails may hold NaN.  `lim` (per lane: its
  // column's last visible row + 1) is the causal limit of multi-token queries.
  // With SkipWhole, a sub-tile with every row stored and no causal limit
  // (nearly every one in decode) skips the selects behind a uniform branch;
  // the 16-bit kernels keep the unconditional form (the branch costs them
  // registers they do not have).
  const bool masked = !SkipWhole || n_valid < kRows || lim < kRows;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] *= qk_scale;
    if (masked && (t0 + r >= n_valid || t0 + r >= lim)) s[r] = -INFINITY;
  }
  // Online softmax with a lazily moved base: only when some score of the
  // wavefront exceeds its column's base by more than kRescaleLog2 (always on
  // the first sub-tile, where m = -inf) does the wavefront take the column
  // maxima across lanes and rescale l and acc -- a uniform branch; otherwise
  // both are skipped.
  bool over = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) over |= s[r] > st.m + kRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(over) != 0) {
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = xor_max(bm);
    const float m_new = fmaxf(st.m, bm);
    const float alpha = fast_exp2(st.m - (m_new == -INFINITY ? 0.f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) st.acc[n] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == -INFINITY ? 0.f : st.m;
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] - base);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  pv(p, t0);
}

// The 16-bit matrix-core step over K chunks and V dim tiles read through
// `kf(m)` and `vf(n)` (registers, or FP8 codes widened at the point of use).
// acc[d][h] += V^T P with P split into a high and a low part placed in the two
// k halves against a duplicated V fragment.  Tail tokens of V are zeroed
// (their P is zero, but 0 * NaN is NaN).
template <class Tag, int D, bool SkipWhole = false, class KF, class VF>
__device__ inline void attend16(KF kf, VF vf, const QFrag<Tag, D>& qf, State<D>& st, int n_valid,
                                float qk_scale, int lane, int lim = kRows) {
  auto qk = [&]() {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m) s = mma32<Tag>(kf(m), qf.q[m], s);
    return s;
  };
  auto pv = [&](const float* p, int t0) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[r] = narrow16<Tag>(p[r]);
      lo[r] = narrow16<Tag>(p[r] - widen16<Tag>(hi[r]));
    }
    const u32x4 pb = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                      lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    uint32_t keep0 = 0xffffffffu, keep1 = 0xffffffffu;
    if (n_valid < kRows) {
      keep0 = (t0 + 0 < n_valid ? 0x0000ffffu : 0u) | (t0 + 1 < n_valid ? 0xffff0000u : 0u);
      keep1 = (t0 + 2 < n_valid ? 0x0000ffffu : 0u) | (t0 + 3 < n_valid ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const u32x2 v = vf(n);
      const uint32_t a0 = v[0] & keep0, a1 = v[1] & keep1;
      const u32x4 va = {a0, a1, a0, a1};
      st.acc[n] = mma32<Tag>(va, pb, st.acc[n]);
    }
  };
  attend_core<D, SkipWhole>(qk, pv, st, n_valid, qk_scale, lane, lim);
}

template <class Tag, int D>
__device__ inline void attend_block(const Frag<Tag, D>& f, const QFrag<Tag, D>& qf, State<D>& st,
                                    int n_valid, float qk_scale, int lane, int lim = kRows) {
  if constexpr (Is16<Tag>::value) {
    attend16<Tag, D>([&](int m) { return f.k[m]; }, [&](int n) { return f.v[n]; }, qf, st,
                     n_valid, qk_scale, lane, lim);
  } else {
    // fp32: v_mfma_f32_16x16x4_f32, one k per lane.
    auto qk = [&]() {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 16; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = mma4(f.k[j][e], qf.q[j][e], s);
      return s;
    };
    auto pv = [&](const float* p, int t0) {
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
        f32x4 va = f.v[n];
        if (n_valid < kRows) {
#pragma unroll
          for (int e = 0; e < 4; ++e) va[e] = (t0 + e < n_valid) ? va[e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) st.acc[n] = mma4(va[e], p[e], st.acc[n]);
      }
    };
    attend_core<D>(qk, pv, st, n_valid, qk_scale, lane, lim);
  }
}

// FP8 codes: the same step with each K chunk and V dim tile widened to bf16
// just before its matrix product, so only that chunk's widened registers are
// live (the raw codes are half the registers of the widened fragment).
template <int D>
__device__ inline void attend_block_fp8(const Frag<TagFP8, D>& f, const QFrag<TagFP8, D>& qf,
                                        State<D>& st, int n_valid, float qk_scale, int lane) {
  attend16<TagBF16, D, true>(
      [&](int m) {
        return u32x4{fp8x2_to_bf16x2<false>(f.k[m][0]), fp8x2_to_bf16x2<true>(f.k[m][0]),
                     fp8x2_to_bf16x2<false>(f.k[m][1]), fp8x2_to_bf16x2<true>(f.k[m][1])};
      },
      [&](int n) { return u32x2{fp8x2_to_bf16x2<false>(f.v[n]), fp8x2_to_bf16x2<true>(f.v[n])}; },
      qf, st, n_valid, qk_scale, lane);
}

// Output dimension of accumulator element acc[n][i] (the MFMA C layout puts
// row 4*(lane/16) + i of dim tile n in this lane): 16n + row, or for FP8
// storage row*D/16 + n (the V layout's permutation).
template <class Tag, int D> __device__ inline int out_dim(int n, int i, int lane) {
  const int row = 4 * (lane >> 4) + i;
  return IsFP8<Tag>::value ? row * (D / 16) + n : 16 * n + row;
}

template <class OutT> __device__ inline void store_out(OutT* o, float x);
template <> __device__ inline void store_out<float>(float* o, float x) { *o = x; }
template <> __device__ inline void store_out<__bf16>(__bf16* o, float x) { *o = static_cast<__bf16>(x); }
template <> __device__ inline void store_out<_Float16>(_Float16* o, float x) { *o = static_cast<_Float16>(x); }

// Bytes per stored element (Elt) and per input element -- q, k_new, v_new --
// (In): bf16 inputs for FP8 storage.
template <class Tag> struct Elt { using T = uint16_t; static constexpr int bytes = 2; };
template <> struct Elt<TagF32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elt<TagFP8> { using T = uint8_t; static constexpr int bytes = 1; };
template <class Tag> struct In { static constexpr int bytes = Is16<Tag>::value ? 2 : 4; };


}  // namespace pa
