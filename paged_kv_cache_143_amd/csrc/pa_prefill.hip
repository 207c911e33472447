// Multi-token (prefill and chunked-prefill) paged attention for gfx950 (MI355X).
//
// What it computes: sequence i holds L_i tokens in the pool; its chunk is the
// n_i newest of them (positions L_i - n_i .. L_i - 1, K/V already written).
// Chunk row t (position p = L_i - n_i + t), query head h, KV head g = h / G:
//     out[t][h] = sum_{k <= p} softmax_k(scale * q[t][h] . K_i[k][g]) V_i[k][g],
// K_i[k] read through block table i as in decode.  In prefill every prompt
// token is known at once, so the work is a dense matrix product
// ("vLLM and PagedAttention: Virtual Memory for LLM Serving", paragraph 1);
// long prompts are processed in chunks whose older tokens are already cached
// ("Inside vLLM and TGI: Paging, Versioned Schedulers and Operations",
// sections "Read the vLLM0.11.0 scheduler" and "Observability and debugging
// runbook").  The pages give no formula; this is causal scaled dot-product
// attention read through the table.
//
// Work decomposition.  A column is one (chunk row, query head of group g)
// pair; a 16-column group packs floor(16 / G) consecutive rows times the G
// heads of the group.  A wavefront owns NQ column groups and walks the
// sequence's keys from position 0 up to its last row's position: S^T = K q^T
// on the matrix cores, a causal mask per column, online softmax, O^T += V^T
// P^T with P split into high and low bf16 halves (bf16 pools) or rounded once
// to fp16 (fp16 and FP8 pools).  Each K/V fragment serves
// NQ groups; the four wavefronts of a workgroup take consecutive row ranges of
// one (sequence, KV head).
//
// 16-bit and FP8 pools (prefill_ring_kernel): the four wavefronts walk together in
// steps of 32 keys.  Each step's K and V are copied once per workgroup from
// the pool into a four-stage LDS ring (FP8: three) by global-to-LDS loads
// issued ahead (the loading lanes gather the rows through the block table),
// and every wavefront reads its fragments from LDS, the next step's K while
// the current step's softmax runs.  Table entries come in
// windows of 64 blocks, one per lane, and reach the loading lanes by lane
// permutation; FP8 codes land raw and are widened in LDS once per workgroup,
// K to bf16 and V to fp16.  fp32 pools (prefill_kernel): each wavefront walks on
// its own, one sub-tile per step with a second buffer one step ahead, through
// cached buffer loads.  Each XCD runs the row tiles of one (sequence, KV head)
// after another, last rows (the most keys) first, so its resident workgroups
// share K/V in its L2.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "pa_tile.h"

namespace pa {

// ---- two sub-tiles per step (multi-token queries, 16-bit storage) ----------
// 32 keys per step: the P.V product's k dimension holds 4 tokens of each
// sub-tile per lane group (k slots 0..3: sub-tile a, 4..7: sub-tile b), so
// the V operand is two 8-byte loads side by side -- no duplicated V -- and
// with bf16 V the high and low parts of P are two products with the same V.  The
// masks for stored-length tails and causal limits run only on partial
// steps; P is narrowed two values per conversion.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <class Tag> __device__ inline uint32_t pack2(f32x2 x);
template <> __device__ inline uint32_t pack2<TagBF16>(f32x2 x) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
template <> __device__ inline uint32_t pack2<TagF16>(f32x2 x) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}
// Two E4M3 codes (bytes 2*hi, 2*hi+1 of w) -> two fp16 (exact: E4M3's 3
// mantissa bits and exponents 2^-9 .. 2^8 lie inside fp16's).
template <bool Hi> __device__ inline uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, Hi));
}
template <class Tag> __device__ inline f32x2 unpack2(uint32_t w);
template <> __device__ inline f32x2 unpack2<TagBF16>(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(bf16x2, w), f32x2);
}
template <> __device__ inline f32x2 unpack2<TagF16>(uint32_t w) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

// K and V fragments of one step (two 16-row tiles a and b), read from LDS.
template <class Tag, int D> struct FragPair {
  u32x4 k[2][D / 32];     // K of tiles a and b (the Frag<Tag> lane roles)
  u32x4 v[D / 16];        // dim tile n: .xy = tile a's 4 tokens, .zw = b's
};

// S^T of the step's two tiles for one column group.
template <class Tag, int D>
__device__ inline void qk_pair(const FragPair<Tag, D>& f, const QFrag<Tag, D>& qf, f32x4& sa,
                               f32x4& sb) {
  sa = f32x4{0.f, 0.f, 0.f, 0.f};
  sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    sa = mma32<Tag>(f.k[0][m], qf.q[m], sa);
    sb = mma32<Tag>(f.k[1][m], qf.q[m], sb);
  }
}

// Online softmax of one column group over one step, in stages that let the
// scheduler overlap one group's (or step's) vector work with matrix
// products of another.  c = scale * log2(e).
//
// mask_scores: scores of invalid keys (bit k of `valid` clear: a tail past L
// or a block outside the pool) or of keys past the column's causal limit
// become -inf * sign(c), so that c * s = -inf (a select: such rows may hold
// NaN).  lima: per lane, the column's causal limit in rows of tile a (tile
// b's is lima - 16).
template <int D>
__device__ inline void mask_scores(f32x4& sa, f32x4& sb, uint32_t valid, float c, int lane, int lima) {
  const float ninf = c >= 0.f ? -INFINITY : INFINITY;
  const int t0 = 4 * (lane >> 4);
  const uint32_t ma = valid >> t0, mb = valid >> (16 + t0);
  const int limb = lima - kRows;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sa[r] = ((ma >> r) & 1u) && t0 + r < lima ? sa[r] : ninf;
    sb[r] = ((mb >> r) & 1u) && t0 + r < limb ? sb[r] : ninf;
  }
}

// p = exp2(c s - base) against the column's current base (0 while it has
// none) and their sum; returns whether the column needs the exact path: the
// sum exceeds 2^8 (every p > 2^8 is caught, since p >= 0; now and then a
// step whose p are all below that moves the base too, which is harmless) or
// no base yet.
template <int D>
__device__ inline bool take_exps(f32x4 sa, f32x4 sb, const State<D>& st, float c, float* p, float& sum) {
  const float base = st.m == -INFINITY ? 0.f : st.m;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = fast_exp2(__builtin_fmaf(sa[r], c, -base));
    p[4 + r] = fast_exp2(__builtin_fmaf(sb[r], c, -base));
  }
  sum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  return !(sum <= 256.f) || st.m == -INFINITY;
}

// The exact path (rare): move the base to the running maximum, rescale l and
// acc, and take the exponentials again -- the same softmax for any base.
template <int D>
__device__ inline void rebase(f32x4 sa, f32x4 sb, State<D>& st, float c, float* p, float& sum) {
  float bm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) bm = fmaxf(bm, fmaxf(sa[r] * c, sb[r] * c));
  bm = xor_max(bm);
  const float m_new = fmaxf(st.m, bm);
  const float alpha = fast_exp2(st.m - (m_new == -INFINITY ? 0.f : m_new));
  st.l *= alpha;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) st.acc[n] *= alpha;
  st.m = m_new;
  take_exps<D>(sa, sb, st, c, p, sum);
}

// l += sum p; acc += V^T P^T.  bf16: P split into high and low 16-bit parts
// (two products with the same V fragment; one bf16 rounding of P, 2^-9
// relative, measures 2.4e-3 row error on N(0,1) data, above the 2e-3 bar).
// fp16 (fp16 pools, and FP8 pools whose V codes widen to fp16 exactly): one
// product with P rounded to fp16 (2^-11 relative, p <= 2^8 well inside its
// range), which keeps the result within the bar on its own.  V
// rows of invalid keys must be zero (their p is 0, but 0 * NaN is NaN).
template <class Tag> struct SplitP { static constexpr bool value = true; };
template <> struct SplitP<TagF16> { static constexpr bool value = false; };

// The two halves of a step's P.V: narrow_p (l += sum p, P narrowed to the
// product's 16-bit type) runs while the step's LDS reads are in flight,
// pv_products (acc += V^T P^T) after them.
struct PPack {
  u32x4 hi, lo;
};
// The low part of bf16 P, p - hi (exact), one packed bf16 dot product per
// value: hi . (-1, 0) + p0 and hi . (0, -1) + p1.  The pairs come in scalar
// registers (neg.x = 0x0000bf80, neg.y = 0xbf800000): as an immediate the
// compiler encodes (-1, 0) as the inline constant -1.0, which the hardware
// does not read as that pair.
__device__ inline f32x2 minus_hi(uint32_t hi, f32x2 p, uint2 neg) {
  const bf16x2 h = __builtin_bit_cast(bf16x2, hi);
  return f32x2{__builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, neg.x), p[0], false),
               __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, neg.y), p[1], false)};
}
template <class Tag, int D>
__device__ inline PPack narrow_p(const float* p, float sum, State<D>& st, uint2 neg) {
  st.l += sum;
  PPack pk;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 pw = {p[2 * w], p[2 * w + 1]};
    pk.hi[w] = pack2<Tag>(pw);
    if constexpr (SplitP<Tag>::value) pk.lo[w] = pack2<Tag>(minus_hi(pk.hi[w], pw, neg));
  }
  return pk;
}
template <class Tag, class FTag, int D>
__device__ inline void pv_products(const FragPair<FTag, D>& f, const PPack& pk, State<D>& st) {
#pragma unroll
  for (int n = 0; n < D / 16; ++n) st.acc[n] = mma32<Tag>(f.v[n], pk.hi, st.acc[n]);
  if constexpr (SplitP<Tag>::value) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) st.acc[n] = mma32<Tag>(f.v[n], pk.lo, st.acc[n]);
  }
}

constexpr int kPWaves = 4;
constexpr int kPThreads = kWave * kPWaves;
constexpr int kXcds = 8;     // accelerator complex dies of one MI355X

#ifndef PA_PREFILL_NQ
#define PA_PREFILL_NQ 2
#endif
constexpr int kNQ = PA_PREFILL_NQ;

struct PrefillArgs {
  const char* k_pool;
  const char* v_pool;
  const char* q;             // [T][Hq][D]
  void* out;                 // [T][Hq][D]
  const int32_t* q_start;    // [S + 1]: first row of each sequence's chunk
  const int32_t* tables;
  const int32_t* lens;
  int32_t num_blocks;
  int32_t block_size;
  int32_t rows;              // tokens per sub-tile: min(block_size, 16)
  int32_t sub;               // sub-tiles per block
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t group;             // G
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t max_len;
  int32_t tpg;               // chunk rows per 16-column group: 16 / G
  int32_t wave_rows;         // NQ * tpg
  int32_t num_tiles;         // row tiles of kPWaves * wave_rows per sequence
  float qk_scale;            // scale * log2(e)
  const float* k_scales;     // FP8 pools: per-KV-head scales, else null
  const float* v_scales;
};

// ---- 16-bit pools: steps staged in an LDS ring ------------------------------
// A step is 32 consecutive key positions 32j .. 32j + 31: two 16-row tiles
// (a: rows 0-15, b: rows 16-31), taken as four 8-row quarters, each inside
// one block (8 divides the block size).  The four wavefronts of a workgroup
// copy a step's K and V from the pool into one stage of a four-stage LDS ring
// with global-to-LDS loads (1 KiB per instruction, no registers), three steps
// ahead of the computation; every wavefront then reads its fragments from
// LDS, so a tile leaves L2 once per workgroup rather than once per wavefront.
//
// Stage layout (16-bit elements; one 1-KiB chunk per load instruction):
//   K chunk (h, m), m < D/32: [lane][16 B] = row lane % 16 of tile h, dims
//     32m + 8 (lane / 16) .. +7 -- lane's A fragment, one ds_read_b128;
//   V chunk n < D/16: [h][lane][8 B] = tokens 4 (lane / 16) .. +3 of tile h
//     at dim 16n + lane % 16 -- both tiles' B halves, one ds_read2st64_b64.
// The loading lanes gather these from the pool layout (include/pa.h): K
// sub-tile [d/32][R][32] and V sub-tile [R/4][d][4], R = min(b, 16).
#ifndef PA_RING_STAGES
#define PA_RING_STAGES 4
#endif
template <class Tag, int D> struct Ring {
  static constexpr bool kF8 = IsFP8<Tag>::value;
  static constexpr int kChunks = D / 32;                  // 16-bit K chunks per tile
  static constexpr int kKBytes = 2 * kChunks * 1024;      // 16-bit layout: K of both tiles
  static constexpr int kStep = kKBytes + (D / 16) * 1024; // 16-bit layout: one step
  // FP8: the loads land raw codes (half the bytes) in stages of kRawStep,
  // converted to the 16-bit layout in slots of kStep; three of each.
  static constexpr int kRawChunks = D / 64;               // FP8 pieces per tile, K or V
  static constexpr int kRawStep = kStep / 2;
  static constexpr int kStages = kF8 ? 3 : PA_RING_STAGES;
  // Steps loaded ahead.  FP8: 4, and a step's codes are widened into their
  // slot two steps before its scores (during the softmax of step j - 2),
  // three raw stages (j + 2 .. j + 4) and three slots (j .. j + 2).
  static constexpr int kAhead = kF8 ? 4 : kStages - 1;
  static constexpr int kRawBase = kStages * kStep;          // FP8 raw stages after the slots
  static constexpr int kBytes = kStages * kStep + (kF8 ? kStages * kRawStep : 0);
  static constexpr int kPerWave = (kF8 ? kRawStep : kStep) / 1024 / kPWaves;  // loads per step
  static_assert(kPerWave == (kF8 ? kRawChunks : kChunks), "waves 0-1 load K, waves 2-3 load V");
};

typedef const __attribute__((address_space(1))) char* gchar;
typedef __attribute__((address_space(3))) char* lchar;
typedef const __attribute__((address_space(4))) int32_t* cint;

// LDS reads are written as instructions of their own: the compiler cannot
// tell the ring's stages apart and would otherwise wait for every
// outstanding global-to-LDS load before each read.  Their waits are explicit
// (lgkm_wait), and `reg_after` orders a register's uses after such a wait.
template <int OFF> __device__ inline u32x4 lds_read_b128(uint32_t addr) {
  u32x4 x;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "n"(OFF));
  return x;
}
template <int O64> __device__ inline u32x4 lds_read2st64_b64(uint32_t addr) {
  u32x4 x;
  asm volatile("ds_read2st64_b64 %0, %1 offset0:%2 offset1:%3"
               : "=v"(x) : "v"(addr), "n"(O64), "n"(O64 + 1));
  return x;
}
template <int N> __device__ inline void lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N)); }
template <int N> __device__ inline void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N)); }
__device__ inline void reg_after(u32x4& x) { asm volatile("" : "+v"(x)); }

// All K and V fragments of one stage (byte offset Base in the ring), with
// the stage and chunk offsets in the instructions' offset fields.
template <int Base, class Tag, int D, int... I>
__device__ inline void read_k(FragPair<Tag, D>& f, uint32_t ka, std::integer_sequence<int, I...>) {
  ((f.k[I / (D / 32)][I % (D / 32)] = lds_read_b128<Base + I * 1024>(ka)), ...);
}
template <int Base, int... I>
__device__ inline void read_raw(u32x4* x, uint32_t addr, std::integer_sequence<int, I...>) {
  ((x[I] = lds_read_b128<Base + I * 1024>(addr)), ...);
}
template <int Base, class Tag, int D, int... I>
__device__ inline void read_v(FragPair<Tag, D>& f, uint32_t va, std::integer_sequence<int, I...>) {
  static_assert(Base % 512 == 0, "stage offsets are whole 512-byte units");
  ((f.v[I] = lds_read2st64_b64<(Base + I * 1024) / 512>(va)), ...);
}

template <class Tag, int D, int NQ, class OutT>
__global__ __launch_bounds__(kPThreads) void prefill_ring_kernel(PrefillArgs a) {
  using RG = Ring<Tag, D>;
  using CT = typename ComputeTag<Tag>::type;   // FP8 codes become bf16 in the slots
  constexpr bool F8 = RG::kF8;
  using PT = std::conditional_t<F8, TagF16, CT>;   // P.V: FP8 V codes become fp16
  constexpr int ES = Elt<Tag>::bytes;
  __shared__ __attribute__((aligned(1024))) char ring[RG::kBytes];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // Workgroup order: as in prefill_kernel below.
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;
  const int pair = xcd + kXcds * (k / a.num_tiles);
  if (pair >= a.num_seqs * a.num_kv_heads) return;
  const int seq = pair / a.num_kv_heads;
  const int g = pair - seq * a.num_kv_heads;
  const int tile = a.num_tiles - 1 - k % a.num_tiles;

  const int qs = a.q_start[seq];
  const int n = a.q_start[seq + 1] - qs;
  int L = a.lens[seq];
  L = L < 0 ? 0 : L;
  L = L > a.max_len ? a.max_len : L;
  const int64_t cap = (int64_t)a.max_blocks * a.block_size;
  if ((int64_t)L > cap) L = (int)cap;

  // The whole workgroup leaves together or not at all (barriers below);
  // a wavefront without rows still loads its share of every step.
  const int wg_row0 = tile * kPWaves * a.wave_rows;
  if (wg_row0 >= n) return;
  const int wg_end = min(n, wg_row0 + kPWaves * a.wave_rows);
  const int row0 = wg_row0 + wave * a.wave_rows;
  const int row_end = min(n, row0 + a.wave_rows);
  const int G = a.group;
  const int head0 = g * G;

  const int c = lane & 15;
  const int cr = c / G;
  const int chh = c - cr * G;
  const bool col_ok = c < a.tpg * G;
  QFrag<Tag, D> qf[NQ];
  int pos[NQ];
  bool has[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int t = row0 + q * a.tpg + cr;
    const int p = L - n + t;
    has[q] = col_ok && t < row_end && p >= 0;
    pos[q] = has[q] ? p : 0;              // idle columns see key 0 only (their q is 0)
    const int64_t qrow = has[q] ? ((int64_t)(qs + t) * a.num_q_heads + head0 + chh) : 0;
    qf[q].load(a.q + qrow * D * 2, has[q], lane);
  }
  // FP8: the head's K scale folds into the score scale, its V scale into the
  // output (a zero product becomes the smallest normal float, as on the host).
  float qk_scale = a.qk_scale;
  float v_scale = 1.f;
  if constexpr (F8) {
    qk_scale *= a.k_scales[g];
    if (qk_scale == 0.f) qk_scale = 1.17549435e-38f;
    v_scale = a.v_scales[g];
  }
  State<D> st[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    st[q].m = -INFINITY;
    st[q].l = 0.f;
#pragma unroll
    for (int d = 0; d < D / 16; ++d) st[q].acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Keys 0 .. p_wg for the workgroup's rows; every wavefront walks them all
  // (keys past a wavefront's last row are masked by the causal limits).
  const int p_wg = L - n + wg_end - 1;
  const int nsteps = p_wg >= 0 ? p_wg / 32 + 1 : 0;

  const int R = a.rows;
  const int r_shift = R == 8 ? 3 : 4;
  const int b_shift = a.block_size == 8 ? 3 : a.block_size == 16 ? 4 : 5;
  const int64_t tile_bytes = (int64_t)a.block_size * D * ES;
  const int sub_bytes = R * D * ES;
  const uint32_t block_stride = (uint32_t)(a.num_kv_heads * tile_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lchar)ring;

  // Each lane's part of a step's loads, fixed for the whole walk.  16-bit
  // pools: wavefront h < 2 loads K of tile h, lane (t, piece) = (lane % 16,
  // lane / 16); wavefronts 2-3 load V, lane (tile, token group, dim pair) =
  // (lane / 32, (lane / 8) % 4, lane % 8).  FP8 pools (raw codes, the pool's
  // own per-lane pieces, include/pa.h): wavefront h < 2 loads K of tile h,
  // lane (row, dim quarter) = (lane % 16, lane / 16); wavefront 2 + h loads V
  // of tile h, lane (dim row, token group) = (lane % 16, lane / 16).  The
  // lane's rows lie in quarter qi (keys 8 qi .. 8 qi + 7 of the step), in
  // block qblk counted from the step's first block (a step starts on a block
  // boundary), at byte offset lane_off inside that block's tile of this KV
  // head; instruction i adds i * inst_stride.
  int qi;
  if constexpr (F8) qi = wave < 2 ? 2 * wave + ((lane >> 3) & 1) : 2 * (wave - 2) + (lane >> 5);
  else qi = wave < 2 ? 2 * wave + ((lane >> 3) & 1) : (lane >> 4) & 3;
  const int in_blk = (8 * qi) & (a.block_size - 1);
  const int qblk = (8 * qi) >> b_shift;
  const int row_q = in_blk & (R - 1);
  uint32_t lane_off = (uint32_t)((in_blk >> r_shift) * sub_bytes);
  uint32_t inst_stride;
  if constexpr (F8) {
    if (wave < 2) {
      lane_off += (uint32_t)((row_q + (lane & 7)) * 16 + (lane >> 4) * (R * D / 4));
      inst_stride = (uint32_t)(R * 16);
    } else {
      lane_off += (uint32_t)(((row_q >> 2) + ((lane >> 4) & 1)) * 4 * D + (lane & 15) * 16);
      inst_stride = 256u;
    }
  } else {
    if (wave < 2) {
      lane_off += (uint32_t)((row_q + (lane & 7)) * 64 + (lane >> 4) * 16);
      inst_stride = (uint32_t)(R * 64);
    } else {
      lane_off += (uint32_t)(((row_q >> 2) + ((lane >> 3) & 1)) * D * 8 + (lane & 7) * 16 +
                             (wave - 2) * RG::kChunks * 128);   // first dim tile of this wavefront
      inst_stride = 128u;
    }
  }
  const uint64_t lane_base = (wave < 2 ? (uint64_t)a.k_pool : (uint64_t)a.v_pool) +
                             (uint64_t)((int64_t)g * tile_bytes) + lane_off;

  // Table window: lane i holds block B0 + i's physical id (0 when outside
  // the pool or past the stored length, so every address stays in the
  // pool); okw bit i says whether that block holds stored keys.
  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  const int blocks_per_step = 32 >> b_shift;
  int B0 = 0;
  int win = 0;
  uint64_t okw = 0;
  auto load_window = [&](int b0) {
    B0 = b0;
    const int B = b0 + lane;
    const int phys = (int64_t)B * a.block_size < L ? trow[B] : -1;
    const bool ok = phys >= 0 && phys < a.num_blocks;
    win = ok ? phys : 0;
    okw = __builtin_amdgcn_ballot_w64(ok);
  };
  load_window(0);

  // Loads of step j, in two parts: `prepare` (table window, this lane's
  // source address, the step's valid-key bits: key k valid when position
  // 32 j + k is below L and its block is in the pool) runs before the
  // barrier; `dma` copies into a stage, after it.
  struct Prep {
    uint64_t src;
    uint32_t valid;
  };
  auto prepare = [&](int j) -> Prep {
    const int Bs = (32 * j) >> b_shift;        // the step's first block
    if (Bs + blocks_per_step > B0 + kWave) load_window(Bs);
    const int phys = __builtin_amdgcn_ds_bpermute((Bs - B0 + qblk) * 4, win);
    Prep pr;
    pr.src = lane_base + (uint64_t)(uint32_t)phys * block_stride;
    const uint32_t okq = (uint32_t)(okw >> (Bs - B0));     // bit k: block Bs + k
    const uint32_t all = (1u << blocks_per_step) - 1u;
    if (32 * j + 32 <= L && (okq & all) == all) {
      pr.valid = 0xffffffffu;
    } else {
      uint32_t valid = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nv = (okq >> ((8 * i) >> b_shift)) & 1u ? min(8, L - 32 * j - 8 * i) : 0;
        valid |= nv > 0 ? ((1u << nv) - 1u) << (8 * i) : 0u;
      }
      pr.valid = valid;
    }
    return pr;
  };
  // Destination chunk of this wavefront's instruction i in a stage:
  // 16-bit K (h, m) -> h * kChunks + m, V dim tile n -> kKBytes / 1024 + n;
  // FP8 raw K (h, piece) -> h * kRawChunks + piece, V -> 2 kRawChunks + ...
  auto dma = [&](const Prep& pr, int stg) {
    const uint32_t dst = lds0 + (F8 ? RG::kRawBase + stg * RG::kRawStep : stg * RG::kStep);
    const int c0 = wave * RG::kPerWave;
#pragma unroll
    for (int i = 0; i < RG::kPerWave; ++i)
      __builtin_amdgcn_global_load_lds((gchar)(pr.src + (uint32_t)(i * inst_stride)),
                                       (lchar)(uintptr_t)(dst + (c0 + i) * 1024), 16, 0, 0);
  };

  // Landing of step j's loads in stage stg, by each lane for the pieces it
  // loaded, once its own loads of that step are done (before the barrier
  // that publishes the stage).  16-bit pools: on a step with invalid keys the
  // V-loading lanes zero those keys' elements (a tail past L or a block
  // outside the pool may hold NaN, and 0 * NaN would reach the accumulators).
  // FP8 pools: every lane widens its raw codes into the stage's 16-bit slot,
  // K to bf16 and V to fp16 (both exact for every E4M3 value), V with the
  // same zeroing.  V piece of lane (d, tg) holds tokens 4 tg .. 4 tg + 3.
  auto v_keep = [&](uint32_t valid, int tile, uint32_t& k0, uint32_t& k1) {
    const uint32_t bits = valid >> (16 * tile + 4 * (F8 ? lane >> 4 : (lane >> 3) & 3));
    k0 = (bits & 1u ? 0x0000ffffu : 0u) | (bits & 2u ? 0xffff0000u : 0u);
    k1 = (bits & 4u ? 0x0000ffffu : 0u) | (bits & 8u ? 0xffff0000u : 0u);
  };
  // FP8: widen this lane's raw pieces x (of the step in raw stage rs) into
  // slot stg.  land() reads the pieces itself; the main loop reads them
  // early (raw_read) and widens them during the softmax.
  auto widen = [&](int stg, uint32_t valid, const u32x4* x) {
    char* slot = ring + stg * RG::kStep;
    if (wave < 2) {                     // K of tile `wave`: piece p -> fragments m = 2p, 2p + 1
#pragma unroll
      for (int pc = 0; pc < RG::kRawChunks; ++pc)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          *reinterpret_cast<u32x4*>(slot + (wave * RG::kChunks + 2 * pc + u) * 1024 + lane * 16) =
              u32x4{fp8x2_to_bf16x2<false>(x[pc][2 * u]), fp8x2_to_bf16x2<true>(x[pc][2 * u]),
                    fp8x2_to_bf16x2<false>(x[pc][2 * u + 1]), fp8x2_to_bf16x2<true>(x[pc][2 * u + 1])};
    } else {                            // V of tile h: dword e of piece p is dim tile 4p + e
      const int h = wave - 2;
      uint32_t k0 = 0xffffffffu, k1 = 0xffffffffu;
      if (valid != 0xffffffffu) v_keep(valid, h, k0, k1);
#pragma unroll
      for (int pc = 0; pc < RG::kRawChunks; ++pc)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<u32x2*>(slot + RG::kKBytes + (4 * pc + e) * 1024 + h * 512 + lane * 8) =
              u32x2{fp8x2_to_f16x2<false>(x[pc][e]) & k0, fp8x2_to_f16x2<true>(x[pc][e]) & k1};
    }
  };
  const uint32_t rawa = lds0 + (uint32_t)(RG::kRawBase + wave * RG::kRawChunks * 1024 + lane * 16);
  auto land = [&](int stg, uint32_t valid) {
    if constexpr (F8) {
      const char* raw = ring + RG::kRawBase + stg * RG::kRawStep;
      u32x4 x[RG::kRawChunks];
#pragma unroll
      for (int pc = 0; pc < RG::kRawChunks; ++pc)
        x[pc] = *reinterpret_cast<const u32x4*>(raw + (wave * RG::kRawChunks + pc) * 1024 + lane * 16);
      widen(stg, valid, x);
      lgkm_wait<0>();
    } else {
      if (wave >= 2 && valid != 0xffffffffu) {
        uint32_t k0, k1;
        v_keep(valid, lane >> 5, k0, k1);
        const int n0 = (wave - 2) * RG::kChunks;
#pragma unroll
        for (int i = 0; i < RG::kChunks; ++i) {
          u32x4* piece = reinterpret_cast<u32x4*>(ring + stg * RG::kStep + RG::kKBytes +
                                                  (n0 + i) * 1024 + lane * 16);
          const u32x4 x = *piece;
          *piece = u32x4{x[0] & k0, x[1] & k1, x[2] & k0, x[3] & k1};
        }
        lgkm_wait<0>();
      }
    }
  };

  // Step j (stage S = j % 4), software-pipelined across steps: the scores
  // S^T of step j were computed during step j - 1.  Read V of step j and K of
  // step j + 1 from LDS; while those reads are in flight, mask step j's
  // scores where needed, take its exponentials (and move the base if one
  // exceeds 2^8) and narrow P; then, held behind a scheduling barrier so that
  // the compiler does not sink that vector work into the matrix phase, step
  // j + 1's scores and step j's P.V products (measured: 820 -> 795 us on 16 x
  // 2048 prompts).  LDS reads complete in order.  On the last step the next stage holds no
  // step (stale or never written LDS): its scores are computed and unused,
  // which keeps the step free of branches.
  const uint32_t ka = lds0 + lane * 16, va = lds0 + lane * 8;
  uint2 neg = {0x0000bf80u, 0xbf800000u};   // bf16 pairs (-1, 0), (0, -1): minus_hi
  asm("" : "+s"(neg.x));
  asm("" : "+s"(neg.y));
  FragPair<CT, D> f;                    // f.k: next step's K, f.v: this step's V
  f32x4 sa[NQ], sb[NQ];                 // this step's scores
  auto scores = [&](f32x4* xa, f32x4* xb) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) qk_pair<CT, D>(f, qf[q], xa[q], xb[q]);
  };
  // vm_steps(k): wait until at most k steps' loads of this wavefront are
  // outstanding.
  auto vm_steps = [](int k) {
    if (k >= 2) vm_wait<2 * RG::kPerWave>(); else if (k == 1) vm_wait<RG::kPerWave>(); else vm_wait<0>();
  };
  static_assert(F8 || RG::kAhead <= 3, "vm_steps covers up to two newer steps");
  // Valid-key bits per slot (of the step whose K/V it holds); FP8 also per
  // raw stage (of the step loading into it).
  uint32_t valid[RG::kStages], vraw[RG::kStages];
#pragma unroll
  for (int i = 0; i < RG::kStages; ++i) valid[i] = vraw[i] = 0u;
  auto compute = [&](auto stage_c, int j, uint32_t valid_j) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int S1 = (S + 1) % RG::kStages;
    constexpr int S2 = (S + 2) % RG::kStages;
    // FP8: the raw pieces of step j + 2, read between this step's V and K
    // fragments and widened into their slot during the softmax.
    u32x4 rx[RG::kRawChunks];
    const bool widen_next = F8 && j + 2 < nsteps;
    read_v<S * RG::kStep + RG::kKBytes>(f, va, std::make_integer_sequence<int, D / 16>());
    if constexpr (F8) {
      if (widen_next) {
        vm_steps(nsteps - 3 - j);         // this lane's loads of step j + 2 have landed
        read_raw<S2 * RG::kRawStep>(rx, rawa, std::make_integer_sequence<int, RG::kRawChunks>());
      }
    }
    read_k<S1 * RG::kStep>(f, ka, std::make_integer_sequence<int, 2 * RG::kChunks>());
    const int key0 = 32 * j;
    bool need = valid_j != 0xffffffffu;
#pragma unroll
    for (int q = 0; q < NQ; ++q) need |= __builtin_amdgcn_ballot_w64(pos[q] - key0 + 1 < 2 * kRows) != 0;
    if (need) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) mask_scores<D>(sa[q], sb[q], valid_j, qk_scale, lane, pos[q] - key0 + 1);
    }
    float p[NQ][8], ps[NQ];
    bool fix = false;
#pragma unroll
    for (int q = 0; q < NQ; ++q) fix |= take_exps<D>(sa[q], sb[q], st[q], qk_scale, p[q], ps[q]);
    if (__builtin_amdgcn_ballot_w64(fix) != 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) rebase<D>(sa[q], sb[q], st[q], qk_scale, p[q], ps[q]);
    }
    PPack pk[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) pk[q] = narrow_p<PT, D>(p[q], ps[q], st[q], neg);
    if constexpr (F8) {
      if (widen_next) {
        lgkm_wait<2 * RG::kChunks>();     // V fragments and the raw pieces (K may be in flight)
#pragma unroll
        for (int pc = 0; pc < RG::kRawChunks; ++pc) reg_after(rx[pc]);
        widen(S2, vraw[S2], rx);
        valid[S2] = vraw[S2];
      }
    }
    // The softmax of this step runs while its LDS reads are in flight; the
    // matrix products wait for them.
    __builtin_amdgcn_sched_barrier(0);
    lgkm_wait<0>();                     // V of this step and K of the next
#pragma unroll
    for (int d = 0; d < D / 16; ++d) reg_after(f.v[d]);
    f32x4 na[NQ], nb[NQ];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < RG::kChunks; ++m) reg_after(f.k[h][m]);
    scores(na, nb);
#pragma unroll
    for (int q = 0; q < NQ; ++q) pv_products<PT>(f, pk[q], st[q]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      sa[q] = na[q];
      sb[q] = nb[q];
    }
  };

  // Ring of kStages stages; loads run kAhead = kStages - 1 steps ahead of the
  // computation: at step j the stage of step j - 1 (all of its reads done,
  // by the barrier) takes the loads of step j + kAhead.  Before the barrier
  // of step j this wavefront's loads of step j + 1 are done (later steps' may
  // still run), so after it every wavefront may read step j + 1's K.
  // vm_steps(k): wait until at most k steps' loads of this wavefront are
  // outstanding.
  auto start = [&](int i) {             // loads of step i into stage i % kStages
    const Prep pr = prepare(i);
    (F8 ? vraw : valid)[i % RG::kStages] = pr.valid;
    dma(pr, i % RG::kStages);
  };
  if constexpr (F8) {
    // Steps 0 and 1 are widened before the first barrier; step 3's loads
    // reuse step 0's raw stage once this lane has widened it.
    for (int i = 0; i < 3 && i < nsteps; ++i) start(i);
    if (nsteps > 0) {
      vm_steps(min(2, nsteps - 1));
      valid[0] = vraw[0];
      land(0, valid[0]);
      if (nsteps > 3) start(3);
    }
    if (nsteps > 1) {
      vm_steps((nsteps > 2) + (nsteps > 3));
      valid[1] = vraw[1];
      land(1, valid[1]);
    }
  } else {
    for (int i = 0; i < RG::kAhead && i < nsteps; ++i) start(i);
    if (nsteps > 0) {
      vm_steps(min(RG::kAhead, nsteps) - 1);
      land(0, valid[0]);
    }
  }
  if (nsteps > 0) {
    __builtin_amdgcn_s_barrier();
    read_k<0>(f, ka, std::make_integer_sequence<int, 2 * RG::kChunks>());
    lgkm_wait<0>();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < RG::kChunks; ++m) reg_after(f.k[h][m]);
    scores(sa, sb);
  }
  auto step = [&](auto stage_c, int j) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int S1 = (S + 1) % RG::kStages;
    constexpr int SA = (S + RG::kAhead) % RG::kStages;
    Prep pr;
    const bool more = j + RG::kAhead < nsteps;
    if (more) pr = prepare(j + RG::kAhead);
    if constexpr (!F8) {
      if (j + 1 < nsteps) {
        vm_steps(min(RG::kAhead - 2, nsteps - j - 2));
        land(S1, valid[S1]);              // this wavefront's loads of step j + 1 are done
      }
    }
    __builtin_amdgcn_s_barrier();
    if (more) {
      (F8 ? vraw : valid)[SA] = pr.valid;
      dma(pr, SA);
    }
    compute(stage_c, j, valid[S]);
  };
  for (int j = 0; j < nsteps; j += RG::kStages) {
    step(std::integral_constant<int, 0>(), j);
    if (j + 1 >= nsteps) break;
    step(std::integral_constant<int, 1>(), j + 1);
    if (j + 2 >= nsteps) break;
    step(std::integral_constant<int, 2>(), j + 2);
    if constexpr (RG::kStages > 3) {
      if (j + 3 >= nsteps) break;
      step(std::integral_constant<int, 3 % RG::kStages>(), j + 3);
    }
  }

#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float l_tot = xor_sum(st[q].l);
    const int t = row0 + q * a.tpg + cr;
    if (!(col_ok && t < row_end)) continue;
    const float inv = (has[q] && l_tot > 0.f) ? v_scale / l_tot : 0.f;
    OutT* o = reinterpret_cast<OutT*>(a.out) +
              ((int64_t)(qs + t) * a.num_q_heads + head0 + chh) * D;
#pragma unroll
    for (int d = 0; d < D / 16; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_out<OutT>(o + out_dim<Tag, D>(d, r, lane), st[q].acc[d][r] * inv);
  }
}

// fp32 pools: each wavefront walks on its own, one sub-tile per step with a
// second buffer one step ahead, through cached buffer loads.
template <class Tag, int D, int NQ, class OutT>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  static_assert(!Is16<Tag>::value, "16-bit and FP8 pools run prefill_ring_kernel");
  constexpr int ES = Elt<Tag>::bytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // Workgroup order.  The dispatcher places workgroup i on XCD i % kXcds,
  // each XCD with its own L2.  XCD x takes (sequence, KV head) pairs x,
  // x + kXcds, ... and runs all row tiles of one pair (last rows, the most
  // keys, first) before the next, so its resident workgroups share one or two
  // K/V prefixes in its L2; with kXcds KV heads every XCD holds one head of
  // every sequence, which also balances their work.
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;
  const int pair = xcd + kXcds * (k / a.num_tiles);
  if (pair >= a.num_seqs * a.num_kv_heads) return;
  const int seq = pair / a.num_kv_heads;
  const int g = pair - seq * a.num_kv_heads;
  const int tile = a.num_tiles - 1 - k % a.num_tiles;

  const int qs = a.q_start[seq];
  const int n = a.q_start[seq + 1] - qs;
  int L = a.lens[seq];
  L = L < 0 ? 0 : L;
  L = L > a.max_len ? a.max_len : L;
  const int64_t cap = (int64_t)a.max_blocks * a.block_size;
  if ((int64_t)L > cap) L = (int)cap;

  const int row0 = (tile * kPWaves + wave) * a.wave_rows;   // this wavefront's first chunk row
  if (row0 >= n) return;                                     // no barriers below
  const int row_end = min(n, row0 + a.wave_rows);
  const int G = a.group;
  const int head0 = g * G;

  // Columns: lane c (= lane % 16) of group q is chunk row row0 + q*tpg + c/G,
  // head head0 + c%G; columns past tpg*G or past the chunk are idle.
  const int c = lane & 15;
  const int cr = c / G;
  const int chh = c - cr * G;
  const bool col_ok = c < a.tpg * G;
  QFrag<Tag, D> qf[NQ];
  int pos[NQ];
  bool has[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int t = row0 + q * a.tpg + cr;
    const int p = L - n + t;
    has[q] = col_ok && t < row_end && p >= 0;
    pos[q] = has[q] ? p : 0;              // idle columns see key 0 only (their q is 0)
    const int64_t qrow = has[q] ? ((int64_t)(qs + t) * a.num_q_heads + head0 + chh) : 0;
    qf[q].load(a.q + qrow * D * In<Tag>::bytes, has[q], lane);
  }
  const float qk_scale = a.qk_scale;

  // Keys 0 .. p_last, where p_last is the position of the wavefront's last row.
  const int p_last = L - n + row_end - 1;
  State<D> st[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    st[q].m = -INFINITY;
    st[q].l = 0.f;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) st[q].acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t tile_bytes = (int64_t)a.block_size * D * ES;
  const int sub_bytes = a.rows * D * ES;
  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  const int64_t head_tile = (int64_t)g * tile_bytes;
  const int64_t block_stride = (int64_t)a.num_kv_heads * tile_bytes;
  const int cnt = p_last >= 0 ? p_last / a.rows + 1 : 0;    // sub-tiles to walk

  int c0 = 0, nc = 0, tb = 0;
  // Sub-tile i of the current chunk: its physical tile offset and stored-token
  // count (0 past the walk or for a table entry outside the pool, whose
  // resource then has size 0 and reads zeros).
  auto locate = [&](int i, int64_t& off, int& bytes, int& nv) {
    int phys = __builtin_amdgcn_readlane(tb, min(i, nc - 1));
    const int j = c0 + i;
    const bool ok = i < nc && phys >= 0 && phys < a.num_blocks;
    nv = ok ? min(a.rows, L - j * a.rows) : 0;
    if (!ok) phys = 0;
    off = (int64_t)phys * block_stride + head_tile + (int64_t)(j % a.sub) * sub_bytes;
    bytes = ok ? sub_bytes : 0;
  };
  auto open_table = [&]() {
    nc = min(kWave, cnt - c0);
    tb = lane < nc ? trow[(c0 + lane) / a.sub] : 0;
  };

  Frag<Tag, D> fa, fb;
  int nva = 0, nvb = 0;
  auto load_into = [&](Frag<Tag, D>& f, int i, int& nv) {
    int64_t off;
    int bytes;
    locate(i, off, bytes, nv);
    f.template load<kPolicyCached>(tile_rsrc(a.k_pool + off, bytes),
                                   tile_rsrc(a.v_pool + off, bytes), lane, a.rows);
  };
  auto attend = [&](const Frag<Tag, D>& f, int nv, int i) {
    if (nv <= 0) return;
    const int key0 = (c0 + i) * a.rows;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      attend_block<Tag, D>(f, qf[q], st[q], nv, qk_scale, lane, pos[q] - key0 + 1);
  };
  for (; c0 < cnt; c0 += kWave) {
    open_table();
    load_into(fa, 0, nva);
    for (int i = 0; i < nc; i += 2) {
      load_into(fb, i + 1, nvb);
      attend(fa, nva, i);
      if (i + 1 >= nc) break;
      load_into(fa, i + 2, nva);
      attend(fb, nvb, i + 1);
    }
  }

  // Normalise and store: acc[k][r] is output dim out_dim(k, r) of the lane's column.
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float l_tot = xor_sum(st[q].l);
    const int t = row0 + q * a.tpg + cr;
    if (!(col_ok && t < row_end)) continue;
    const float inv = (has[q] && l_tot > 0.f) ? 1.f / l_tot : 0.f;
    OutT* o = reinterpret_cast<OutT*>(a.out) +
              ((int64_t)(qs + t) * a.num_q_heads + head0 + chh) * D;
#pragma unroll
    for (int k = 0; k < D / 16; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_out<OutT>(o + out_dim<Tag, D>(k, r, lane), st[q].acc[k][r] * inv);
  }
}

template <class Tag, int D, class OutT>
static pa_status launch_prefill(const PrefillArgs& a, int64_t units, hipStream_t s) {
  if constexpr (Is16<Tag>::value)
    prefill_ring_kernel<Tag, D, kNQ, OutT><<<(unsigned)units, kPThreads, 0, s>>>(a);
  else
    prefill_kernel<Tag, D, kNQ, OutT><<<(unsigned)units, kPThreads, 0, s>>>(a);
  return launch_status();
}

template <class Tag, class OutT>
static pa_status dispatch_prefill(int D, const PrefillArgs& a, int64_t units, hipStream_t s) {
  if (D == 128) return launch_prefill<Tag, 128, OutT>(a, units, s);
  return launch_prefill<Tag, 64, OutT>(a, units, s);
}

}  // namespace pa

using namespace pa;

extern "C" {

pa_status pa_prefill_attention(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                               const void* q, void* out, pa_dtype out_dtype,
                               const int32_t* q_start, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, float scale,
                               int32_t max_chunk_len, int32_t max_context_len, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 0 || max_context_len < 0 ||
      max_chunk_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads) return PA_ERR_INVALID_ARG;
  const int32_t G = num_q_heads / pool->num_kv_heads;
  if (G > 16) return PA_ERR_UNSUPPORTED;
  const pa_dtype out16 = pool->dtype == PA_FP8_E4M3 ? PA_BF16 : pool->dtype;
  if (out_dtype != PA_F32 && out_dtype != out16) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_chunk_len == 0) return PA_OK;
  if (!k_pool || !v_pool || !q || !out || !q_start || !context_lens) return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq > 0 && !block_tables) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(q) || !aligned16(out))
    return PA_ERR_INVALID_ARG;
  if (!(scale == scale)) return PA_ERR_INVALID_ARG;

  PrefillArgs a;
  a.k_pool = (const char*)k_pool;
  a.v_pool = (const char*)v_pool;
  a.q = (const char*)q;
  a.out = out;
  a.q_start = q_start;
  a.tables = block_tables;
  a.lens = context_lens;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.rows = std::min(pool->block_size, 16);
  a.sub = pool->block_size / a.rows;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = G;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.max_len = max_context_len;
  a.tpg = 16 / G;
  a.wave_rows = kNQ * a.tpg;
  const int32_t wg_rows = kPWaves * a.wave_rows;
  a.num_tiles = (max_chunk_len + wg_rows - 1) / wg_rows;
  a.qk_scale = scale * 1.4426950408889634f;
  // A zero scale becomes the smallest normal float: every exponential is still
  // exactly 1, and a masked score (-inf) still gives -inf rather than NaN.
  if (a.qk_scale == 0.f) a.qk_scale = 1.17549435e-38f;
  a.k_scales = pool->k_scales;
  a.v_scales = pool->v_scales;
  const int64_t pairs = (int64_t)a.num_kv_heads * num_seqs;
  const int64_t units = (pairs + kXcds - 1) / kXcds * kXcds * a.num_tiles;
  if (units > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  const int D = pool->head_dim;
  switch (pool->dtype) {
    case PA_BF16:
      return out_dtype == PA_F32 ? dispatch_prefill<TagBF16, float>(D, a, units, s)
                                 : dispatch_prefill<TagBF16, __bf16>(D, a, units, s);
    case PA_F16:
      return out_dtype == PA_F32 ? dispatch_prefill<TagF16, float>(D, a, units, s)
                                 : dispatch_prefill<TagF16, _Float16>(D, a, units, s);
    case PA_FP8_E4M3:
      return out_dtype == PA_F32 ? dispatch_prefill<TagFP8, float>(D, a, units, s)
                                 : dispatch_prefill<TagFP8, __bf16>(D, a, units, s);
    case PA_F32:
      return dispatch_prefill<TagF32, float>(D, a, units, s);
    default:
      return PA_ERR_UNSUPPORTED;
  }
}

}  // extern "C"
