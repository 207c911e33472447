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
// sequence's 16-token sub-tiles from position 0 up to its last row's
// position: S^T = K q^T on the matrix cores, a causal mask per column, online
// softmax, O^T += V^T P^T with P split into high and low 16-bit halves.  Each
// K/V fragment serves NQ groups; the four wavefronts of a workgroup take
// consecutive row ranges of one (sequence, KV head) and re-read the same
// tiles, which the L1 and L2 serve (cached loads, unlike decode's streaming
// ones).  For 16-bit pools a step is two sub-tiles held in one register
// buffer that is refilled in phases (the next K once this step's S^T products
// are issued, the next V once its P.V products are), which keeps the kernel
// under 256 registers: two wavefronts per SIMD.  Sub-tile addresses are built
// 64 at a time, one per lane, and broadcast per step.  FP8 and fp32 pools take
// one sub-tile per step with a second buffer one step ahead.  Each XCD runs
// the row tiles of one (sequence, KV head) after another, last rows (the most
// keys) first, so its resident workgroups share K/V in its L2.
#include <algorithm>

#include "pa_tile.h"

namespace pa {

// ---- two sub-tiles per step (multi-token queries, 16-bit storage) ----------
// 32 keys per step: the P.V product's k dimension holds 4 tokens of each
// sub-tile per lane group (k slots 0..3: sub-tile a, 4..7: sub-tile b), so
// the V operand is two 8-byte loads side by side -- no duplicated V -- and
// the high and low 16-bit parts of P are two products with the same V.  The
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
template <class Tag> __device__ inline f32x2 unpack2(uint32_t w);
template <> __device__ inline f32x2 unpack2<TagBF16>(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(bf16x2, w), f32x2);
}
template <> __device__ inline f32x2 unpack2<TagF16>(uint32_t w) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

typedef const __attribute__((address_space(1))) char* gchar;

template <class Tag, int D> struct FragPair {
  u32x4 k[2][D / 32];     // K of sub-tiles a and b (the Frag<Tag> lane roles)
  u32x4 v[D / 16];        // dim tile n: .xy = sub-tile a's 4 tokens, .zw = b's
  // ka, kb: the two K sub-tiles (wave-uniform); kro[m]: this lane's byte
  // offset of K dims 32m.. (rows-dependent).  Plain cached global loads.
  __device__ inline void load_k(gchar ka, gchar kb, const uint32_t* kro) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      // The empty statement pins the 32-bit offset here, so the address stays
      // "uniform base + zero-extended lane offset" (one load, no 64-bit adds)
      // instead of a hoisted 64-bit per-lane value.
      uint32_t o = kro[m];
      asm volatile("" : "+v"(o));
      k[0][m] = *(const __attribute__((address_space(1))) u32x4*)(ka + o);
      k[1][m] = *(const __attribute__((address_space(1))) u32x4*)(kb + o);
    }
  }
  // va, vb: the two V sub-tiles; vr: this lane's byte offset of V dim-tile 0
  // (tile n adds 128 n).
  __device__ inline void load_v(gchar va, gchar vb, uint32_t vr) {
    asm volatile("" : "+v"(vr));
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const u32x2 x = *(const __attribute__((address_space(1))) u32x2*)(va + vr + n * 128);
      const u32x2 y = *(const __attribute__((address_space(1))) u32x2*)(vb + vr + n * 128);
      v[n] = u32x4{x[0], x[1], y[0], y[1]};
    }
  }
};

// Zero the V tokens at and past each sub-tile's stored count, in place (a
// tail may hold NaN, and 0 * NaN would reach the accumulators).  The masks
// depend on the stored counts only, so one pass serves every column group.
template <class Tag, int D>
__device__ inline void mask_v_tails(FragPair<Tag, D>& f, int nva, int nvb, int lane) {
  const int t0 = 4 * (lane >> 4);
  uint32_t keep[4];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    keep[w] = (t0 + 2 * w < nva ? 0x0000ffffu : 0u) | (t0 + 2 * w + 1 < nva ? 0xffff0000u : 0u);
    keep[2 + w] = (t0 + 2 * w < nvb ? 0x0000ffffu : 0u) | (t0 + 2 * w + 1 < nvb ? 0xffff0000u : 0u);
  }
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[n][e] &= keep[e];
}

// S^T of the pair's two sub-tiles for one column group.
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

// Online softmax and O^T += V^T P^T for one column group, from its scores.
// nva, nvb: stored tokens of the two sub-tiles (0 for none); lima, limb: per
// lane, the column's causal limit in rows of each sub-tile (>= 16: all
// visible).  V tails must already be masked (mask_v_tails).
template <class Tag, int D>
__device__ inline void softmax_pv(const FragPair<Tag, D>& f, f32x4 sa, f32x4 sb, State<D>& st,
                                  int nva, int nvb, float qk_scale, int lane, int lima,
                                  int limb) {
  float x[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = sa[r] * qk_scale;
    x[4 + r] = sb[r] * qk_scale;
  }
  if (nva < kRows || nvb < kRows ||
      __builtin_amdgcn_ballot_w64(lima < kRows || limb < kRows) != 0) {
    const int t0 = 4 * (lane >> 4);
    const int ea = min(nva, lima), eb = min(nvb, limb);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // select, never multiply: tails may hold NaN
      if (t0 + r >= ea) x[r] = -INFINITY;
      if (t0 + r >= eb) x[4 + r] = -INFINITY;
    }
  }
  bool over = false;
#pragma unroll
  for (int r = 0; r < 8; ++r) over |= x[r] > st.m + kRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(over) != 0) {
    float bm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    bm = xor_max(bm);
    const float m_new = fmaxf(st.m, bm);
    const float alpha = fast_exp2(st.m - (m_new == -INFINITY ? 0.f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) st.acc[n] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == -INFINITY ? 0.f : st.m;
  float p[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) p[r] = fast_exp2(x[r] - base);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  u32x4 hi, lo;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 pw = {p[2 * w], p[2 * w + 1]};
    hi[w] = pack2<Tag>(pw);
    lo[w] = pack2<Tag>(pw - unpack2<Tag>(hi[w]));
  }
#pragma unroll
  for (int n = 0; n < D / 16; ++n) st.acc[n] = mma32<Tag>(f.v[n], hi, st.acc[n]);
#pragma unroll
  for (int n = 0; n < D / 16; ++n) st.acc[n] = mma32<Tag>(f.v[n], lo, st.acc[n]);
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

template <class Tag, int D, int NQ, class OutT>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
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
  // FP8: the head's K scale folds into the score scale, its V scale into the output.
  float qk_scale = a.qk_scale;
  float v_scale = 1.f;
  if constexpr (Elt<Tag>::bytes == 1) {
    qk_scale *= a.k_scales[g];
    v_scale = a.v_scales[g];
  }

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

  if constexpr (Is16<Tag>::value && !IsFP8<Tag>::value) {
    // Two sub-tiles per step, two steps in registers (one ahead).  Sub-tile
    // descriptors are built 64 at a time, one per lane (K address and stored
    // count), and read with lane broadcasts; a pair never straddles two sets.
    // Sub-tiles past the walk or behind a table entry outside the pool get
    // count 0 and the address of block 0's tile (in bounds: a pool holds at
    // least one block), so every load is valid and the masks drop them.
    const uint64_t k_base = (uint64_t)a.k_pool;
    const uint64_t v_delta = (uint64_t)a.v_pool - k_base;
    uint32_t d_lo = 0, d_hi = 0;
    int d_nv = 0, dbase = -kWave;
    auto open_set = [&](int first) {
      const int j = first + lane;
      const int phys = j < cnt ? trow[j / a.sub] : -1;
      const bool ok = phys >= 0 && phys < a.num_blocks;
      d_nv = ok ? min(a.rows, L - j * a.rows) : 0;
      const uint64_t addr = k_base + (uint64_t)(ok ? phys : 0) * (uint64_t)block_stride +
                            (uint64_t)head_tile + (uint64_t)(j % a.sub) * (uint64_t)sub_bytes;
      d_lo = (uint32_t)addr;
      d_hi = (uint32_t)(addr >> 32);
    };
    // Lane offsets.  An 8-row sub-tile (8-token blocks) has no rows 8..15:
    // those lanes read rows 0..7 again (in bounds; their scores and V are
    // masked since no sub-tile stores more than `rows` tokens).
    uint32_t kro[D / 32];
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
      kro[m] = (uint32_t)(((lane & 15) & (a.rows - 1)) * 64 + (lane >> 4) * 16 + m * a.rows * 64);
    const uint32_t vro = (uint32_t)(((lane >> 4) & (a.rows / 4 - 1)) * (D * 8) + (lane & 15) * 8);

    // One fragment buffer, refilled in phases: the next pair's K as soon as
    // this pair's S^T products are issued, its V once the P.V products are.
    FragPair<Tag, D> f;
    int nv[2] = {0, 0};
    uint64_t ka = 0, kb = 0;
    auto locate_pair = [&](int P, int* n2) {
      const int s0 = 2 * P;
      if (s0 - dbase >= kWave) {
        dbase += kWave;
        open_set(dbase);
      }
      const int i = s0 - dbase;
      ka = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(d_hi, i) << 32) |
           (uint32_t)__builtin_amdgcn_readlane(d_lo, i);
      kb = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(d_hi, i + 1) << 32) |
           (uint32_t)__builtin_amdgcn_readlane(d_lo, i + 1);
      n2[0] = __builtin_amdgcn_readlane(d_nv, i);
      n2[1] = __builtin_amdgcn_readlane(d_nv, i + 1);
    };
    const int np = (cnt + 1) / 2;
    if (np > 0) {
      locate_pair(0, nv);
      f.load_k((gchar)ka, (gchar)kb, kro);
      f.load_v((gchar)(ka + v_delta), (gchar)(kb + v_delta), vro);
    }
    for (int P = 0; P < np; ++P) {
      const bool more = P + 1 < np;
      int nn[2] = {0, 0};
      f32x4 sa[NQ], sb[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) qk_pair<Tag, D>(f, qf[q], sa[q], sb[q]);
      if (more) {
        locate_pair(P + 1, nn);
        f.load_k((gchar)ka, (gchar)kb, kro);
      }
      if (nv[0] > 0 || nv[1] > 0) {
        if (nv[0] < kRows || nv[1] < kRows) mask_v_tails(f, nv[0], nv[1], lane);
        const int key0 = 2 * P * a.rows;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          softmax_pv<Tag, D>(f, sa[q], sb[q], st[q], nv[0], nv[1], qk_scale, lane,
                             pos[q] - key0 + 1, pos[q] - key0 - a.rows + 1);
      }
      if (more) f.load_v((gchar)(ka + v_delta), (gchar)(kb + v_delta), vro);
      nv[0] = nn[0];
      nv[1] = nn[1];
    }
  } else {
    Frag<Tag, D> fa, fb;
    int nva = 0, nvb = 0;
    auto load_into = [&](Frag<Tag, D>& f, int i, int& nv) {
      int64_t off;
      int bytes;
      locate(i, off, bytes, nv);
      f.template load<kPolicyCached>(tile_rsrc(a.k_pool + off, bytes),
                                     tile_rsrc(a.v_pool + off, bytes), lane, a.rows);
    };
    using CT = typename ComputeTag<Tag>::type;
    auto attend = [&](const Frag<Tag, D>& f, int nv, int i) {
      if (nv <= 0) return;
      const int key0 = (c0 + i) * a.rows;
      const Frag<CT, D> w = compute_regs(f);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        attend_block<CT, D>(w, qf[q], st[q], nv, qk_scale, lane, pos[q] - key0 + 1);
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
  }

  // Normalise and store: acc[k][r] is output dim out_dim(k, r) of the lane's column.
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float l_tot = xor_sum(st[q].l);
    const int t = row0 + q * a.tpg + cr;
    if (!(col_ok && t < row_end)) continue;
    const float inv = (has[q] && l_tot > 0.f) ? v_scale / l_tot : 0.f;
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
