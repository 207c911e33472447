// Single-query paged decode attention for gfx950 (MI355X).
//
// What it computes: for sequence i, query head h (KV head g = h / G) and the
// L_i tokens stored through block table i,
//     out[i][h] = sum_t softmax_t(scale * q[i][h] . K_i[t][g]) V_i[t][g],
// with K_i[t] read at offset t % b of physical block table_i[t / b] (b-token
// blocks, b = 8, 16 or 32)
// ("vLLM and PagedAttention: Virtual Memory for LLM Serving", paragraph 3:
// the kernel reads through the block table and token order stays correct;
// "Inside vLLM and TGI: Paging, Versioned Schedulers and Operations",
// section "Block addresses and fragmentation arithmetic").  The pages give
// neither the formula nor a kernel; this is ordinary scaled dot-product
// attention, computed with a running (online) softmax.
//
// Work decomposition.  A workgroup of 4 wavefronts owns one work unit:
// (KV head g, sequence i, partition p) where a partition is `ps`
// consecutive positions (the whole sequence when ps covers it).  Wavefront w
// takes the w-th contiguous quarter of the unit's blocks (on a pool where a
// sequence holds consecutive blocks, four wavefronts reading neighbouring
// blocks at the same moment ran 7 % slower than four reading far apart).
// Per block it
//   1. takes its address and stored count from registers built once for up
//      to 64 blocks (one per lane) and broadcast with readlane,
//   2. loads the K tile (4 KiB: 4 x 1 KiB fully contiguous dwordx4 loads per
//      wavefront, for 16 x 128 16-bit elements) and the V tile (8 x 512 B
//      contiguous dwordx2 loads), one block ahead of the computation,
//   3. S[t][h] = K[t] . q[h] on the matrix cores: v_mfma_f32_16x16x32 with the
//      16 tokens of the tile as rows and the G <= 16 query heads of the group
//      as columns (rows of q beyond G are zero), accumulated over head_dim,
//   4. online softmax on the 16 x G scores (wavefront max across the four
//      16-lane rows), in the log2 domain,
//   5. acc[d][h] += V^T[d][t] P[t][h], again v_mfma_f32_16x16x32, whose B
//      operand is exactly the register layout S came out in: P is split into
//      a high and a low 16-bit part (P = hi + lo to about 2^-17), placed in the
//      two halves of the k dimension against a duplicated V fragment, so the
//      products keep fp32-level accuracy.
// The four wavefronts' (m, l, acc) are merged in LDS; a single-partition unit
// writes the normalised output, otherwise (m, l, o / l) partials go to the
// workspace and a reduce kernel rescales them by exp2(m_p - max m).
//
// fp32 pools use v_mfma_f32_16x16x4_f32 in the same roles (one k per lane).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pa_tile.h"

namespace pa {

#ifndef PA_WAVES
#define PA_WAVES 4
#endif
constexpr int kWaves = PA_WAVES;
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  char* k_pool;        // written only by the fused step (the current token)
  char* v_pool;
  const char* k_new;   // fused step: current token's K/V per sequence, else null
  const char* v_new;
  int64_t new_stride;  // elements between sequences in k_new / v_new
  int32_t stage_off;   // LDS byte offset of the staged current token
  const char* q;
  void* out;
  const int32_t* tables;
  const int32_t* lens;
  float* part;         // split partials: one record per (seq, KV head, partition):
                       // o/l [G][D], then m [G], then l [G], padded to 128 bytes
  int32_t part_stride; // floats per record
  int32_t num_blocks;
  int32_t block_size;  // tokens per block: 8, 16 or 32
  int32_t rows;        // tokens per 16-row sub-tile: min(block_size, 16)
  int32_t sub;         // sub-tiles per block: block_size / rows
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t group;       // G = Hq / Hkv
  int32_t num_seqs;
  int32_t max_blocks;  // table row width
  int32_t max_len;     // clip for lengths
  int32_t ps;          // partition size in tokens (a multiple of the block size)
  int32_t num_parts;   // P = ceil(max_len / ps); planned split: units per KV head
  int32_t longest_first;  // 1: map workgroups to sequences in decreasing length
  int32_t planned;     // 1: split planned from the lengths (automatic partitioning)
  int32_t part_shift;  // planned split: log2 of tokens per tile (16 when 8-token blocks pair up)
  int32_t min_tiles;   // planned split: smallest unit worth its start-up, in tiles
  int32_t* plan_hdr;   // planned split: per sequence {record index of unit 0, units}
  float qk_scale;      // scale * log2(e)
  const float* k_scales;  // FP8 pools: per-KV-head scales, else null
  const float* v_scales;
};

// Longest-first dispatch.  Workgroups start roughly in blockIdx order, so
// giving consecutive indices to sequences in decreasing length (longest
// processing time first) keeps the last workgroups to finish short.  Each
// workgroup finds the sequence of rank r itself by counting: a histogram of
// block counts (descending; counts >= kRankBins - 1 share the last bin) in
// LDS, a prefix scan that locates the bin holding rank r, then the position
// within that bin in index order (ballots).  About six barriers and
// O(S / threads + kRankBins / threads) work per thread.
constexpr int kRankBins = 2048;
constexpr int kRankLdsInts = kRankBins + kWaves + 4;
// Up to this many sequences, ranking by pairwise comparison (O(S^2 / threads),
// two barriers) is cheaper than the counting selection's fixed cost.
#ifndef PA_PAIRWISE_RANK_MAX
#define PA_PAIRWISE_RANK_MAX 128
#endif
constexpr int kPairwiseRankMax = PA_PAIRWISE_RANK_MAX;



// A stored length as attended: clipped to [0, max_len] and to what a table
// row can address.
__device__ inline int clip_stored(const DecodeArgs& a, int L) {
  L = L < 0 ? 0 : L;
  L = L > a.max_len ? a.max_len : L;
  const int64_t cap = (int64_t)a.max_blocks * a.block_size;
  return (int64_t)L > cap ? (int)cap : L;
}
__device__ inline int clip_len(const DecodeArgs& a, int i) { return clip_stored(a, a.lens[i]); }

// Lengths are ranked in bins of 2^PA_RANK_SHIFT 16-token tiles (128 tokens),
// and sequences of one bin keep their batch order: the forks of one request,
// which share their prompt's blocks and sit side by side in the batch, then
// run at the same time and share those tiles in L2 (measured on 32 x 8 forks
// of a 1024-token prompt: 183 -> 129 us with cached loads for shared units,
// below; exact ranking: 142 us; the batch-256 GQA step unchanged).
#ifndef PA_RANK_SHIFT
#define PA_RANK_SHIFT 3
#endif
__device__ inline int bin_of_stored(const DecodeArgs& a, int stored) {
  const int L = clip_stored(a, stored);
  int nb = ((L + kRows - 1) / kRows) >> PA_RANK_SHIFT;   // work measure: 16-token sub-tiles
  nb = nb > kRankBins - 1 ? kRankBins - 1 : nb;
  return kRankBins - 1 - nb;                   // longest first
}
__device__ inline int rank_bin(const DecodeArgs& a, int i) { return bin_of_stored(a, a.lens[i]); }

// Both rankings return (sequence, its stored length as read while ranking):
// the unit then needs no second read of the length before its first table
// load (under a full memory pipeline each dependent read costs microseconds).

__device__ inline int2 seq_of_rank(const DecodeArgs& a, int r, int* lds) {
  static_assert(kRankBins % kThreads == 0, "bins per thread");
  constexpr int kPer = kRankBins / kThreads;
  int* hist = lds;
  int* scratch = lds + kRankBins;              // [kWaves] partial counts, then results
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int w = t / kWave;
  const int S = a.num_seqs;
#pragma unroll
  for (int b = 0; b < kPer; ++b) hist[t * kPer + b] = 0;
  __syncthreads();
  // Each thread's first sequence's bin, kept for the final pass: one round
  // of length reads per workgroup when S <= kThreads (about 1 us at the start
  // of a launch, several under a full memory pipeline).
  const int my_len = t < S ? a.lens[t] : 0;
  const int my_bin = t < S ? bin_of_stored(a, my_len) : -1;
  if (t < S) atomicAdd(&hist[my_bin], 1);
  for (int i = t + kThreads; i < S; i += kThreads) atomicAdd(&hist[rank_bin(a, i)], 1);
  __syncthreads();
  // Exclusive prefix of the bin counts, kPer bins per thread.
  int c = 0;
#pragma unroll
  for (int b = 0; b < kPer; ++b) c += hist[t * kPer + b];
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) scratch[w] = incl;
  __syncthreads();
  int before = incl - c;
  for (int v = 0; v < w; ++v) before += scratch[v];
  if (r >= before && r < before + c) {         // the one thread whose bins hold rank r
    int acc = before;
    for (int b = 0; b < kPer; ++b) {
      const int h = hist[t * kPer + b];
      if (r < acc + h) {
        scratch[kWaves] = t * kPer + b;
        scratch[kWaves + 1] = r - acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
  const int bin = scratch[kWaves];
  int within = scratch[kWaves + 1];
  __syncthreads();
  // The `within`-th sequence (by index) of that bin.
  for (int base = 0; base < S; base += kThreads) {
    const int i = base + t;
    const int len_i = base == 0 ? my_len : i < S ? a.lens[i] : 0;
    const bool hit = i < S && (base == 0 ? my_bin : bin_of_stored(a, len_i)) == bin;
    const unsigned long long m = __ballot(hit);
    if (lane == 0) scratch[w] = __popcll(m);
    __syncthreads();
    int wbefore = 0, total = 0;
    for (int v = 0; v < kWaves; ++v) {
      wbefore += v < w ? scratch[v] : 0;
      total += scratch[v];
    }
    if (within < total) {                      // uniform across the workgroup
      const int mine = wbefore + __popcll(m & ((1ull << lane) - 1ull));
      if (hit && mine == within) {
        scratch[kWaves + 2] = i;
        scratch[kWaves + 3] = len_i;
      }
      __syncthreads();
      const int2 found = make_int2(scratch[kWaves + 2], scratch[kWaves + 3]);
      __syncthreads();                         // LDS is reused afterwards
      return found;
    }
    within -= total;
    __syncthreads();
  }
  return make_int2(0, 0);                      // not reached: r < S
}

// rank(i) = #{j : key_j > key_i} with unique keys (block count, then lower index).
// LDS: keys [0, S), the result at kPairwiseRankMax and +1, lengths from +2.
__device__ inline int2 seq_of_rank_pairwise(const DecodeArgs& a, int r, int* lds) {
  static_assert(2 * kPairwiseRankMax + 2 <= kRankLdsInts, "pairwise ranking's LDS");
  const int S = a.num_seqs;
  int* lens = lds + kPairwiseRankMax + 2;
  for (int i = threadIdx.x; i < S; i += kThreads) {
    const int len = a.lens[i];
    lens[i] = len;
    lds[i] = ((kRankBins - 1 - bin_of_stored(a, len)) << 12) | (4095 - i);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < S; i += kThreads) {
    const int ki = lds[i];
    int rank = 0;
    for (int j = 0; j < S; ++j) rank += lds[j] > ki ? 1 : 0;
    if (rank == r) {
      lds[kPairwiseRankMax] = i;
      lds[kPairwiseRankMax + 1] = lens[i];
    }
  }
  __syncthreads();
  const int2 found = make_int2(lds[kPairwiseRankMax], lds[kPairwiseRankMax + 1]);
  __syncthreads();
  return found;
}

// ---- planned split (automatic partitioning) ----
// When the (sequence, KV head) pairs are fewer than the resident workgroups,
// each sequence's tiles are split into units sized from the lengths: a
// sequence of n tiles gets ceil(n / u) units (one if it is empty), each a
// near-equal range of its tiles, where u is the smallest tile count of at
// least min_tiles for which one KV head's units number at most num_parts.
// This divisor rule gives the smallest largest unit for that many units, so
// the grid is one round of units of nearly equal work.  Every wavefront of
// the partition kernel derives the same plan from the lengths; the unit that
// starts a sequence's first KV head leaves the sequence's (first record,
// units) in a header for the combine kernel.  Reductions are DPP sums.
__device__ inline int plan_tiles_of(const DecodeArgs& a, int L) {
  return (L + (1 << a.part_shift) - 1) >> a.part_shift;
}
__device__ inline int plan_tiles(const DecodeArgs& a, int i) { return plan_tiles_of(a, clip_len(a, i)); }

// Units of a sequence of n tiles under unit size u, capped at num_parts + 1
// (only comparisons with num_parts are made; the cap keeps sums in range).
__device__ inline int plan_units(const DecodeArgs& a, int n, int u) {
  const int c = n <= u ? 1 : (n - 1) / u + 1;
  return c > a.num_parts ? a.num_parts + 1 : c;
}

// One KV head's units under unit size u (n0: the tiles of sequence `lane`).
__device__ inline int plan_count(const DecodeArgs& a, int n0, int u, int lane) {
  int c = lane < a.num_seqs ? plan_units(a, n0, u) : 0;
  for (int i = kWave + lane; i < a.num_seqs; i += kWave) c += plan_units(a, plan_tiles(a, i), u);
  return __reduce_add_sync(~0ull, c);
}

// Unit size u of the plan.  L0 receives the length of sequence `lane` (the
// first 64 sequences stay in registers across the search).
__device__ inline int plan_unit_size(const DecodeArgs& a, int lane, int& L0) {
  const int S = a.num_seqs;
  L0 = lane < S ? clip_len(a, lane) : 0;
  const int n0 = plan_tiles_of(a, L0);
  // The total in 16-bit halves: each half's 32-bit sum cannot overflow.
  int lo16 = n0 & 0xffff, hi16 = n0 >> 16, mx = n0;
  for (int i = kWave + lane; i < S; i += kWave) {
    const int n = plan_tiles(a, i);
    lo16 += n & 0xffff;
    hi16 += n >> 16;
    mx = max(mx, n);
  }
  const int tot_hi = __reduce_add_sync(~0ull, hi16), tot_lo = __reduce_add_sync(~0ull, lo16);
  mx = __reduce_max_sync(~0ull, mx);
  int lo;
  if (tot_hi < 0x7c00) {                       // the total fits 31 bits: 32-bit division
    lo = (int)(((unsigned)tot_hi << 16) + (unsigned)tot_lo);
    lo = (int)(((unsigned)lo + a.num_parts - 1) / (unsigned)a.num_parts);
  } else {
    lo = (int)(((int64_t)tot_hi * 65536 + tot_lo + a.num_parts - 1) / a.num_parts);
  }
  lo = max(lo, a.min_tiles);
  int hi = max(lo, mx);
  if (hi > lo && plan_count(a, n0, lo, lane) <= a.num_parts) hi = lo;   // the floor fits
  while (lo < hi) {                            // smallest u with count(u) <= num_parts
    const int mid = lo + ((hi - lo) >> 1);
    if (plan_count(a, n0, mid, lane) <= a.num_parts) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

struct PlanUnit {
  int seq;     // -1: past the plan's last unit
  int part;    // unit index within the sequence
  int count;   // units of the sequence
  int first;   // record index of the sequence's unit 0 among its KV head's records
  int len;     // the sequence's clipped length
};

// Unit r of one KV head: units are numbered sequence by sequence.
__device__ inline PlanUnit plan_locate(const DecodeArgs& a, int L0, int u, int r, int lane) {
  const int S = a.num_seqs;
  int base = 0;
  for (int c = 0; c < S; c += kWave) {
    const int i = c + lane;
    const int Li = c == 0 ? L0 : (i < S ? clip_len(a, i) : 0);
    const int np = i < S ? plan_units(a, plan_tiles_of(a, Li), u) : 0;
    int incl = np;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const unsigned long long hit = __ballot(base + incl > r);
    if (hit) {
      // Lane values, made scalar: they stay live to the end of the kernel.
      const int l = __builtin_ctzll(hit);
      const int excl = __builtin_amdgcn_readlane(incl - np, l);
      return {c + l, r - base - excl, __builtin_amdgcn_readlane(np, l), base + excl,
              __builtin_amdgcn_readlane(Li, l)};
    }
    base += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return {-1, 0, 0, 0, 0};
}


// The fused step writes the current token (offset o of its block) to the pool
// and, for the one block that holds it, replaces the loaded values of that
// token with the staged copy -- the tile load may have raced the store.
// Perm: the dimension order of FP8 storage (see Frag<TagFP8>).
template <class Tag, int D, bool Perm = false>
__device__ inline void patch_token(Frag<Tag, D, true>& f, const char* stage, int o, int lane) {
  if ((lane & 15) == o) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const int dim0 = Perm ? (lane >> 4) * (D / 4) + 8 * m : 8 * (4 * m + (lane >> 4));
      f.k[m] = *reinterpret_cast<const u32x4*>(stage + dim0 * 2);
    }
  }
  // Element indices below are runtime values: select, never index registers
  // dynamically (that would move the fragment to scratch memory).
  if ((lane >> 4) == (o >> 2)) {
    const int dl = lane & 15;
    const int shift = (o & 1) * 16;
    const uint32_t keep = ~(0xffffu << shift);
    const bool second = (o & 2) != 0;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const int dim = Perm ? dl * (D / 16) + n : 16 * n + dl;
      const uint32_t val = *reinterpret_cast<const uint16_t*>(stage + D * 2 + dim * 2);
      const uint32_t w0 = f.v[n][0], w1 = f.v[n][1];
      f.v[n][0] = second ? w0 : (w0 & keep) | (val << shift);
      f.v[n][1] = second ? (w1 & keep) | (val << shift) : w1;
    }
  }
}
template <class Tag, int D, bool Perm = false>
__device__ inline void patch_token(Frag<Tag, D, false>& f, const char* stage, int o, int lane) {
  if ((lane & 15) == o) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
      f.k[j] = *reinterpret_cast<const f32x4*>(stage + (4 * j + (lane >> 4)) * 16);
  }
  if ((lane >> 4) == (o >> 2)) {
    const int dl = lane & 15;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const float val = *reinterpret_cast<const float*>(stage + D * 4 + (16 * n + dl) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) f.v[n][e] = (e == (o & 3)) ? val : f.v[n][e];
    }
  }
}

// FP8: the same patch on the raw codes (stage: K codes then V codes, dim
// order; the fragment roles of Frag<TagFP8>: K lane (t, g) k[m] = dims
// g*D/4 + 8m .. +7 of row t; V lane (r, tg) v[n] = 4 tokens of dim r*D/16 + n).
template <int D>
__device__ inline void patch_token_codes(Frag<TagFP8, D, true>& f, const char* stage, int o,
                                         int lane) {
  if ((lane & 15) == o) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
      f.k[m] = *reinterpret_cast<const u32x2*>(stage + (lane >> 4) * (D / 4) + 8 * m);
  }
  if ((lane >> 4) == (o >> 2)) {
    const int shift = 8 * (o & 3);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const uint32_t code = (uint8_t)stage[D + (lane & 15) * (D / 16) + n];
      f.v[n] = (f.v[n] & ~(0xFFu << shift)) | (code << shift);
    }
  }
}

// The current token's K/V for KV head g: loaded into registers when the
// workgroup starts (one 16-byte vector per thread), staged in LDS once the
// first blocks are in flight (for patch_token), and stored to its slot after
// the block loop -- K as 16-byte vectors (four 64-byte pieces in four lines
// for 128 bf16 dims), V as elements interleaved by 4 tokens (eight lines).
// Writes cost per line touched while reads stream.
template <class Tag, int D> struct NewToken {
  static constexpr int ES = Is16<Tag>::value ? 2 : 4;
  static constexpr int X = 16 / ES;
  static constexpr int NC = D / X;            // 16-byte vectors per head row
  u32x4 vec;

  __device__ inline void load(const DecodeArgs& a, int seq, int g) {
    const int t = threadIdx.x;
    if (t < 2 * NC) {
      const bool is_v = t >= NC;
      const int c = is_v ? t - NC : t;
      const char* src = (is_v ? a.v_new : a.k_new) +
                        ((int64_t)seq * a.new_stride + (int64_t)g * D) * ES;
      vec = *reinterpret_cast<const u32x4*>(src + c * 16);
    }
  }

  __device__ inline void stage(char* stage) const {
    const int t = threadIdx.x;
    if (t >= 2 * NC) return;
    const bool is_v = t >= NC;
    const int c = is_v ? t - NC : t;
    *reinterpret_cast<u32x4*>(stage + (is_v ? D * ES : 0) + c * 16) = vec;
  }

  // j: table entry of the block holding the token, o: its offset in the block.
  __device__ inline void store(const DecodeArgs& a, const int32_t* trow, int j, int g,
                               int o) const {
    const int64_t kTile = (int64_t)a.block_size * D * ES;
    const int t = threadIdx.x;
    if (t >= 2 * NC) return;
    const int phys = trow[j];
    if (phys < 0 || phys >= a.num_blocks) return;
    const bool is_v = t >= NC;
    const int c = is_v ? t - NC : t;
    char* tile = (is_v ? a.v_pool : a.k_pool) + ((int64_t)phys * a.num_kv_heads + g) * kTile;
    if (!is_v) {
      if constexpr (ES == 2)
        *reinterpret_cast<u32x4*>(tile + k16_offset(o, c * X, a.block_size, D)) = vec;
      else
        *reinterpret_cast<u32x4*>(tile + ((int64_t)o * D + c * X) * ES) = vec;
    } else {
      char* vb = tile + ((int64_t)(o >> 2) * D * 4 + (o & 3)) * ES;
#pragma unroll
      for (int e = 0; e < X; ++e) {
        const int d = c * X + e;
        if constexpr (ES == 4)
          *reinterpret_cast<uint32_t*>(vb + (int64_t)d * 4 * ES) = vec[e];
        else
          *reinterpret_cast<uint16_t*>(vb + (int64_t)d * 4 * ES) =
              (uint16_t)(vec[e >> 1] >> ((e & 1) * 16));
      }
    }
  }

};

// FP8 pools: the bf16 current token is quantized with its head's scales when
// loaded; the stage holds the dequantized codes (what a read of the pool
// returns, unscaled), and the store writes the codes at the FP8 tile
// layout's offsets -- K as one 8-byte piece per thread, V as bytes.
template <int D> struct NewToken<TagFP8, D> {
  static constexpr int NC = D / 8;            // 16-byte bf16 input vectors per head row
  uint32_t code[2];                           // the thread's 8 E4M3 codes

  __device__ inline void load(const DecodeArgs& a, int seq, int g) {
    const int t = threadIdx.x;
    if (t < 2 * NC) {
      const bool is_v = t >= NC;
      const int c = is_v ? t - NC : t;
      const char* src = (is_v ? a.v_new : a.k_new) +
                        ((int64_t)seq * a.new_stride + (int64_t)g * D) * 2;
      const u32x4 vec = *reinterpret_cast<const u32x4*>(src + c * 16);
      const float scale = is_v ? a.v_scales[g] : a.k_scales[g];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * w + j;
          const float f = bf16_bits_to_float((vec[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
          x |= fp8_code(f, scale) << (8 * j);
        }
        code[w] = x;
      }
    }
  }

  // The stage holds the codes: K's D bytes, then V's D bytes (dim order).
  __device__ inline void stage(char* stage) const {
    const int t = threadIdx.x;
    if (t >= 2 * NC) return;
    const bool is_v = t >= NC;
    const int c = is_v ? t - NC : t;
    *reinterpret_cast<u32x2*>(stage + (is_v ? D : 0) + c * 8) = u32x2{code[0], code[1]};
  }

  __device__ inline void store(const DecodeArgs& a, const int32_t* trow, int j, int g,
                               int o) const {
    const int64_t kTile = (int64_t)a.block_size * D;
    const int t = threadIdx.x;
    if (t >= 2 * NC) return;
    const int phys = trow[j];
    if (phys < 0 || phys >= a.num_blocks) return;
    const bool is_v = t >= NC;
    const int c = is_v ? t - NC : t;
    char* tile = (is_v ? a.v_pool : a.k_pool) + ((int64_t)phys * a.num_kv_heads + g) * kTile;
    if (!is_v) {
      // 8 consecutive dims from a multiple of 8: contiguous in a 16-byte piece
      *reinterpret_cast<u32x2*>(tile + fp8_k_offset(o, c * 8, a.block_size, D)) =
          u32x2{code[0], code[1]};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tile[fp8_v_offset(o, c * 8 + e, a.block_size, D)] =
            (char)((code[e >> 2] >> (8 * (e & 3))) & 0xFFu);
    }
  }
};

// One workgroup per (KV head, sequence, partition); see the file comment.
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 3
#endif

#ifndef PA_FP8_WAVES_PER_EU
#define PA_FP8_WAVES_PER_EU 4
#endif

// Occupancy target: 3 wavefronts per SIMD (<= 168 VGPRs) keeps a block in
// flight per wavefront on top of the one being computed; fp32 tiles of 128
// dims need twice the fragment registers, so they run at 2.  FP8 tiles keep
// raw codes (half the registers) widened chunk by chunk, which fits 4
// wavefronts per SIMD (<= 128 VGPRs): measured 2-3 % faster than 3
// wavefronts with a deeper ring.
template <class Tag, int D> struct WavesPerEU {
  static constexpr int value = (!Is16<Tag>::value && D == 128) ? 2
                               : IsFP8<Tag>::value             ? PA_FP8_WAVES_PER_EU
                                                               : PA_WAVES_PER_EU;
};

// 8-token blocks, 16-bit pools: two blocks fill one 16-row tile -- rows 0-7
// from block a, rows 8-15 from block b (each lane's K pieces come from the
// block of its row; V token groups 0-1 from a, 2-3 from b) -- with streaming
// global loads from per-lane addresses, so one load instruction covers whole
// lines of both blocks instead of half a tile.  ka, kb: the blocks' K tiles of
// this KV head; their V tiles are v_delta further.
template <class Tag, int D, bool Cached = false>
__device__ inline void load_pair8(Frag<Tag, D, true>& f, uint64_t ka, uint64_t kb,
                                  uint64_t v_delta, int lane) {
  typedef const __attribute__((address_space(1))) u32x4* g16;
  typedef const __attribute__((address_space(1))) u32x2* g8;
  const uint64_t kl = ((lane & 15) < 8 ? ka : kb) + (uint32_t)((lane & 7) * 64 + (lane >> 4) * 16);
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
    f.k[m] = Cached ? *(g16)(kl + m * 8 * 64) : __builtin_nontemporal_load((g16)(kl + m * 8 * 64));
  const uint64_t vl = ((lane >> 4) < 2 ? ka : kb) + v_delta +
                      (uint32_t)(((lane >> 4) & 1) * (D * 8) + (lane & 15) * 8);
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    f.v[n] = Cached ? *(g8)(vl + n * 128) : __builtin_nontemporal_load((g8)(vl + n * 128));
}

// 16-row tiles of 16-bit pools (16- and 32-token blocks) read with per-lane
// 64-bit addresses, the same lane roles as Frag::load: the address of each
// load is a vector add, where a buffer load needs the tile's descriptor built
// in scalar registers first (measured 1.5-2 % faster on the 16-bit decode
// workloads).  Every lane's K and V pieces lie inside the 16-row sub-tile at
// ka (and ka + v_delta), so the caller needs only a tile that exists.
template <class Tag, int D, bool Cached>
__device__ inline void load_tile16(Frag<Tag, D, true>& f, uint64_t ka, uint64_t v_delta,
                                   int lane) {
  static_assert(Is16<Tag>::value && !IsFP8<Tag>::value, "16-bit tiles only");
  typedef const __attribute__((address_space(1))) u32x4* g16;
  typedef const __attribute__((address_space(1))) u32x2* g8;
  const uint64_t kl = ka + (uint32_t)((lane & 15) * 64 + (lane >> 4) * 16);
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
    f.k[m] = Cached ? *(g16)(kl + m * kRows * 64) : __builtin_nontemporal_load((g16)(kl + m * kRows * 64));
  const uint64_t vl = ka + v_delta + (uint32_t)((lane >> 4) * (D * 8) + (lane & 15) * 8);
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    f.v[n] = Cached ? *(g8)(vl + n * 128) : __builtin_nontemporal_load((g8)(vl + n * 128));
}

// How a decode kernel instance reads its tiles: buffer loads through a
// per-tile resource (any row count; FP8 and fp32 pools, and 16-bit pools with
// 8-row tiles), pairs of 8-token blocks as one tile (load_pair8), or 16-row
// tiles of 16-bit pools through per-lane addresses (load_tile16).
enum LoadMode : int { kLoadBuffer = 0, kLoadPair8 = 1, kLoadGlobal16 = 2 };

// Cache policy for units whose sequence shares its first block with a
// neighbouring row of the batch (0: stream every unit).
#ifndef PA_SHARED_CACHED
#define PA_SHARED_CACHED 1
#endif

// Register buffers in the block ring (one block ahead of the one being
// computed); FP8 runs more wavefronts per SIMD instead of a deeper ring.
#ifndef PA_FP8_BUFS
#define PA_FP8_BUFS 2
#endif
template <class Tag> struct RingBufs { static constexpr int value = IsFP8<Tag>::value ? PA_FP8_BUFS : 2; };

// LM: the tile loads (LoadMode).  kLoadPair8: 8-token blocks of a 16-bit
// pool, walked as 16-token tiles of two blocks; `rows` below is then 16 while
// a block holds 8.
template <class Tag, int D, class OutT, int LM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEU<Tag, D>::value)))
void decode_kernel(DecodeArgs a) {
  constexpr bool P8 = LM == kLoadPair8;
  static_assert(LM != kLoadGlobal16 || (Is16<Tag>::value && !IsFP8<Tag>::value),
                "per-lane tile addresses are for 16-bit pools");
  constexpr int NBuf = RingBufs<Tag>::value;
  extern __shared__ float smem[];
  constexpr int ES = Elt<Tag>::bytes;
  // A block of 32 tokens is two 16-row sub-tiles (each contiguous in both
  // tile layouts); a block of 8 is one sub-tile whose rows 8..15 fall outside
  // its buffer resource and read as zero.
  const int64_t tile_bytes = (int64_t)a.block_size * D * ES;
  const int sub_bytes = a.rows * D * ES;
  const int lane = threadIdx.x & (kWave - 1);
  // The wavefront index is uniform; saying so keeps the block loop scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  const int unit = blockIdx.x;
  const int g = unit % a.num_kv_heads;
  const int rest = unit / a.num_kv_heads;
  PlanUnit pu{0, 0, 0, 0, 0};
  if (a.planned) {
    int L0;
    const int u = plan_unit_size(a, lane, L0);
    pu = plan_locate(a, L0, u, rest, lane);
    if (pu.seq < 0) return;                      // the grid's spare units
  }
  // The combine kernel's header of a planned sequence, stored where few
  // registers are live (at exit).
  auto put_header = [&]() {
    if (a.planned && g == 0 && pu.part == 0 && threadIdx.x == 0)
      *reinterpret_cast<int2*>(a.plan_hdr + 2 * pu.seq) = make_int2(pu.first, pu.count);
  };
  const int part = a.planned ? pu.part : rest / a.num_seqs;
  // (sequence, stored length), both uniform; a negative length field means
  // the length was not read by a ranking (or is itself negative, which
  // clips to 0) and is read here.
  int2 sr = make_int2(a.planned ? pu.seq : rest % a.num_seqs, -1);
  if (!a.planned && a.longest_first)
    sr = a.num_seqs <= kPairwiseRankMax
             ? seq_of_rank_pairwise(a, rest % a.num_seqs, reinterpret_cast<int*>(smem))
             : seq_of_rank(a, rest % a.num_seqs, reinterpret_cast<int*>(smem));
  const int seq = __builtin_amdgcn_readfirstlane(sr.x);
  const int stored = sr.y >= 0 ? __builtin_amdgcn_readfirstlane(sr.y)
                     : a.planned && a.k_new == nullptr ? 0
                                                       : a.lens[seq];

  const int L = a.planned ? pu.len : clip_stored(a, stored);
  const int n_parts = a.planned ? pu.count : (L + a.ps - 1) / a.ps;
  const int G = a.group;
  const int head0 = g * G;

  const int32_t* trow = a.tables + (int64_t)seq * a.max_blocks;
  // Fused step: the current token sits at position lens[seq] - 1, which the
  // three-call form (slot mapping, write, attention) writes whenever the
  // table row reaches it -- also when that position lies beyond the attended
  // length L (a length clipped to max_len).  It joins the attention only when
  // it is attended, i.e. when the length was not clipped.
  const int raw_len = a.k_new != nullptr ? stored : 0;
  const bool store_new = raw_len >= 1 && (raw_len - 1) / a.block_size < a.max_blocks;
  const bool patch_new = store_new && raw_len == L;
  NewToken<Tag, D> tok;

  if (L == 0) {                                  // no tokens: zero output row
    if (part == 0) {
      OutT* o = reinterpret_cast<OutT*>(a.out) + ((int64_t)seq * a.num_q_heads + head0) * D;
      for (int i = threadIdx.x; i < G * D; i += kThreads) store_out<OutT>(o + i, 0.f);
      if (store_new) {                           // a length clipped to zero: still written
        tok.load(a, seq, g);
        tok.store(a, trow, (raw_len - 1) / a.block_size, g, (raw_len - 1) % a.block_size);
      }
    }
    put_header();
    return;
  }
  if (part >= n_parts) return;

  // From here on j counts tiles of `rows` tokens (sub-tiles, or pairs of
  // 8-token blocks when P8).
  const int rows = P8 ? kRows : a.rows;
  const int nsub_seq = (L + rows - 1) / rows;
  const int j0 = a.planned ? (int)((int64_t)part * nsub_seq / n_parts) : part * (a.ps / rows);
  const int j1 = a.planned ? (int)((int64_t)(part + 1) * nsub_seq / n_parts)
                           : min(nsub_seq, j0 + a.ps / rows);
  const int per = (j1 - j0 + kWaves - 1) / kWaves;  // tiles per wavefront: contiguous quarters
  const int first = min(j1, j0 + wave * per);
  const int cnt = max(0, min(j1, first + per) - first);

  const int h = lane & 15;
  QFrag<Tag, D> qf;
  qf.load(a.q + (((int64_t)seq * a.num_q_heads + head0 + (h < G ? h : 0)) * D) * In<Tag>::bytes,
          h < G, lane);
  // FP8: the K scale of the head folds into the score scale, the V scale
  // into the output.
  float qk_scale = a.qk_scale;
  float v_scale = 1.f;
  if constexpr (IsFP8<Tag>::value) {
    qk_scale *= a.k_scales[g];
    v_scale = a.v_scales[g];
  }

  State<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t head_tile = (int64_t)g * tile_bytes;
  const int64_t block_stride = (int64_t)a.num_kv_heads * tile_bytes;

  // Fused step: the unit holding the last attended tile writes the current
  // token (and, when it is attended, at position L-1, patches it in).
  const int j_new = (L - 1) / rows;            // the tile of position L-1
  int o_new = (L - 1) % rows;                  // its register row
  const bool own_new = store_new && j_new >= j0 && j_new < j1;
  const bool own_patch = own_new && patch_new;
  if (P8 && own_patch && o_new >= 8) {         // in block b: it moves up when block a is out
    const int pa_ = trow[2 * j_new];          // of the pool (valid blocks are packed first)
    if (pa_ < 0 || pa_ >= a.num_blocks) o_new -= 8;
  }
  char* stage = reinterpret_cast<char*>(smem) + a.stage_off;
  if (own_new) tok.load(a, seq, g);             // in flight with the first blocks

  // Blocks are processed in chunks of up to 64 per wavefront: one table load
  // per chunk, each id broadcast with readlane.
  using CT = typename ComputeTag<Tag>::type;
  Frag<Tag, D> f[NBuf];
  int nv[NBuf];
  int c0 = 0, n = 0;
  // Per-lane descriptors of the chunk's blocks, lane i for block i: the K
  // address of its sub-tile and its valid-token count (0 for a table entry
  // outside the pool, negated for the block that holds the current token,
  // which is patched first).  A block is then a lane broadcast, not address
  // arithmetic.  Blocks past the wavefront's last one (the ring's prefetch)
  // get count 0 and a size-0 resource: no memory access, static wait counts
  // (pair and per-lane-address loads read block 0's tile of the head instead,
  // see open_table).
  const uint64_t k_base = (uint64_t)a.k_pool;
  const uint64_t v_delta = (uint64_t)a.v_pool - k_base;
  const int sub_shift = a.sub >> 1;          // sub-tiles per block: 1 or 2
  uint32_t d_lo = 0, d_hi = 0, d_lo2 = 0, d_hi2 = 0;   // d_*2: block b when P8
  int d_nv = 0;
  // cached_c: std::true_type when this unit's tiles go through the caches.
  auto load_into = [&](auto cached_c, Frag<Tag, D>& fr, int i, int& nvr) {
    constexpr bool Cached = decltype(cached_c)::value;
    const int li = min(i, kWave - 1);
    nvr = i < n ? __builtin_amdgcn_readlane(d_nv, li) : 0;
    const uint64_t ka = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(d_hi, li) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane(d_lo, li);
    if constexpr (P8) {
      const uint64_t kb = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(d_hi2, li) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane(d_lo2, li);
      load_pair8<Tag, D, Cached>(fr, ka, kb, v_delta, lane);
    } else if constexpr (LM == kLoadGlobal16) {
      load_tile16<Tag, D, Cached>(fr, ka, v_delta, lane);
    } else {
      const int bytes = nvr != 0 ? sub_bytes : 0;
      fr.template load<Cached ? kPolicyCached : kKvCachePolicy>(
          tile_rsrc((const char*)ka, bytes), tile_rsrc((const char*)(ka + v_delta), bytes), lane,
          a.rows);
    }
  };
  auto attend_regs = [&](Frag<CT, D>& w, int nvr) {
    if (nvr < 0) {
      patch_token<CT, D, IsFP8<Tag>::value>(w, stage, o_new, lane);
      nvr = -nvr;
    }
    if (nvr > 0) attend_block<CT, D>(w, qf, st, nvr, qk_scale, lane);
  };
  auto attend = [&](Frag<Tag, D>& fr, int nvr) {
    if constexpr (IsFP8<Tag>::value) {
      // Codes are widened chunk by chunk at their matrix products; the tile
      // holding the current token gets the staged codes patched in first.
      if (nvr < 0) {
        patch_token_codes<D>(fr, stage, o_new, lane);
        nvr = -nvr;
      }
      if (nvr > 0) attend_block_fp8<D>(fr, qf, st, nvr, qk_scale, lane);
    } else {
      attend_regs(fr, nvr);
    }
  };
  // The chunk's table entries and tile descriptors (no tile loads).
  int t_a = -1, t_b = -1;                      // this lane's table entries (P8: two)
  auto read_table = [&]() {
    n = min(kWave, cnt - c0);
    const int j = first + c0 + lane;
    if constexpr (P8) {
      t_a = lane < n ? trow[2 * j] : -1;
      t_b = lane < n && (2 * j + 1) * 8 < L ? trow[2 * j + 1] : -1;
    } else {
      t_a = lane < n ? trow[j >> sub_shift] : -1;
    }
  };
  auto open_table = [&]() {
    const int j = first + c0 + lane;
    if constexpr (P8) {
      // Blocks 2j and 2j+1.  Decode has no causal order, so valid blocks are
      // packed first and the tile's valid rows stay a prefix: block a out of
      // the pool -> block b takes rows 0-7.  Missing blocks, and tiles past
      // the wavefront's last (the ring's prefetch), read block 0's tile of
      // this head (in bounds; shared by every such read, so it stays cached)
      // and are masked by the count.
      const int pa_ = t_a, pb_ = t_b;
      const bool oka = pa_ >= 0 && pa_ < a.num_blocks;
      const bool okb = pb_ >= 0 && pb_ < a.num_blocks;
      const int ca = oka ? min(8, L - 16 * j) : 0;
      const int cb = okb ? min(8, L - 16 * j - 8) : 0;
      int c = ca + cb;
      if (own_patch && j == j_new) c = -c;
      d_nv = c;
      const int first_blk = oka ? pa_ : (okb ? pb_ : 0);
      const int second_blk = oka && okb ? pb_ : 0;
      const uint64_t a0 = k_base + (uint64_t)head_tile;
      const uint64_t aa = a0 + (uint64_t)first_blk * (uint64_t)block_stride;
      const uint64_t ab = a0 + (uint64_t)second_blk * (uint64_t)block_stride;
      d_lo = (uint32_t)aa;
      d_hi = (uint32_t)(aa >> 32);
      d_lo2 = (uint32_t)ab;
      d_hi2 = (uint32_t)(ab >> 32);
    } else {
      const int phys = t_a;
      const bool ok = phys >= 0 && phys < a.num_blocks;
      int c = ok ? min(a.rows, L - j * a.rows) : 0;
      if (own_patch && j == j_new) c = -c;
      d_nv = c;
      // Entries outside the pool and lanes past the chunk address block 0
      // (in the pool: what per-lane-address loads need; buffer loads give
      // them a size-0 resource).
      const uint64_t addr = k_base + (uint64_t)(ok ? phys : 0) * (uint64_t)block_stride +
                            (uint64_t)head_tile + (uint64_t)(j & (a.sub - 1)) * (uint64_t)sub_bytes;
      d_lo = (uint32_t)addr;
      d_hi = (uint32_t)(addr >> 32);
    }
  };
  // The ring's first NBuf - 1 tiles of the chunk.
  auto prefetch = [&](auto cached_c) {
#pragma unroll
    for (int u = 0; u + 1 < NBuf; ++u) load_into(cached_c, f[u], u, nv[u]);
  };

  // The block loop, compiled for each cache policy (one policy per unit keeps
  // the loads unconditional and their wait counts static).
  auto block_loop = [&](auto cached_c) {
    if (cnt > 0) {
      open_table();
      prefetch(cached_c);
    }
    if (own_patch) {                            // every wavefront reaches this barrier
      tok.stage(stage);
      __syncthreads();
    }
  // A ring of NBuf register buffers, NBuf - 1 blocks ahead.  Loads are
  // unconditional so that every computation waits only for its own block (a
  // conditional load makes the wait counts path-dependent and the compiler
  // falls back to waiting for everything); past the last block the load is an
  // empty-resource one (pair and per-lane-address loads: a re-read of block
  // 0's tile of the head, the same lines for every unit).  The ring index is a
  // compile-time constant in the unrolled body (registers are never indexed at
  // run time).
    for (; c0 < cnt; c0 += kWave) {
      if (c0 > 0) {
        read_table();
        open_table();
        prefetch(cached_c);
      }
      for (int i = 0; i < n; i += NBuf) {
#pragma unroll
        for (int u = 0; u < NBuf; ++u) {
          if (i + u >= n) break;
          load_into(cached_c, f[(u + NBuf - 1) % NBuf], i + u + NBuf - 1,
                    nv[(u + NBuf - 1) % NBuf]);
          attend(f[u], nv[u]);
        }
      }
    }
  };
  // The first chunk's table entries and the sharing test below read in one
  // memory round trip with the q and current-token loads above.
  if (cnt > 0) read_table();
  // A sequence whose first block the neighbouring row of the batch also
  // lists (forks of one prompt, placed side by side) reads its tiles through
  // the caches, so the forks' units share the prompt's tiles in L2; any other
  // sequence streams its tiles, which are read once per call (a false match
  // would only change how a unit's tiles are cached).  The three entries are
  // read unconditionally (in-bounds indexes) so the reads go out together.
  // FP8 pools keep one (streaming) loop: the second copy measured 2-3 %
  // slower there.
  bool cached_unit = false;
  if constexpr (!IsFP8<Tag>::value) {
    if (PA_SHARED_CACHED) {
      const int mb = a.max_blocks;
      const bool has_prev = seq > 0, has_next = seq + 1 < a.num_seqs;
      const int32_t b0 = trow[0];                // L > 0 here, so the row has an entry
      const int32_t bp = trow[has_prev ? -mb : 0];
      const int32_t bn = trow[has_next ? mb : 0];
      cached_unit = (has_prev & (bp == b0)) | (has_next & (bn == b0));
    }
  }
  if constexpr (IsFP8<Tag>::value) {
    block_loop(std::false_type());
  } else {
    if (cached_unit) block_loop(std::true_type());
    else block_loop(std::false_type());
  }
  // Pool write of the current token after the loop: a store while the same
  // tile streams in makes those loads wait on it.
  if (own_new)
    tok.store(a, trow, (raw_len - 1) / a.block_size, g, (raw_len - 1) % a.block_size);

  // ---- merge the four wavefronts (LDS) ----
  const float l_tot = xor_sum(st.l);
  float* sm_m = smem;                      // [W][G]
  float* sm_l = smem + kWaves * G;         // [W][G]
  float* sm_a = smem + 2 * kWaves * G;     // [W][G][D]
  if (h < G) {
    if (lane < 16) {
      sm_m[wave * G + h] = st.m;
      sm_l[wave * G + h] = l_tot;
    }
    float* dst = sm_a + ((int64_t)wave * G + h) * D;
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[out_dim<Tag, D>(n, r, lane)] = st.acc[n][r];
  }
  __syncthreads();

  put_header();
  const bool single = n_parts == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D;
    const int d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * G + hh]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float c = fast_exp2(sm_m[w * G + hh] - M);
        num += c * sm_a[((int64_t)w * G + hh) * D + d];
        den += c * sm_l[w * G + hh];
      }
    }
    const float val = den > 0.f ? num / den * v_scale : 0.f;
    const int64_t row = (int64_t)seq * a.num_q_heads + head0 + hh;
    if (single) {
      store_out<OutT>(reinterpret_cast<OutT*>(a.out) + row * D + d, val);
    } else {
      // One contiguous record per unit: its writes touch the fewest lines.
      const int64_t r = a.planned ? (int64_t)g * a.num_parts + pu.first + part
                                  : ((int64_t)seq * a.num_kv_heads + g) * a.num_parts + part;
      float* rec = a.part + r * a.part_stride;
      rec[hh * D + d] = val;
      if (d == 0) {
        rec[G * D + hh] = M;
        rec[G * D + G + hh] = den;
      }
    }
  }
}

// Combine partitions: out = sum_p c_p l_p o_p / sum_p c_p l_p, c_p = exp2(m_p - max m).
// RT threads per (sequence, query head) row: a whole workgroup when rows are
// few or partitions many, one wavefront (four rows per workgroup) when rows
// are many and partitions few.  Rows with one partition were already written
// by the partition kernel.  The partitions are read in parallel, not one
// after another: each thread takes one partition's (m, l) (chunks of RT), the
// weights c_p l_p go to LDS, and the G-row slices o_p are summed as float4
// quads by RT / (D / 4) partition slots at once, then across slots in LDS.
// A row then costs about two memory round trips up to RT partitions.
template <int RT>
__device__ inline void row_sync() {
  if constexpr (RT == kWave) {                 // wave-synchronous LDS
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

template <int RT>
__device__ inline float row_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if constexpr (RT == kWave) {
    return x;
  } else {
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = x;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < RT / kWave; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
  }
}

template <int D, class OutT, int RT>
__global__ __launch_bounds__(kThreads) void reduce_kernel(DecodeArgs a) {
  constexpr int Q = D / 4;                 // float4 quads of one head's row
  constexpr int kSlots = RT / Q;           // partitions summed at once
  constexpr int kRowsPer = kThreads / RT;
  constexpr int kWavesPer = RT / kWave;    // wavefronts of one row
  __shared__ float s_w_all[kThreads];
  __shared__ f32x4 s_acc_all[kThreads];
  __shared__ float s_red_all[kWaves];
  const int t = threadIdx.x % RT;
  const int sub = threadIdx.x / RT;
  float* s_w = s_w_all + sub * RT;
  f32x4* s_acc = s_acc_all + sub * RT;
  float* s_red = s_red_all + sub * kWavesPer;
  const int64_t row = (int64_t)blockIdx.x * kRowsPer + sub;
  if (row >= (int64_t)a.num_seqs * a.num_q_heads) return;     // RT == kWave only
  const int seq = (int)(row / a.num_q_heads);
  int n_parts, first = 0;
  if (a.planned) {
    const int2 hd = *reinterpret_cast<const int2*>(a.plan_hdr + 2 * seq);
    first = hd.x;
    n_parts = first >= 0 && hd.y <= a.num_parts - first ? hd.y : 0;   // in the records
  } else {
    n_parts = (clip_len(a, seq) + a.ps - 1) / a.ps;
  }
  if (n_parts <= 1) return;
  const int h = (int)(row - (int64_t)seq * a.num_q_heads);
  const int G = a.group;
  const int g = h / G, hh = h - g * G;
  const int64_t rec_first = a.planned ? (int64_t)g * a.num_parts + first
                                      : ((int64_t)seq * a.num_kv_heads + g) * a.num_parts;
  const float* rec0 = a.part + rec_first * a.part_stride;
  const int64_t stride = a.part_stride;
  const float* pm = rec0 + G * D + hh;             // m of partition p at pm[p * stride]
  const float* pl = pm + G;

  // This thread's slices of its first kPre partitions do not depend on the
  // row's maximum: they are loaded together with (m, l), one round trip.
  const int q = t % Q, slot = t / Q;
  constexpr int kPre = 8;
  f32x4 pre[kPre];
  {
    const int n0 = min(RT, n_parts);
    const float* ob = rec0 + hh * D + 4 * q;
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int i = slot + k * kSlots;
      pre[k] = i < n0 ? *reinterpret_cast<const f32x4*>(ob + (int64_t)i * stride)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const float m_own = t < n_parts ? pm[t * stride] : -INFINITY;
  const float l_own = t < n_parts ? pl[t * stride] : 0.f;
  float M = m_own;
  for (int p = t + RT; p < n_parts; p += RT) M = fmaxf(M, pm[p * stride]);
  M = row_max<RT>(M, s_red);

  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {                            // uniform over the row
    for (int p0 = 0; p0 < n_parts; p0 += RT) {
      const int p = p0 + t;
      float w = 0.f;
      if (p0 == 0) w = fast_exp2(m_own - M) * l_own;
      else if (p < n_parts) w = fast_exp2(pm[p * stride] - M) * pl[p * stride];
      den += w;
      s_w[t] = w;
      row_sync<RT>();
      const int n = min(RT, n_parts - p0);
      int i = slot;
      if (p0 == 0) {
#pragma unroll
        for (int k = 0; k < kPre; ++k, i += kSlots)
          if (i < n) num += s_w[i] * pre[k];
      }
      const float* o0 = rec0 + (int64_t)p0 * stride + hh * D + 4 * q;
#pragma unroll 4
      for (; i < n; i += kSlots) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(o0 + (int64_t)i * stride);
        const float wi = s_w[i];
        num += wi * o;
      }
      row_sync<RT>();
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  if ((t & (kWave - 1)) == 0) s_red[t / kWave] = den;
  s_acc[t] = num;
  row_sync<RT>();
  if (slot == 0) {
    float dsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPer; ++w) dsum += s_red[w];
#pragma unroll
    for (int k = 1; k < kSlots; ++k) num += s_acc[k * Q + q];
    OutT* out = reinterpret_cast<OutT*>(a.out) + row * D + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<OutT>(out + e, dsum > 0.f ? num[e] / dsum : 0.f);
  }
}

// Rows of the combine kernel at or above which, with few partitions per row,
// one wavefront per row beats a workgroup per row (measured: 8192 rows of
// 2..8 partitions 6-7 us faster; 1024 rows of ~40 partitions 13 us slower).
constexpr int64_t kWaveRowsMin = 4096;
constexpr int32_t kWaveRowsMaxParts = 32;

template <class Tag, int D, class OutT, int LM>
static pa_status launch(const DecodeArgs& a, int64_t units, size_t lds, hipStream_t stream) {
  decode_kernel<Tag, D, OutT, LM><<<(unsigned)units, kThreads, lds, stream>>>(a);
  pa_status st = launch_status();
  if (st != PA_OK || (a.num_parts <= 1 && !a.planned)) return st;
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
  // Partitions per row: planned splits give num_parts units per KV head to
  // num_seqs sequences.
  const int64_t per_row = a.planned ? (a.num_parts + (int64_t)a.num_seqs - 1) / a.num_seqs
                                    : a.num_parts;
  if (rows >= kWaveRowsMin && per_row <= kWaveRowsMaxParts)
    reduce_kernel<D, OutT, kWave><<<(unsigned)((rows + kWaves - 1) / kWaves), kThreads, 0, stream>>>(a);
  else
    reduce_kernel<D, OutT, kThreads><<<(unsigned)rows, kThreads, 0, stream>>>(a);
  return launch_status();
}

template <class Tag, class OutT, int LM = kLoadBuffer>
static pa_status dispatch_d(int D, const DecodeArgs& a, int64_t units, size_t lds, hipStream_t s) {
  if (D == 128) return launch<Tag, 128, OutT, LM>(a, units, lds, s);
  return launch<Tag, 64, OutT, LM>(a, units, lds, s);
}
// 16-bit pools: 8-token blocks walk pairs of blocks whenever the partitions
// hold whole pairs (else 8-row tiles through buffer loads); 16-row tiles use
// per-lane addresses.
template <class Tag, class OutT>
static pa_status dispatch_16(bool p8, int rows, int D, const DecodeArgs& a, int64_t units,
                             size_t lds, hipStream_t s) {
  if (p8) return dispatch_d<Tag, OutT, kLoadPair8>(D, a, units, lds, s);
  if (rows == kRows) return dispatch_d<Tag, OutT, kLoadGlobal16>(D, a, units, lds, s);
  return dispatch_d<Tag, OutT, kLoadBuffer>(D, a, units, lds, s);
}

// Partition geometry shared by the size query and the launch.
// Automatic partitioning: one unit per (sequence, KV head) already fills the
// GPU when there are at least as many units as resident workgroups (one per
// wavefront slot of a SIMD on every compute unit); otherwise the split is
// planned from the lengths in the kernels (one round of near-equal units,
// num_parts of them per KV head), unless no sequence can be longer than the
// smallest unit worth splitting off.
constexpr int32_t kMinPlannedTokens = 512;

static int32_t resident_per_cu(pa_dtype dt, int32_t D) {
  if (dt == PA_F32 && D == 128) return 2;
  return dt == PA_FP8_E4M3 ? PA_FP8_WAVES_PER_EU : PA_WAVES_PER_EU;
}

struct Geometry {
  int32_t ps;        // partition size in tokens (fixed partitions)
  int32_t parts;     // partitions per sequence, or units per KV head when planned
  bool planned;
};

static Geometry geometry(const pa_pool_desc* pool, int32_t num_seqs, int32_t max_len,
                         int32_t partition_size) {
  Geometry geo{0, 1, false};
  if (partition_size == PA_PARTITION_AUTO) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t slots =
        (int64_t)(cus > 0 ? cus : 256) * resident_per_cu(pool->dtype, pool->head_dim);
    if ((int64_t)num_seqs * pool->num_kv_heads < slots && max_len > kMinPlannedTokens) {
      geo.planned = true;
      geo.parts = (int32_t)(slots / pool->num_kv_heads);
      return geo;
    }
    partition_size = 0;
  }
  // One partition: whole 16-token tiles (8-token blocks then walk in pairs).
  const int32_t b = pool->block_size;
  const int32_t unit = b < 16 ? 16 : b;
  const int32_t whole = ((max_len > 0 ? max_len : 1) + unit - 1) / unit * unit;
  geo.ps = partition_size == 0 ? whole : partition_size;
  geo.parts = max_len > 0 ? (max_len + geo.ps - 1) / geo.ps : 1;
  return geo;
}

static bool partition_ok(int32_t partition_size, int32_t b) {
  return partition_size == PA_PARTITION_AUTO || (partition_size >= 0 && partition_size % b == 0);
}

// Floats per partial record: G rows of D, then G maxima and G sums, rounded up
// to whole 128-byte lines.
static int32_t record_floats(int32_t G, int32_t D) { return (G * D + 2 * G + 31) / 32 * 32; }

// Records: one per (KV head, unit) when planned, else per (sequence, KV head,
// partition); none without a split.
static size_t record_bytes(const Geometry& geo, int32_t num_seqs, int32_t Hkv, int32_t G,
                           int32_t D) {
  int64_t records;
  if (geo.planned) records = (int64_t)Hkv * geo.parts;
  else if (geo.parts > 1) records = (int64_t)num_seqs * Hkv * geo.parts;
  else return 0;
  return (size_t)(records * (int64_t)record_floats(G, D) * 4);
}

// The records, then (planned split) two ints per sequence.
static size_t workspace_bytes(const Geometry& geo, int32_t num_seqs, int32_t Hkv, int32_t G,
                              int32_t D) {
  return record_bytes(geo, num_seqs, Hkv, G, D) + (geo.planned ? (size_t)num_seqs * 8 : 0);
}


// Shared by pa_decode_attention (k_new == null) and pa_decode_step.
static pa_status decode_impl(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                             const void* k_new, const void* v_new, int64_t new_stride,
                             const void* q, void* out, pa_dtype out_dtype,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                             float scale, int32_t max_context_len, int32_t partition_size,
                             void* workspace, size_t workspace_size, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 0 || max_context_len < 0 ||
      !partition_ok(partition_size, pool->block_size))
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads) return PA_ERR_INVALID_ARG;
  const int32_t G = num_q_heads / pool->num_kv_heads;
  if (G > 16) return PA_ERR_UNSUPPORTED;
  const pa_dtype out16 = pool->dtype == PA_FP8_E4M3 ? PA_BF16 : pool->dtype;
  if (out_dtype != PA_F32 && out_dtype != out16) return PA_ERR_UNSUPPORTED;
  const int es = input_bytes(pool->dtype);
  if (k_new) {
    if (new_stride < (int64_t)pool->num_kv_heads * pool->head_dim || (new_stride * es) % 16 ||
        !aligned16(k_new) || !aligned16(v_new))
      return PA_ERR_INVALID_ARG;
  }
  if (num_seqs == 0) return PA_OK;
  if (!k_pool || !v_pool || !q || !out || !context_lens) return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq > 0 && !block_tables) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(q)) return PA_ERR_INVALID_ARG;
  if (!(scale == scale)) return PA_ERR_INVALID_ARG;

  const Geometry geo = geometry(pool, num_seqs, max_context_len, partition_size);
  const size_t need = workspace_bytes(geo, num_seqs, pool->num_kv_heads, G, pool->head_dim);
  if (need > 0 && (!workspace || workspace_size < need || !aligned16(workspace)))
    return PA_ERR_WORKSPACE;
  const int64_t units = (int64_t)pool->num_kv_heads * (geo.planned ? 1 : num_seqs) * geo.parts;
  // A dispatch counts its work-items in 32 bits.
  constexpr int64_t kMaxGroups = (int64_t)UINT32_MAX / kThreads;
  if (units > kMaxGroups) return PA_ERR_UNSUPPORTED;
  if ((geo.planned || geo.parts > 1) && (int64_t)num_seqs * num_q_heads > kMaxGroups)
    return PA_ERR_UNSUPPORTED;                   // the combine kernel's rows

  DecodeArgs a;
  a.k_pool = (char*)k_pool;
  a.v_pool = (char*)v_pool;
  a.k_new = (const char*)k_new;
  a.v_new = (const char*)v_new;
  a.new_stride = new_stride;
  a.q = (const char*)q;
  a.out = out;
  a.tables = block_tables;
  a.lens = context_lens;
  a.part = need > 0 ? (float*)workspace : nullptr;
  a.plan_hdr = geo.planned ? (int32_t*)((char*)workspace +
                                        record_bytes(geo, num_seqs, pool->num_kv_heads, G,
                                                     pool->head_dim))
                           : nullptr;
  a.part_stride = record_floats(G, pool->head_dim);
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
  a.ps = geo.ps;
  a.num_parts = geo.parts;
  a.planned = geo.planned;
#ifdef PA_NO_LONGEST_FIRST
  a.longest_first = 0;
#else
  a.longest_first = !geo.planned;                // planned units are of near-equal work
#endif
  a.qk_scale = scale * kLog2e;
  a.k_scales = pool->k_scales;
  a.v_scales = pool->v_scales;
  // LDS: [merge area | staged current token]; the ranking keys alias the start.
  const size_t merge = ((size_t)kWaves * G * (pool->head_dim + 2) * sizeof(float) + 15) / 16 * 16;
  a.stage_off = (int32_t)merge;
  size_t lds = merge + (k_new ? (size_t)2 * pool->head_dim * es : 0);
  if (a.longest_first) lds = std::max(lds, (size_t)kRankLdsInts * sizeof(int));
  const hipStream_t s = (hipStream_t)stream;
  const int D = pool->head_dim;
  const bool p8 = pool->block_size == 8 && (geo.planned || geo.ps % 16 == 0);
  const int part_rows = p8 && (pool->dtype == PA_BF16 || pool->dtype == PA_F16) ? 16 : a.rows;
  a.part_shift = part_rows == 16 ? 4 : 3;      // rows: 8 or 16
  a.min_tiles = kMinPlannedTokens / part_rows;

  switch (pool->dtype) {
    case PA_BF16:
      return out_dtype == PA_F32 ? dispatch_16<TagBF16, float>(p8, a.rows, D, a, units, lds, s)
                                 : dispatch_16<TagBF16, __bf16>(p8, a.rows, D, a, units, lds, s);
    case PA_F16:
      return out_dtype == PA_F32 ? dispatch_16<TagF16, float>(p8, a.rows, D, a, units, lds, s)
                                 : dispatch_16<TagF16, _Float16>(p8, a.rows, D, a, units, lds, s);
    case PA_FP8_E4M3:
      return out_dtype == PA_F32 ? dispatch_d<TagFP8, float>(D, a, units, lds, s)
                                 : dispatch_d<TagFP8, __bf16>(D, a, units, lds, s);
    case PA_F32:
      return dispatch_d<TagF32, float>(D, a, units, lds, s);
    default:
      return PA_ERR_UNSUPPORTED;
  }
}

// Device scratch of pa_decode_step_noalloc: the split workspace for callers
// that cannot allocate.  One copy per GPU, created when the library's code
// object loads there and held until the process ends.  In host code
// `scratch` names a host-side stand-in: only the per-device address that
// hipGetSymbolAddress returns may reach a kernel or a copy.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept; null if the lookup fails.
static void* scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace pa

using namespace pa;

extern "C" {

pa_status pa_decode_workspace_size(const pa_pool_desc* pool, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_context_len,
                                   int32_t partition_size, size_t* bytes) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (!bytes || num_seqs < 0 || num_q_heads < 1 || max_context_len < 0 ||
      !partition_ok(partition_size, pool->block_size))
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads) return PA_ERR_INVALID_ARG;
  const Geometry geo = geometry(pool, num_seqs, max_context_len, partition_size);
  *bytes = workspace_bytes(geo, num_seqs, pool->num_kv_heads, num_q_heads / pool->num_kv_heads,
                           pool->head_dim);
  return PA_OK;
}

pa_status pa_decode_attention(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                              const void* q, void* out, pa_dtype out_dtype,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, float scale, int32_t max_context_len,
                              int32_t partition_size, void* workspace, size_t workspace_size,
                              void* stream) {
  return decode_impl(pool, (void*)k_pool, (void*)v_pool, nullptr, nullptr, 0, q, out, out_dtype,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                     scale, max_context_len, partition_size, workspace, workspace_size, stream);
}

pa_status pa_decode_step(const pa_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                         const void* v_new, int64_t new_stride, const void* q, void* out,
                         pa_dtype out_dtype, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, float scale,
                         int32_t max_context_len, int32_t partition_size, void* workspace,
                         size_t workspace_size, void* stream) {
  if (!k_new || !v_new) return PA_ERR_INVALID_ARG;
  return decode_impl(pool, k_pool, v_pool, k_new, v_new, new_stride, q, out, out_dtype,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                     scale, max_context_len, partition_size, workspace, workspace_size, stream);
}

pa_status pa_decode_step_noalloc(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                                 const void* k_new, const void* v_new, int64_t new_stride,
                                 const void* q, void* out, pa_dtype out_dtype,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, float scale, int32_t max_context_len,
                                 int32_t partition_size, void* stream) {
  if (!k_new || !v_new) return PA_ERR_INVALID_ARG;
  size_t need = 0;
  const pa_status st = pa_decode_workspace_size(pool, num_seqs, num_q_heads, max_context_len,
                                                partition_size, &need);
  if (st != PA_OK) return st;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_on_current_device())) return PA_ERR_HIP;
  return decode_impl(pool, k_pool, v_pool, k_new, v_new, new_stride, q, out, out_dtype,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                     scale, max_context_len, partition_size, ws,
                     need > 0 ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"
