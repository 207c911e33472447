// Cache-side kernels of libpa: slot mapping, token writes, block copies and
// table validation.  All are byte movers or integer arithmetic; the bound is
// HBM bandwidth (or launch latency at decode sizes).
//
// Address rule ("Inside vLLM and TGI: Paging, Versioned Schedulers and
// Operations", section "Block addresses and fragmentation arithmetic"):
// position t lives at offset t % b of physical block table[t / b].
// Copy-on-write of a shared partial last block (same page, section "Exact
// CPU block manager and copy-on-write"; "vLLM and PagedAttention"
// transcript, paragraph 4) is a whole-block copy in both pools.
#include "pa_internal.h"

namespace pa {

// ---------------------------------------------------------------------------
// slot = table[seq][p / b] * b + p % b   (one thread per new token)
// ---------------------------------------------------------------------------
__global__ void slot_mapping_kernel(const int32_t* __restrict__ tables, int32_t max_blocks,
                                    int32_t num_seqs, const int32_t* __restrict__ seq_ids,
                                    const int32_t* __restrict__ positions, int32_t n,
                                    int32_t block_size, int32_t* __restrict__ slots) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int32_t s = seq_ids[t];
  const int32_t pos = positions[t];
  int32_t out = -1;
  if (s >= 0 && s < num_seqs && pos >= 0) {
    const int32_t j = pos / block_size;
    if (j < max_blocks) {
      const int32_t phys = tables[(int64_t)s * max_blocks + j];
      const int64_t flat = (int64_t)phys * block_size + pos % block_size;
      if (phys >= 0 && flat <= INT32_MAX) out = (int32_t)flat;
    }
  }
  slots[t] = out;
}

// ---------------------------------------------------------------------------
// Token writes.  One thread moves one 16-byte vector of X consecutive dims of
// one (token, KV head).  16-bit K tiles are sub-tiled ([d/32][R][4][8] per R
// = min(b, 16) rows): the vector is one 16-byte store, a token's row four
// 64-byte pieces; fp32 K tiles are token-major.  V tiles interleave groups of
// 4 tokens per dim ([b/4][d][4]): X element stores, stride 4 elements.
// ---------------------------------------------------------------------------
template <int ES>  // element size in bytes: 2 or 4
__global__ void write_kv_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                const char* __restrict__ k_new, const char* __restrict__ v_new,
                                int64_t new_stride, const int32_t* __restrict__ slots, int32_t n,
                                int32_t num_heads, int32_t head_dim, int32_t block_size,
                                int64_t num_slots) {
  constexpr int X = 16 / ES;
  const int chunks = head_dim / X;                 // vectors per (token, head)
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)num_heads * chunks;
  if (gid >= (int64_t)n * per_tok) return;
  const int t = (int)(gid / per_tok);
  const int rem = (int)(gid - (int64_t)t * per_tok);
  const int h = rem / chunks;
  const int c = rem - h * chunks;
  const int32_t slot = slots[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int32_t blk = slot / block_size;
  const int32_t off = slot - blk * block_size;
  const int64_t src = ((int64_t)t * new_stride + (int64_t)h * head_dim + (int64_t)c * X) * ES;
  const int64_t tile = ((int64_t)blk * num_heads + h) * (int64_t)block_size * head_dim;  // elements
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + src);
  if constexpr (ES == 2)      // 16-bit K: sub-tiled layout, one 16-byte piece
    *reinterpret_cast<u32x4*>(k_pool + tile * ES + k16_offset(off, c * X, block_size, head_dim)) = kv;
  else                        // fp32 K: token-major rows
    *reinterpret_cast<u32x4*>(k_pool + (tile + (int64_t)off * head_dim + (int64_t)c * X) * ES) = kv;
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + src);
  char* vb = v_pool + (tile + ((int64_t)(off >> 2) * head_dim + (int64_t)c * X) * 4 + (off & 3)) * ES;
  if constexpr (ES == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(vb + (int64_t)e * 4 * 4) = vv[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t half = (uint16_t)(vv[e >> 1] >> ((e & 1) * 16));
      *reinterpret_cast<uint16_t*>(vb + (int64_t)e * 4 * 2) = half;
    }
  }
}

// 16-bit pools, many tokens (prefill chunks): one wavefront per 4 input
// tokens and KV head.  A token whose slot opens an aligned group of 4 slots,
// with the next three input tokens on the next three slots, leads that group:
// the wavefront writes the group's 4 K rows (per 32-dim chunk, 4 x 64 bytes
// contiguous) and its V group (4 tokens x head_dim elements, contiguous) as
// whole 128-byte lines, reading 4 bytes (V) or 16 bytes (K) of the inputs per
// lane.  A token inside a group led from an earlier input position was
// written by that group's wavefront; every other token is written on its own
// by 16 lanes as in write_kv_kernel.  Writes cost per line touched while
// other traffic streams, and a lone token's V is 2 bytes in each of
// head_dim / 4 lines, so grouped tokens cost about a quarter as much.
__device__ inline bool group_lead(const int32_t* slots, int32_t n, int t, int64_t num_slots) {
  if (t < 0 || t + 3 >= n) return false;
  const int32_t s = slots[t];
  if (s < 0 || (s & 3) != 0 || (int64_t)s + 3 >= num_slots) return false;
  return slots[t + 1] == s + 1 && slots[t + 2] == s + 2 && slots[t + 3] == s + 3;
}

__global__ __launch_bounds__(64) void write_kv_groups_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, int64_t new_stride, const int32_t* __restrict__ slots,
    int32_t n, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_slots) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x % num_heads;
  const int t0 = (blockIdx.x / num_heads) * 4;
  const int R = block_size < 16 ? block_size : 16;
  // The group led from t0 .. t0 + 3, if any (at most one: a leader's next
  // three tokens sit on slots that are not multiples of 4).
  int lead = -1;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (lead < 0 && group_lead(slots, n, t0 + k, num_slots)) lead = t0 + k;
  if (lead >= 0 && lane < head_dim / 2) {
    const int32_t s = slots[lead];
    const int32_t blk = s / block_size;
    const int32_t o = s - blk * block_size;                    // multiple of 4
    const int64_t tile = ((int64_t)blk * num_heads + h) * (int64_t)block_size * head_dim * 2;
    // K: lane -> (chunk m, row r, 16-byte quarter q) of the group's 4 rows.
    const int m = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
    const int64_t ks = ((int64_t)(lead + r) * new_stride + (int64_t)h * head_dim + m * 32 + q * 8) * 2;
    const int64_t kd = tile + (int64_t)(o / R) * R * head_dim * 2 + m * R * 64 +
                       (int64_t)((o % R) + r) * 64 + q * 16;
    *reinterpret_cast<u32x4*>(k_pool + kd) = *reinterpret_cast<const u32x4*>(k_new + ks);
    // V: lane -> dims 2 lane, 2 lane + 1 of the 4 tokens: 16 contiguous bytes.
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = *reinterpret_cast<const uint32_t*>(
          v_new + ((int64_t)(lead + j) * new_stride + (int64_t)h * head_dim + 2 * lane) * 2);
    const u32x4 vv = {(w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16),
                      (w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u)};
    *reinterpret_cast<u32x4*>(v_pool + tile + (int64_t)(o >> 2) * head_dim * 8 + lane * 16) = vv;
  }
  // Tokens of t0 .. t0 + 3 outside every group: 16 lanes each.
  const int t = t0 + (lane >> 4);
  const int c = lane & 15;
  if (t >= n || c >= head_dim / 8) return;
  const int32_t slot = slots[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  if (lead >= 0 && t >= lead && t < lead + 4) return;           // in this wavefront's group
  if (group_lead(slots, n, t - (slot & 3), num_slots) && slots[t - (slot & 3)] == slot - (slot & 3))
    return;                                                     // in an earlier group
  const int32_t blk = slot / block_size;
  const int32_t off = slot - blk * block_size;
  const int64_t src = ((int64_t)t * new_stride + (int64_t)h * head_dim + (int64_t)c * 8) * 2;
  const int64_t tile = ((int64_t)blk * num_heads + h) * (int64_t)block_size * head_dim;  // elements
  *reinterpret_cast<u32x4*>(k_pool + tile * 2 + k16_offset(off, c * 8, block_size, head_dim)) =
      *reinterpret_cast<const u32x4*>(k_new + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + src);
  char* vb = v_pool + (tile + ((int64_t)(off >> 2) * head_dim + (int64_t)c * 8) * 4 + (off & 3)) * 2;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint16_t*>(vb + (int64_t)e * 8) = (uint16_t)(vv[e >> 1] >> ((e & 1) * 16));
}

// FP8 pools: bf16 inputs; a thread quantizes 16 consecutive dims of one
// (token, head) with that head's scales into one 16-byte K store and 16
// one-byte V stores, at the offsets of the FP8 tile layout.
__device__ inline uint32_t pack4_fp8(const u32x4& a, const u32x4& b, int q, float scale) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * q + j;                         // element 0..15
    const uint32_t word = e < 8 ? a[(e & 7) >> 1] : b[(e & 7) >> 1];
    const float x = bf16_bits_to_float((word >> ((e & 1) * 16)) & 0xFFFFu);
    w |= fp8_code(x, scale) << (8 * j);
  }
  return w;
}

// One 16-dim chunk c of token t, head h (a thread's share of the per-token path).
__device__ inline void write_fp8_chunk(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                       const char* __restrict__ k_new,
                                       const char* __restrict__ v_new, int64_t new_stride,
                                       int t, int h, int c, int32_t slot, int32_t num_heads,
                                       int32_t head_dim, int32_t block_size,
                                       const float* __restrict__ k_scales,
                                       const float* __restrict__ v_scales) {
  constexpr int X = 16;
  const int32_t blk = slot / block_size;
  const int32_t off = slot - blk * block_size;
  const int64_t src = ((int64_t)t * new_stride + (int64_t)h * head_dim + (int64_t)c * X) * 2;
  const int64_t tile = ((int64_t)blk * num_heads + h) * (int64_t)block_size * head_dim;  // bytes
  const u32x4 k0 = *reinterpret_cast<const u32x4*>(k_new + src);
  const u32x4 k1 = *reinterpret_cast<const u32x4*>(k_new + src + 16);
  const float ks = k_scales[h];
  u32x4 kc;
#pragma unroll
  for (int q = 0; q < 4; ++q) kc[q] = pack4_fp8(k0, k1, q, ks);
  // 16 consecutive dims starting at a multiple of 16 are one 16-byte piece
  *reinterpret_cast<u32x4*>(k_pool + tile + fp8_k_offset(off, c * X, block_size, head_dim)) = kc;
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(v_new + src);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(v_new + src + 16);
  const float vs = v_scales[h];
  char* vt = v_pool + tile;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = pack4_fp8(v0, v1, q, vs);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      vt[fp8_v_offset(off, c * X + 4 * q + j, block_size, head_dim)] = (char)((w >> (8 * j)) & 0xFFu);
  }
}

__global__ void write_kv_fp8_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                    const char* __restrict__ k_new, const char* __restrict__ v_new,
                                    int64_t new_stride, const int32_t* __restrict__ slots,
                                    int32_t n, int32_t num_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_slots,
                                    const float* __restrict__ k_scales,
                                    const float* __restrict__ v_scales) {
  const int chunks = head_dim / 16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)num_heads * chunks;
  if (gid >= (int64_t)n * per_tok) return;
  const int t = (int)(gid / per_tok);
  const int rem = (int)(gid - (int64_t)t * per_tok);
  const int h = rem / chunks;
  const int c = rem - h * chunks;
  const int32_t slot = slots[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  write_fp8_chunk(k_pool, v_pool, k_new, v_new, new_stride, t, h, c, slot, num_heads, head_dim,
                  block_size, k_scales, v_scales);
}

// FP8 pools, 4 or more tokens: as write_kv_groups_kernel, a wavefront per 4
// input tokens and KV head writes a run of 4 consecutive slots from a
// multiple of 4 as whole pieces: K as head_dim / 16 runs of 64 bytes (the 4
// rows' 16-byte pieces are adjacent), V as the token group's 4 * head_dim
// contiguous bytes, each lane one 16-byte chunk of 4 dims x 4 tokens (no
// byte stores).  Lanes 0 .. D/4 - 1 write K, D/4 .. D/2 - 1 write V.  Other
// tokens are written per 16-dim chunk as above.
__global__ __launch_bounds__(64) void write_kv_fp8_groups_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, int64_t new_stride, const int32_t* __restrict__ slots,
    int32_t n, int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_slots,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x % num_heads;
  const int t0 = (blockIdx.x / num_heads) * 4;
  const int D = head_dim;
  int lead = -1;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (lead < 0 && group_lead(slots, n, t0 + k, num_slots)) lead = t0 + k;
  if (lead >= 0 && lane < D / 2) {
    const int32_t s = slots[lead];
    const int32_t blk = s / block_size;
    const int32_t o = s - blk * block_size;                    // multiple of 4
    char* kt = k_pool + ((int64_t)blk * num_heads + h) * (int64_t)block_size * D;
    char* vt = v_pool + ((int64_t)blk * num_heads + h) * (int64_t)block_size * D;
    if (lane < D / 4) {
      // K: lane -> (row r of the group, 16-dim chunk c); rows of one chunk adjacent.
      const int r = lane & 3, c = lane >> 2;
      const int64_t src = ((int64_t)(lead + r) * new_stride + (int64_t)h * D + c * 16) * 2;
      const u32x4 a = *reinterpret_cast<const u32x4*>(k_new + src);
      const u32x4 b = *reinterpret_cast<const u32x4*>(k_new + src + 16);
      const float ks = k_scales[h];
      u32x4 kc;
#pragma unroll
      for (int q = 0; q < 4; ++q) kc[q] = pack4_fp8(a, b, q, ks);
      *reinterpret_cast<u32x4*>(kt + fp8_k_offset(o + r, c * 16, block_size, D)) = kc;
    } else {
      // V: chunk v of the group's 4*D bytes = (piece hh, dim row dr): dims
      // dr*D/16 + 4hh .. +3, byte (e, j) = dim e, token j.
      const int v = lane - D / 4;
      const int hh = v >> 4, dr = v & 15;
      const int d0 = dr * (D / 16) + 4 * hh;
      const float vs = v_scales[h];
      uint32_t w[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(
            v_new + ((int64_t)(lead + j) * new_stride + (int64_t)h * D + d0) * 2);
        w[j][0] = x[0];
        w[j][1] = x[1];
      }
      u32x4 vc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float f = bf16_bits_to_float((w[j][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
          word |= fp8_code(f, vs) << (8 * j);
        }
        vc[e] = word;
      }
      *reinterpret_cast<u32x4*>(vt + fp8_v_offset(o, d0, block_size, D)) = vc;
    }
  }
  // Tokens of t0 .. t0 + 3 outside every group: 16 lanes each, a 16-dim chunk per lane.
  const int t = t0 + (lane >> 4);
  const int c = lane & 15;
  if (t >= n || c >= D / 16) return;
  const int32_t slot = slots[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  if (lead >= 0 && t >= lead && t < lead + 4) return;           // in this wavefront's group
  if (group_lead(slots, n, t - (slot & 3), num_slots) && slots[t - (slot & 3)] == slot - (slot & 3))
    return;                                                     // in an earlier group
  write_fp8_chunk(k_pool, v_pool, k_new, v_new, new_stride, t, h, c, slot, num_heads, D,
                  block_size, k_scales, v_scales);
}

// ---------------------------------------------------------------------------
// Whole-block copies: every 16-byte vector of the (src) block in both pools.
// ---------------------------------------------------------------------------
__global__ void copy_blocks_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                   const int32_t* __restrict__ pairs, int32_t n_pairs,
                                   int64_t block_vecs, int32_t num_blocks) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_pair = 2 * block_vecs;
  if (gid >= (int64_t)n_pairs * per_pair) return;
  const int p = (int)(gid / per_pair);
  int64_t r = gid - (int64_t)p * per_pair;
  char* pool = k_pool;
  if (r >= block_vecs) { pool = v_pool; r -= block_vecs; }
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(pool) + (int64_t)src * block_vecs + r;
  u32x4* d = reinterpret_cast<u32x4*>(pool) + (int64_t)dst * block_vecs + r;
  *d = *s;
}

// ---------------------------------------------------------------------------
// Swap: whole blocks between the device pools and pinned host pools of the
// same layout (preemption by swapping; the K/V of an evicted sequence is
// moved to CPU memory and restored later).  A workgroup moves one 16 KiB
// segment of one block of one pool: wavefront w, lane l handles 16-byte
// vectors seg*1024 + 256w + 64j + l, j = 0..3, all four loads issued before
// the stores, so each instruction covers 1 KiB contiguous and a host read
// keeps four requests in flight per lane.
// ---------------------------------------------------------------------------
constexpr int kSwapSegVecs = 1024;

__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const char* __restrict__ src_k, const char* __restrict__ src_v, char* __restrict__ dst_k,
    char* __restrict__ dst_v, const int32_t* __restrict__ pairs, int32_t n_pairs,
    int64_t block_vecs, int32_t segs, int32_t src_blocks, int32_t dst_blocks) {
  const int unit = blockIdx.x;
  const int per_pair = 2 * segs;
  const int p = unit / per_pair;
  if (p >= n_pairs) return;
  int r = unit - p * per_pair;
  const bool is_v = r >= segs;
  if (is_v) r -= segs;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(is_v ? src_v : src_k) + (int64_t)src * block_vecs;
  u32x4* d = reinterpret_cast<u32x4*>(is_v ? dst_v : dst_k) + (int64_t)dst * block_vecs;
  const int64_t base = (int64_t)r * kSwapSegVecs + (threadIdx.x >> 6) * 256 + (threadIdx.x & 63);
  u32x4 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = base + 64 * j;
    if (i < block_vecs) x[j] = s[i];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = base + 64 * j;
    if (i < block_vecs) d[i] = x[j];
  }
}

// Device address of a pinned host range [p, p + bytes), or null when the range
// is not page-locked host memory mapped for the current device.
static char* pinned_device_address(void* p, int64_t bytes) {
  hipPointerAttribute_t first, last;
  if (hipPointerGetAttributes(&first, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (hipPointerGetAttributes(&last, (char*)p + bytes - 1) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (first.type != hipMemoryTypeHost || last.type != hipMemoryTypeHost ||
      !first.devicePointer || !last.devicePointer)
    return nullptr;
  char* d = (char*)first.devicePointer;
  if ((char*)last.devicePointer != d + bytes - 1) return nullptr;    // one mapping
  return d;
}

// ---------------------------------------------------------------------------
// Validation: count lengths out of range and referenced entries out of range.
// ---------------------------------------------------------------------------
__global__ void zero_int_kernel(int32_t* p) { *p = 0; }

__global__ void validate_kernel(const int32_t* __restrict__ tables, int32_t max_blocks,
                                const int32_t* __restrict__ lens, int32_t num_seqs,
                                int32_t max_len, int32_t num_blocks, int32_t block_size,
                                int32_t* bad) {
  const int s = blockIdx.x;
  if (s >= num_seqs) return;
  const int32_t L = lens[s];
  const int64_t cap = (int64_t)max_blocks * block_size;
  int32_t local = 0;
  int32_t check_blocks;
  if (L < 1 || L > max_len || (int64_t)L > cap) {
    if (threadIdx.x == 0) local += 1;
    check_blocks = (L < 1) ? 0 : (int32_t)min<int64_t>((L + block_size - 1) / block_size, max_blocks);
  } else {
    check_blocks = (L + block_size - 1) / block_size;
  }
  for (int j = threadIdx.x; j < check_blocks; j += blockDim.x) {
    const int32_t phys = tables[(int64_t)s * max_blocks + j];
    if (phys < 0 || phys >= num_blocks) local += 1;
  }
  if (local) atomicAdd(bad, local);
}

// Debug check of one batch of block copies: pair i counts once when its
// destination is the destination of another pair or the source of any pair
// (its own included).  Pairs with an id outside the pool are skipped by the
// copy and take no part.  Each workgroup walks all pairs in chunks of its
// size staged in LDS: n^2 comparisons in all, meant for debug batches.
__global__ void validate_pairs_kernel(const int32_t* __restrict__ pairs, int32_t n,
                                      int32_t num_blocks, int32_t* bad) {
  __shared__ int2 chunk[256];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto in_pool = [&](int2 p) {
    return p.x >= 0 && p.x < num_blocks && p.y >= 0 && p.y < num_blocks;
  };
  const int2 me = i < n ? make_int2(pairs[2 * i], pairs[2 * i + 1]) : make_int2(-1, -1);
  const bool live = i < n && in_pool(me);
  bool hit = false;
  for (int64_t base = 0; base < n; base += blockDim.x) {
    const int64_t j = base + threadIdx.x;
    const int2 p = j < n ? make_int2(pairs[2 * j], pairs[2 * j + 1]) : make_int2(-1, -1);
    chunk[threadIdx.x] = j < n && in_pool(p) ? p : make_int2(-1, -1);
    __syncthreads();
    const int m = (int)min((int64_t)blockDim.x, (int64_t)n - base);
    if (live) {
      for (int k = 0; k < m; ++k) {
        const int2 q = chunk[k];
        if (q.x < 0) continue;                   // a skipped pair
        hit |= q.x == me.y || (base + k != i && q.y == me.y);
      }
    }
    __syncthreads();
  }
  if (hit) atomicAdd(bad, 1);
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t pa_version(void) { return 100; }

pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t num_seqs, const int32_t* seq_ids, const int32_t* positions,
                          int32_t n, int32_t block_size, int32_t* slots, void* stream) {
  if (n < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || block_size < 1) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!seq_ids || !positions || !slots) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && max_blocks_per_seq > 0 && !block_tables) return PA_ERR_INVALID_ARG;
  const int threads = 256;
  slot_mapping_kernel<<<(n + threads - 1) / threads, threads, 0, (hipStream_t)stream>>>(
      block_tables, max_blocks_per_seq, num_seqs, seq_ids, positions, n, block_size, slots);
  return launch_status();
}

pa_status pa_write_kv(const pa_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, int64_t new_stride, const int32_t* slot_mapping,
                      int32_t n, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  const int es = elem_bytes(pool->dtype);
  const int ies = input_bytes(pool->dtype);
  const int64_t row = (int64_t)pool->num_kv_heads * pool->head_dim;
  if (new_stride < row) return PA_ERR_INVALID_ARG;
  // 16-byte vector moves need 16-byte aligned pools, rows and token strides.
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new) ||
      (new_stride * ies) % 16 != 0)
    return PA_ERR_INVALID_ARG;
  const int64_t vecs = (int64_t)n * pool->num_kv_heads * (pool->head_dim * es / 16);
  const int threads = 256;
  const int64_t blocks = (vecs + threads - 1) / threads;
  if (blocks > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int64_t num_slots = (int64_t)pool->num_blocks * pool->block_size;
  if (es == 1 && n >= 4) {
    const int64_t groups = ((int64_t)n + 3) / 4 * pool->num_kv_heads;
    if (groups > INT32_MAX) return PA_ERR_UNSUPPORTED;
    write_kv_fp8_groups_kernel<<<(unsigned)groups, 64, 0, (hipStream_t)stream>>>(
        (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, new_stride,
        slot_mapping, n, pool->num_kv_heads, pool->head_dim, pool->block_size, num_slots,
        pool->k_scales, pool->v_scales);
  } else if (es == 1)
    write_kv_fp8_kernel<<<(unsigned)blocks, threads, 0, (hipStream_t)stream>>>(
        (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, new_stride,
        slot_mapping, n, pool->num_kv_heads, pool->head_dim, pool->block_size, num_slots,
        pool->k_scales, pool->v_scales);
  else if (es == 2 && n >= 4) {
    const int64_t groups = ((int64_t)n + 3) / 4 * pool->num_kv_heads;
    if (groups > INT32_MAX) return PA_ERR_UNSUPPORTED;
    write_kv_groups_kernel<<<(unsigned)groups, 64, 0, (hipStream_t)stream>>>(
        (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, new_stride,
        slot_mapping, n, pool->num_kv_heads, pool->head_dim, pool->block_size, num_slots);
  } else if (es == 2)
    write_kv_kernel<2><<<(unsigned)blocks, threads, 0, (hipStream_t)stream>>>(
        (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, new_stride,
        slot_mapping, n, pool->num_kv_heads, pool->head_dim, pool->block_size, num_slots);
  else
    write_kv_kernel<4><<<(unsigned)blocks, threads, 0, (hipStream_t)stream>>>(
        (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, new_stride,
        slot_mapping, n, pool->num_kv_heads, pool->head_dim, pool->block_size, num_slots);
  return launch_status();
}

pa_status pa_copy_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                         const int32_t* block_pairs, int32_t n_pairs, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n_pairs < 0) return PA_ERR_INVALID_ARG;
  if (n_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_pairs) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)pool->num_kv_heads * tile_elems(pool) * elem_bytes(pool->dtype);
  const int64_t block_vecs = block_bytes / 16;
  const int64_t total = (int64_t)n_pairs * 2 * block_vecs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > INT32_MAX) return PA_ERR_UNSUPPORTED;
  copy_blocks_kernel<<<(unsigned)blocks, threads, 0, (hipStream_t)stream>>>(
      (char*)k_pool, (char*)v_pool, block_pairs, n_pairs, block_vecs, pool->num_blocks);
  return launch_status();
}

pa_status pa_swap_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool, void* host_k,
                         void* host_v, int32_t host_num_blocks, const int32_t* block_pairs,
                         int32_t n_pairs, int32_t direction, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n_pairs < 0 || host_num_blocks < 0 ||
      (direction != PA_SWAP_OUT && direction != PA_SWAP_IN))
    return PA_ERR_INVALID_ARG;
  if (n_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !host_k || !host_v || !block_pairs || host_num_blocks == 0)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(host_k) || !aligned16(host_v))
    return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)pool->num_kv_heads * tile_elems(pool) * elem_bytes(pool->dtype);
  const int64_t host_bytes = (int64_t)host_num_blocks * block_bytes;
  char* hk = pinned_device_address(host_k, host_bytes);
  char* hv = pinned_device_address(host_v, host_bytes);
  if (!hk || !hv) return PA_ERR_INVALID_ARG;
  const int64_t block_vecs = block_bytes / 16;
  const int64_t segs = (block_vecs + kSwapSegVecs - 1) / kSwapSegVecs;
  const int64_t units = (int64_t)n_pairs * 2 * segs;
  if (units > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const bool out = direction == PA_SWAP_OUT;
  swap_blocks_kernel<<<(unsigned)units, 256, 0, (hipStream_t)stream>>>(
      out ? (const char*)k_pool : hk, out ? (const char*)v_pool : hv, out ? hk : (char*)k_pool,
      out ? hv : (char*)v_pool, block_pairs, n_pairs, block_vecs, (int32_t)segs,
      out ? pool->num_blocks : host_num_blocks, out ? host_num_blocks : pool->num_blocks);
  return launch_status();
}

pa_status pa_validate_copy_pairs(const pa_pool_desc* pool, const int32_t* block_pairs,
                                 int32_t n_pairs, int32_t* bad_count, void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n_pairs < 0 || !bad_count || (n_pairs > 0 && !block_pairs)) return PA_ERR_INVALID_ARG;
  zero_int_kernel<<<1, 1, 0, (hipStream_t)stream>>>(bad_count);
  if (n_pairs > 0)
    validate_pairs_kernel<<<(unsigned)(((int64_t)n_pairs + 255) / 256), 256, 0,
                            (hipStream_t)stream>>>(block_pairs, n_pairs, pool->num_blocks, bad_count);
  return launch_status();
}

pa_status pa_validate_tables(const pa_pool_desc* pool, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t num_seqs, int32_t max_context_len, int32_t* bad_count,
                             void* stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || !bad_count)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables)))
    return PA_ERR_INVALID_ARG;
  zero_int_kernel<<<1, 1, 0, (hipStream_t)stream>>>(bad_count);
  if (num_seqs > 0)
    validate_kernel<<<num_seqs, 256, 0, (hipStream_t)stream>>>(
        block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
        pool->num_blocks, pool->block_size, bad_count);
  return launch_status();
}

}  // extern "C"
