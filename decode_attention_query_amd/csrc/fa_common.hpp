// fa_common.hpp -- launch parameters and device helpers shared by the decode
// kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_limits.hpp"

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Division of a 32-bit unsigned n by a divisor d fixed at launch, by the
// round-up multiply method: with s = ceil(log2 d) and
// magic = floor(2^32 (2^s - d) / d) + 1, the quotient is (umulhi(n, magic) + n) >> s
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994).  Valid for 1 <= d < 2^31 and every n < 2^32.
struct FastDiv {
  uint32_t d;
  uint32_t magic;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.magic = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, FastDiv f) {
#ifdef __HIP_DEVICE_COMPILE__
  uint32_t hi = __umulhi(n, f.magic);
#else
  uint32_t hi = (uint32_t)(((uint64_t)n * f.magic) >> 32);
#endif
  return (uint32_t)(((uint64_t)hi + n) >> f.shift);
}

// Everything a decode launch needs.  Passed by value as the kernel argument.
struct DecodeParams {
  // tensors
  const void *q;                  // [B, Hq, D] (contiguous: B = 1)
  const void *k;                  // paged [pages, Hkv, P, D]; contiguous [Hkv, max_kv_len, D]
  const void *v;
  void *o;                        // [B, Hq, D]
  float *lse;                     // [B, Hq] or null (contiguous only)
  const int32_t *indices;         // [total_used_pages]
  const int32_t *indptr;          // [B + 1]
  const int32_t *last_page_len;   // [B]
  // geometry
  int batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_total_pages;
  int total_used_pages;
  int group;          // Hq / Hkv
  int n_gblocks;      // workgroups per KV head along the query group
  int heads_per_unit; // query heads per head block (the group, or 16; the last
                      // block of a group may hold fewer)
  int planes;         // Hkv * n_gblocks: workgroups per split unit
  float scale_log2;   // scale * log2(e): scores live in the base-2 domain
  FastDiv page_div;   // row -> (page slot, row in page)
  // split-KV plan
  int chunk;          // KV rows per split unit (a multiple of 256)
  int units_bound;    // work indices launched; those past the real unit count exit at once
  int contig;         // 1: contiguous cache (a single page of max_kv_len rows)
  int nhd;            // 1: token-major K/V ([.., P, Hkv, D]); 0: heads-major ([.., Hkv, P, D])
  int uniform_blocks; // 1: every 16-row block starting at a multiple of 16 lies in one page
  int contig_len;     // contiguous: valid_kv_len
  int contig_units;   // contiguous: units over rows [contig_lo, valid_kv_len), at least 1
  int contig_start;   // contiguous: first row the query attends (sliding window)
  int contig_lo;      // contiguous: contig_start rounded down to a multiple of 16
  // score variants
  int window;         // > 0: the query attends only each request's last `window` rows
  float softcap2;     // > 0: base-2 scores x -> softcap2 * tanh(x / softcap2) (cap * log2 e)
  float softcap2_inv; // 1 / softcap2
  const float *alibi; // [Hq] ALiBi slopes (natural-log units) or null
  const uint8_t *mask; // custom mask, one bit per row of every request (keep = 1), or null
  uint32_t mask_bytes; // its size; bits past it read as 0
  // workspace regions
  float *part_lse;        // [units_bound, Hq]     base-2 lse of each split's partial
  float *part_o;          // [units_bound, Hq, D]  normalised partial outputs
  uint64_t *arrivals;     // [B, Hq, kArrivalStride]  per (request, head block), first word:
                          // kArrivalMark << kCountBits | units done
  uint64_t *tickets;      // one counter line, same format: work indices handed out
  int ticket_from;        // workgroups from this launch index on draw their work index
};

// An arrival counter at rest holds kArrivalMark << kCountBits (count 0): the
// merging workgroup leaves it so.  A counter without the mark -- a workspace
// never used, or last used for something else -- is stale and is set to rest
// by the first unit that meets it, so the workspace needs no clearing.  The
// mark's upper 32 bits are a NaN with a payload no arithmetic produces, so
// left-over partial results (finite floats) never look like a counter.
constexpr unsigned long long kArrivalMark = 0x7FF3A5C35Aull;  // 40 bits


// Query heads a decode workgroup serves at most (two 16-column head blocks):
// the split merge keeps a maximum and a normaliser per head in LDS.
constexpr int kStatHeads = 32;

// ---------------------------------------------------------------- elements
//
// Each element type knows how to widen a 16-byte vector to f32 and how to
// round an f32 back to itself (round-to-nearest-even).

struct F32 {
  static constexpr int kBytes = 4;
  using raw = float;
  __device__ static inline void widen(const uint4 &r, float *out) {
    out[0] = __uint_as_float(r.x);
    out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z);
    out[3] = __uint_as_float(r.w);
  }
  __device__ static inline raw narrow(float f) { return f; }
};

struct BF16 {
  static constexpr int kBytes = 2;
  using raw = uint16_t;
  __device__ static inline void widen(const uint4 &r, float *out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline raw narrow(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  }
};

struct F16 {
  static constexpr int kBytes = 2;
  using raw = uint16_t;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  __device__ static inline void widen(const uint4 &r, float *out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h2 h = __builtin_bit_cast(h2, w[i]);
      out[2 * i] = (float)h[0];
      out[2 * i + 1] = (float)h[1];
    }
  }
  __device__ static inline raw narrow(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
};

// ------------------------------------------------------------ loads

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 16-byte load with the streaming (non-temporal) hint: K/V rows are read once.
__device__ inline uint4 load16_stream(const void *ptr) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(ptr));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ------------------------------------------------------------ math helpers

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// The shift used for an online-softmax rescale: the running max, or 0 while no
// valid score has been seen (keeps -inf - -inf out of the exponent).
__device__ inline float safe_ref(float m) { return m == -INFINITY ? 0.0f : m; }

// Element offset of row r of page `page`, KV head kvh.  Heads-major pages are
// [Hkv, P, D] (baracuda-kernels 0.0.1-alpha.68, src/attention/batch_paged_decode.rs,
// module doc "Layout"); token-major pages are [P, Hkv, D], row t of head g at
// (t * Hkv + g) * D as in ferrox-cuda 0.15.2, src/attn.rs (gqa_decode kernel
// source).  A contiguous cache is the single page 0 of P = max_kv_len rows.
template <bool kNhd>
__device__ inline int64_t kv_elem_offset(const DecodeParams &p, int64_t page, int kvh,
                                         uint32_t r) {
  if (kNhd) return ((page * p.page_size + r) * p.num_kv_heads + kvh) * (int64_t)p.head_dim;
  return ((page * p.num_kv_heads + kvh) * (int64_t)p.page_size + r) * p.head_dim;
}

// Element offset of KV row t (of request b, KV head kvh), lane vector vi
// excluded.  Paged: page = indices[page_base + t / P], row = t % P.  Page ids
// are clamped into the pool so that a table breaking its contract cannot make
// a kernel read outside the K/V buffers.
__device__ inline int64_t kv_row_offset(const DecodeParams &p, int32_t page_base, int kvh,
                                        int t) {
  int64_t page = 0;
  uint32_t row = (uint32_t)t;
  if (!p.contig) {
    const uint32_t slot = fastdiv((uint32_t)t, p.page_div);
    row = (uint32_t)t - slot * (uint32_t)p.page_size;
    int32_t id = p.indices[page_base + slot];
    id = min(max(id, 0), p.num_total_pages - 1);
    page = id;
  }
  return p.nhd ? kv_elem_offset<true>(p, page, kvh, row) : kv_elem_offset<false>(p, page, kvh, row);
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48), in registers: v_permlane16_swap with both operands = v returns,
// at lane l, the values of lanes l & ~16 and l | 16 (rows 0-1 and 2-3
// paired), and v_permlane32_swap those of l & 31 and l | 32; combining each
// pair gives every lane the same bits.  No LDS traffic, unlike a lane shuffle.
//
// Both results of a swap pass through `opaque` (an empty asm statement on a
// register) before use: when the two results feed one operation, this
// compiler otherwise reads the first result for both operands.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ inline void swap_rows16(float v, float &a, float &b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  a = __builtin_bit_cast(float, opaque(r[0]));
  b = __builtin_bit_cast(float, opaque(r[1]));
}

__device__ inline void swap_halves32(float v, float &a, float &b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  a = __builtin_bit_cast(float, opaque(r[0]));
  b = __builtin_bit_cast(float, opaque(r[1]));
}

__device__ inline float rows4_max(float v) {
  float a, b;
  swap_rows16(v, a, b);
  swap_halves32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

__device__ inline float rows4_sum(float v) {
  float a, b;
  swap_rows16(v, a, b);
  swap_halves32(a + b, a, b);
  return a + b;
}

// Value of a partner lane within each 16-lane row (DPP): quad_perm [1,0,3,2]
// and [2,3,0,1] pair lanes l ^ 1 and l ^ 2; row_half_mirror (lane i of each
// 8-lane half -> 7 - i) pairs the two quads of a half, row_mirror (i -> 15 -
// i) the two halves of a row.  After each combining step all lanes of the
// group hold the same bits, so the pairings reduce like an xor butterfly.
template <int kCtrl>
__device__ inline float dpp_partner(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Max and sum over all 64 lanes (every lane active), in registers.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_partner<kDppXor1>(v));
  v = fmaxf(v, dpp_partner<kDppXor2>(v));
  v = fmaxf(v, dpp_partner<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_partner<kDppMirror>(v));
  return rows4_max(v);
}

__device__ inline float wave_sum(float v) {
  v += dpp_partner<kDppXor1>(v);
  v += dpp_partner<kDppXor2>(v);
  v += dpp_partner<kDppHalfMirror>(v);
  v += dpp_partner<kDppMirror>(v);
  return rows4_sum(v);
}

}  // namespace fa
