// fa_kernels.hpp -- split-unit schedule, LSE merge, and the append,
// standalone-merge, schedule and read-probe kernels.
//
// Work decomposition (all kernels): a *split unit* is one request's KV rows
// [c * chunk, min(L_b, (c + 1) * chunk)).  A decode workgroup handles one split
// unit for one KV head and a block of GT query heads of that head's group, so
// every K/V byte of the unit is read from HBM once for all GT heads.  A request
// with one unit writes o and lse directly; otherwise each unit writes a
// normalised partial output and its base-2 log-sum-exp, and the workgroup that
// finishes last for that (request, head block) merges all of them, in unit
// order, so the result does not depend on which workgroup that is.
#pragma once

#include "fa_common.hpp"

namespace fa {

// -------------------------------------------------------------- schedule
//
// No separate plan launch: every wave derives its workgroup's split unit from
// the page table on its own (all four waves reach the same answer), with
// cross-lane operations only -- no LDS, no barrier, so a starting workgroup
// does not queue behind the LDS traffic of the workgroup already running on
// its compute unit.  It recomputes every request's length and unit count (a
// few hundred bytes, served by the cache after the first workgroups) and
// selects the unit its work index names.  baracuda-kernels 0.0.1-alpha.68,
// src/attention/batch_paged_decode.rs, module doc "Layout": request b owns
// pages indices[indptr[b] .. indptr[b+1]), its last page holds
// last_page_len[b] rows.
//
// Work order (longest processing time first, so short work fills the tail of
// the launch): every request's full-length units, in request order; then the
// last, shorter units, longest first by length class (kClasses classes of
// chunk / kClasses rows each; request order inside a class).  The order only
// decides which workgroup runs what: partial results have their own
// numbering, contiguous per request (slot = first slot of the request + index
// of the unit), and are merged in that order.
constexpr int kClasses = 16;   // length classes of last units
constexpr int kRegChunks = 4;  // 64-request chunks held in registers at once

// A split unit: request, unit within the request, units of the request, L_b,
// first partial-result slot of the request, page base, and (gather hook) the
// request's first row in a concatenation of all requests' rows (sum L < 2^31).
// With a sliding window the query attends rows [start, L); the units cover
// rows [lo, L), lo = start rounded down to a multiple of 16 so that 16-row
// blocks stay inside pages, and rows below start are masked.
struct UnitInfo {
  int b, c, n_units, L;
  int u0;
  int32_t page_base;
  int row0;
  int lo, start;
};

struct Request {
  int L, full, part, p0, lo, start;
};

// L_b and the unit counts of a request whose pages are indices[p0 .. p0 + n)
// and whose last page holds lpl_raw rows (clamped to [0, P]).
__device__ inline Request make_request(const DecodeParams &p, int p0, int n, int lpl_raw) {
  Request r;
  r.p0 = p0;
  const int lpl = min(max(lpl_raw, 0), p.page_size);
  r.L = n == 0 ? 0 : (n - 1) * p.page_size + lpl;  // < 2^31: the host checks T * P
  r.start = (p.window > 0 && r.L > p.window) ? r.L - p.window : 0;
  r.lo = r.start & ~15;
  const int rows = r.L - r.lo;  // rows the units cover
  r.full = rows / p.chunk;
  r.part = (rows % p.chunk != 0 || rows == 0) ? 1 : 0;  // an empty request is one empty unit
  return r;
}

// Request b on its own (the append kernel): its page range clamped into
// [0, T], so a table that breaks its contract cannot send a kernel outside
// the buffers.
__device__ inline Request request_of(const DecodeParams &p, int b) {
  const int T = p.total_used_pages;
  const int p0 = min(max(p.indptr[b], 0), T);
  const int n = min(max(p.indptr[b + 1], p0), T) - p0;
  return make_request(p, p0, n, p.last_page_len[b]);
}

// Inclusive prefix maximum over the 64 lanes of a wave, for x >= 0 (lanes
// shifted in from outside a row read 0), by the steps of wave_incl_scan.
__device__ inline int wave_incl_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));   // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));   // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));   // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));   // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}

// Length class of a request's last unit, -1 if it has none (chunk is a
// multiple of kClasses).
__device__ inline int length_class(const DecodeParams &p, const Request &r) {
  if (!r.part) return -1;
  return min((r.L - r.lo - r.full * p.chunk) / (p.chunk / kClasses), kClasses - 1);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row of
// 16 lanes, then the row totals broadcast into the following rows (DPP).
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ inline int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// The split unit of work index w; false for indices past the real unit count.
// Every lane of the calling wave takes part; the result is wave-uniform.
// (Forced inline, as are the tile loads and the split merge: with many call
// sites the compiler may otherwise emit them as real calls, whose arguments
// and results then travel through scratch memory.)
template <bool kRows>
__device__ __forceinline__ bool find_unit(const DecodeParams &p, int w, UnitInfo &u) {
  if (p.contig) {  // one request of contig_len rows, known on the host
    if (w >= p.contig_units) return false;
    u.b = 0;
    u.c = w;
    u.u0 = 0;
    u.n_units = p.contig_units;
    u.L = p.contig_len;
    u.page_base = 0;
    u.row0 = 0;
    u.lo = p.contig_lo;
    u.start = p.contig_start;
    return true;
  }
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kGroup = kRegChunks * kWave;  // requests per register group
  const int groups = (p.batch + kGroup - 1) / kGroup;
  Request rq[kRegChunks];
  // Page ranges: with pm_b = max over k <= b of clamp(indptr[k], 0, T),
  // request b owns indices[pm_b .. pm_{b+1}).  A table that keeps its
  // contract (indptr non-decreasing, indptr[B] <= T) gives exactly
  // [indptr[b], indptr[b+1]).  Any other table gets ranges that neither
  // overlap nor leave [0, T), so the requests' split units never number more
  // than units_bound: every unit of a request runs (no counter is left part
  // counted) and no partial lands past the workspace.  pm_carry holds the
  // maximum over the requests of earlier chunks; each pass starts it at 0.
  int pm_carry = 0;
  auto load_group = [&](int g) {
    const int T = p.total_used_pages;
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const int b0 = (g * kRegChunks + j) * kWave;
      if (b0 < p.batch) {
        const int bb = min(b0 + lane, p.batch - 1);  // loads stay in bounds
        const int c0 = min(max(p.indptr[bb], 0), T);
        const int c1 = min(max(p.indptr[bb + 1], 0), T);
        const int pm0 = max(pm_carry, wave_incl_max(c0));
        const int pm1 = max(pm0, c1);
        pm_carry = lane_value(pm1, kWave - 1);
        rq[j] = b0 + lane < p.batch ? make_request(p, pm0, pm1 - pm0, p.last_page_len[bb])
                                    : Request{0, 0, 0, 0, 0, 0};
      }
    }
  };
  auto take = [&](const Request &r, int src, int b0, int c, int n_units, int u0, int row0) {
    u.b = b0 + src;
    u.c = c;
    u.n_units = n_units;
    u.L = lane_value(r.L, src);
    u.u0 = u0;
    u.page_base = lane_value(r.p0, src);
    u.row0 = row0;
    u.lo = lane_value(r.lo, src);
    u.start = lane_value(r.start, src);
  };

  // pass 1: the full-length units, in request order
  int carry_full = 0, carry_units = 0, carry_rows = 0;
  for (int g = 0; g < groups; ++g) {
    load_group(g);
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const int b0 = (g * kRegChunks + j) * kWave;
      if (b0 >= p.batch) break;
      const Request &r = rq[j];
      const int units = r.full + r.part;
      const int i_full = wave_incl_scan(r.full);
      const int i_units = wave_incl_scan(units);
      const int i_rows = kRows ? wave_incl_scan(r.L) : 0;
      const int e_full = carry_full + i_full - r.full;
      const uint64_t own = __ballot(w >= e_full && w < e_full + r.full);
      if (own) {
        const int src = (int)__builtin_ctzll(own);
        take(r, src, b0, w - lane_value(e_full, src), lane_value(units, src),
             carry_units + lane_value(i_units - units, src),
             kRows ? carry_rows + lane_value(i_rows - r.L, src) : 0);
        return true;
      }
      carry_full += lane_value(i_full, kWave - 1);
      carry_units += lane_value(i_units, kWave - 1);
      if (kRows) carry_rows += lane_value(i_rows, kWave - 1);
    }
  }
  if (w >= carry_units) return false;
  const int rank = w - carry_full;  // among the last units

  // pass 2: last units per length class; lane kClasses-1-k counts class k, so
  // the lane order is the work order
  const bool resident = groups == 1;  // rq[] still holds every request
  int hist = 0;
  pm_carry = 0;
  for (int g = 0; g < groups; ++g) {
    if (!resident) load_group(g);
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      if ((g * kRegChunks + j) * kWave >= p.batch) break;
      const int cls = length_class(p, rq[j]);
#pragma unroll
      for (int k = 0; k < kClasses; ++k) {
        const int cnt = __popcll(__ballot(cls == k));
        if (lane == kClasses - 1 - k) hist += cnt;
      }
    }
  }
  const int i_hist = wave_incl_scan(hist);
  const uint64_t hit = __ballot(rank >= i_hist - hist && rank < i_hist);
  const int slot = (int)__builtin_ctzll(hit);
  const int sel_class = kClasses - 1 - slot;
  const int sel_rank = rank - lane_value(i_hist - hist, slot);

  // pass 3: the request holding that rank within its class
  int carry_sel = 0;
  carry_units = 0;
  carry_rows = 0;
  pm_carry = 0;
  for (int g = 0; g < groups; ++g) {
    if (!resident) load_group(g);
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const int b0 = (g * kRegChunks + j) * kWave;
      if (b0 >= p.batch) break;
      const Request &r = rq[j];
      const int units = r.full + r.part;
      const uint64_t sel = __ballot(length_class(p, r) == sel_class);
      const int i_units = wave_incl_scan(units);
      const int i_rows = kRows ? wave_incl_scan(r.L) : 0;
      const bool mine = ((sel >> lane) & 1) && carry_sel + lanes_below(sel) == sel_rank;
      const uint64_t own = __ballot(mine);
      if (own) {
        const int src = (int)__builtin_ctzll(own);
        take(r, src, b0, lane_value(r.full, src), lane_value(units, src),
             carry_units + lane_value(i_units - units, src),
             kRows ? carry_rows + lane_value(i_rows - r.L, src) : 0);
        return true;
      }
      carry_sel += __popcll(sel);
      carry_units += lane_value(i_units, kWave - 1);
      if (kRows) carry_rows += lane_value(i_rows, kWave - 1);
    }
  }
  return false;  // not reached: the class counts hold the rank
}

// Custom mask: whether row t of the unit's request is kept -- bit row0 + t of
// the packed mask, at byte (row0 + t) / 8, bit (row0 + t) % 8, where row0 is
// the rows of all earlier requests (0 for a contiguous cache).  A bit past the
// caller's mask size reads as 0 and is never loaded.
__device__ inline bool mask_keeps(const DecodeParams &p, int row0, int t) {
  const uint32_t bit = (uint32_t)(row0 + t);
  const uint32_t byte = min(bit >> 3, p.mask_bytes - 1);
  return (bit >> 3) < p.mask_bytes && ((p.mask[byte] >> (bit & 7)) & 1);
}

// ------------------------------------------------------------- LSE merge

// Device-coherent load of data another workgroup wrote (see finish_split).
__device__ inline float coherent_load(const float *ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same for 16 bytes: a buffer load with the sc1 cache-policy bit, which
// is what an agent-scope atomic load sets, so the data comes from memory and
// not from a line this XCD's L2 may still hold from an earlier call.  The
// resource covers 2 GiB from `base` (raw buffer, 32-bit data format, the
// gfx9 descriptor word); voff + soff stays far below that.
constexpr int kCachePolicySc1 = 16;

__device__ inline __amdgpu_buffer_rsrc_t coherent_rsrc(const float *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

__device__ inline f32x4 coherent_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicySc1));
}

// The store counterpart: 16 bytes with the sc1 bit (write-through, device
// coherent).
__device__ inline void coherent_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4 v) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, voff, 0,
                                         kCachePolicySc1);
}

// Four outputs at out .. out + 3 in the element type, one vector store.
template <class E>
__device__ inline void store4(typename E::raw *out, const f32x4 &v) {
  if constexpr (E::kBytes == 4) {
    *reinterpret_cast<f32x4 *>(out) = v;
  } else {
    const uint32_t lo = (uint32_t)E::narrow(v[0]) | ((uint32_t)E::narrow(v[1]) << 16);
    const uint32_t hi = (uint32_t)E::narrow(v[2]) | ((uint32_t)E::narrow(v[3]) << 16);
    *reinterpret_cast<uint2 *>(out) = make_uint2(lo, hi);
  }
}

// Writes the combined result of features d .. d + 3 (d a multiple of 4) of one
// (request, query head) of a unit: the final o / lse if the request has a
// single unit (one vector store of the four outputs), else the partial.
template <class E>
__device__ inline void emit(const DecodeParams &p, const UnitInfo &u, int h, int d, float m2,
                            float l, const float (&a)[4]) {
  const bool any = l > 0.0f;
  if (u.n_units == 1) {
    const int64_t row = (int64_t)u.b * p.num_qo_heads + h;
    store4<E>(static_cast<typename E::raw *>(p.o) + row * p.head_dim + d,
              f32x4{any ? a[0] / l : 0.0f, any ? a[1] / l : 0.0f, any ? a[2] / l : 0.0f,
                    any ? a[3] / l : 0.0f});
    if (d == 0 && p.lse) p.lse[row] = any ? (m2 + fast_log2(l)) * kLn2 : -INFINITY;
  } else {
    // Partials are read by whichever workgroup merges the request, possibly on
    // another XCD: store them device-coherent (sc1 stores, what agent-scope
    // atomic stores compile to, write through to memory) so no L2 write-back
    // of the whole cache is needed.  One 16-byte store per four features,
    // relative to the unit's partial block (a workgroup-uniform base).
    const int64_t row = (int64_t)(u.u0 + u.c) * p.num_qo_heads + h;
    const __amdgpu_buffer_rsrc_t r =
        coherent_rsrc(p.part_o + (int64_t)(u.u0 + u.c) * p.num_qo_heads * p.head_dim);
    coherent_store4(r, (uint32_t)((h * p.head_dim + d) * 4),
                    f32x4{any ? a[0] / l : 0.0f, any ? a[1] / l : 0.0f, any ? a[2] / l : 0.0f,
                          any ? a[3] / l : 0.0f});
    if (d == 0)
      __hip_atomic_store(p.part_lse + row, any ? m2 + fast_log2(l) : -INFINITY,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Combines request b's split partials (o_s normalised over its rows, lse_s in
// base 2) for query heads h0 .. h0 + gt - 1; every thread of the nw-wave
// workgroup takes part.  Per head:
//   M = max_s lse_s,  W = sum_s 2^(lse_s - M),
//   o = sum_s 2^(lse_s - M) o_s / W,  lse = (M + log2 W) * ln 2,
// with s running over the request's units in order (one wave per head for M
// and W, fixed butterfly order), so the result is reproducible bit for bit.
//
// Latency: the merge runs at the very end of one workgroup per (request, head
// block), so it is kept to few dependent memory round trips and little code
// (it runs once per workgroup, from a cold instruction cache).  With up to 64
// units, each wave loads the lse of four of its heads at a time (one unit per
// lane) and writes the weights 2^(lse_s - M) straight to LDS (s_w, the
// kernel's tile area, free by now); with more, the lse is read per head and
// the weights of up to `cap` units at a time are staged.  The partial outputs
// are then read 16 bytes per load, one 4-feature column per thread, kDepth
// units in flight (kDepth is what the kernel's register budget leaves room
// for) and the last units four at a time.
template <class E, int kDepth>
__device__ __forceinline__ void merge_partials(const DecodeParams &p, int b, int u0, int n, int h0, int gt, int nw,
                               float *s_stat /* LDS [2 kStatHeads] */, float *s_w,
                               int w_cap) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nthreads = nw * kWave;
  const int hq = p.num_qo_heads;
  const int D = p.head_dim;
  const float *lse_base = p.part_lse + (int64_t)u0 * hq + h0;
  const int cap = max(1, w_cap / gt);  // units whose weights fit s_w at once
  const bool resident = n <= kWave && n <= cap;
  if (resident) {
    const float *lrow = lse_base + (int64_t)min(lane, n - 1) * hq;
    for (int g0 = wave; g0 < gt; g0 += 4 * nw) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = coherent_load(lrow + min(g0 + j * nw, gt - 1));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = g0 + j * nw;
        if (g < gt) {
          const float x = lane < n ? v[j] : -INFINITY;
          const float mx = wave_max(x);
          const float e = lane < n ? fast_exp2(x - safe_ref(mx)) : 0.0f;
          const float w = wave_sum(e);
          if (lane < n) s_w[lane * gt + g] = e;
          if (lane == 0) {
            s_stat[g] = mx;
            s_stat[kStatHeads + g] = w;
          }
        }
      }
    }
    __syncthreads();
  } else {
    for (int g = wave; g < gt; g += nw) {
      float mx = -INFINITY;
      for (int s = lane; s < n; s += kWave)
        mx = fmaxf(mx, coherent_load(lse_base + (int64_t)s * hq + g));
      mx = wave_max(mx);
      const float ref = safe_ref(mx);
      float w = 0.0f;
      for (int s = lane; s < n; s += kWave)
        w += fast_exp2(coherent_load(lse_base + (int64_t)s * hq + g) - ref);
      w = wave_sum(w);
      if (lane == 0) {
        s_stat[g] = mx;
        s_stat[kStatHeads + g] = w;
      }
    }
  }
  const int q4 = D / 4;  // 4-feature columns per head
  const int cols = gt * q4;
  const uint32_t ustride = (uint32_t)hq * (uint32_t)D * 4u;  // bytes between units
  // uniform trip counts: every thread reaches every barrier
  for (int c0 = 0; c0 < cols; c0 += nthreads) {
    const int c = min(c0 + tid, cols - 1);
    const int g = c / q4;
    const uint32_t voff = (uint32_t)(g * D + 4 * (c - g * q4)) * 4u;
    const bool wave_live = c0 + wave * kWave < cols;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < n; s0 += cap) {
      const int cn = min(cap, n - s0);
      if (!resident && (c0 == 0 || n > cap)) {  // stage the weights of units s0 .. s0 + cn
        __syncthreads();                        // s_stat written; earlier weights no longer read
        for (int i = tid; i < cn * gt; i += nthreads) {
          const int s = i / gt;
          const int gg = i - s * gt;
          s_w[i] = fast_exp2(coherent_load(lse_base + (int64_t)(s0 + s) * hq + gg) -
                             safe_ref(s_stat[gg]));
        }
        __syncthreads();
      }
      if (!wave_live) continue;
      const float *o_base = p.part_o + ((int64_t)(u0 + s0) * hq + h0) * D;
      int sb = 0;
      for (; sb + kDepth <= cn; sb += kDepth) {
        const __amdgpu_buffer_rsrc_t r = coherent_rsrc(o_base + (int64_t)sb * hq * D);
        f32x4 x[kDepth];
#pragma unroll
        for (int k = 0; k < kDepth; ++k) x[k] = coherent_load4(r, voff, k * ustride);
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
          const float w = s_w[(sb + k) * gt + g];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, x[k][e], acc[e]);
        }
      }
      for (; sb < cn; sb += 4) {  // the last 1 .. kDepth - 1 units
        const int rem = cn - sb;
        const __amdgpu_buffer_rsrc_t r = coherent_rsrc(o_base + (int64_t)sb * hq * D);
        f32x4 x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = coherent_load4(r, voff, min(k, rem - 1) * ustride);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float w = s_w[(sb + min(k, rem - 1)) * gt + g];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = k < rem ? fmaf(w, x[k][e], acc[e]) : acc[e];
        }
      }
    }
    if (c0 + tid < cols) {
      const float mx = s_stat[g];
      const float W = s_stat[kStatHeads + g];
      const bool any = W > 0.0f;
      const int64_t orow = (int64_t)b * hq + h0 + g;
      const int d = 4 * (c - g * q4);
      const f32x4 o4 = any ? acc / W : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      store4<E>(static_cast<typename E::raw *>(p.o) + orow * D + d, o4);
      if (d == 0 && p.lse) p.lse[orow] = any ? (mx + fast_log2(W)) * kLn2 : -INFINITY;
    }
  }
}

// After a split unit has written its partials: count it in, and if it is the
// last unit of its (request, head block) to finish, merge them all.
//
// Ordering: every wave waits until its device-coherent partial stores have
// completed (s_waitcnt 0), the barrier gathers the waves, and only then does
// one thread count the unit in with a device-scope atomic.  The workgroup that
// sees the final count reads the partials with device-coherent loads, which
// go to memory rather than to a possibly stale L2 line.  No cache-wide
// write-back or invalidate (what a device-scope fence would emit, once per
// workgroup) is needed, because no non-coherent data crosses workgroups.
//
// The counter holds (kArrivalMark << kCountBits) | units counted.  A unit
// counts in with one atomic add, which also returns the mark; a counter
// without it is stale (never used, or left by other data).  Then the unit
// sets it to rest, (mark, 0), with compare-and-swap -- unless another unit
// already did -- and adds again.  Adds made to the stale value vanish with it,
// but every unit that made one saw the stale value and adds again after the
// swap, so each unit is counted once.  The swap loop ends: a failed swap means
// another unit added to the stale value (fewer than n_units can) or set the
// mark (which ends the loop).  The merging workgroup puts the counter back to
// rest, so the next call, or a replay of a captured graph, counts in with a
// single add per unit; only a counter's first use pays for the swap.
__device__ inline int count_in(unsigned long long *counter) {
  const unsigned long long tag = kArrivalMark;
  unsigned long long old = atomicAdd(counter, 1ull);
  if ((old >> kCountBits) != tag) {
    unsigned long long seen = __hip_atomic_load(counter, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    while ((seen >> kCountBits) != tag) {
      const unsigned long long prev = atomicCAS(counter, seen, tag << kCountBits);
      if (prev == seen) break;
      seen = prev;
    }
    old = atomicAdd(counter, 1ull);
  }
  return int(old & ((1ull << kCountBits) - 1));
}

__device__ inline bool count_in_is_last(unsigned long long *counter, int n_units) {
  return count_in(counter) + 1 == n_units;
}

// Work index of a workgroup that starts after the first resident round: the
// next of n tickets, in the order workgroups reach the counter, so compute
// units (and dies) that finish early take more of the remaining, shorter
// units instead of each running a fixed share of the launch.  The counter
// works like an arrival counter; the workgroup that draws the last ticket is
// the last to touch it and puts it back to rest for the next call.
__device__ inline int draw_ticket(unsigned long long *counter, int n) {
  const int t = count_in(counter);
  if (t == n - 1)
    __hip_atomic_store(counter, kArrivalMark << kCountBits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return t;
}

template <class E, int kDepth>
__device__ __forceinline__ void finish_split(const DecodeParams &p, const UnitInfo &u, int plane, int h0, int gt, int nw,
                             float *s_stat, int *s_last, float *s_w, int w_cap) {
  if (u.n_units <= 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned long long *counter = reinterpret_cast<unsigned long long *>(
      p.arrivals + ((int64_t)u.b * p.num_qo_heads + plane) * kArrivalStride);
  if (threadIdx.x == 0) *s_last = count_in_is_last(counter, u.n_units);
  __syncthreads();
  if (!*s_last) return;
  if (threadIdx.x == 0)
    __hip_atomic_store(counter, kArrivalMark << kCountBits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  merge_partials<E, kDepth>(p, u.b, u.u0, u.n_units, h0, gt, nw, s_stat, s_w, w_cap);
}

// ------------------------------------------------------- standalone merge
//
// The combine step of split-KV decode as a kernel of its own, for partial
// results made outside one decode call: the shares of one request's rows
// decoded on different devices (context-parallel decode, after the partials
// have been gathered), or a caller's own split.  For each output row, S
// partials, each o_s normalised over its rows and lse_s its natural-log
// log-sum-exp:
//   M = max_s lse_s,  W = sum_s exp(lse_s - M),
//   o = sum_s exp(lse_s - M) o_s / W,  lse = M + ln W,
// with s running 0 .. S-1 in order in every thread, so the result is
// reproducible bit for bit.  A partial with lse_s = -inf covers no rows: its
// weight is 0 and its o_s (whatever it holds) does not reach the result.  A
// row whose partials are all empty gets o = 0 and lse = -inf.
//
// Layout: o_parts [S, rows, D] f32, lse_parts [S, rows] f32, o [rows, D] T,
// lse [rows] f32.  One thread per 4-feature column of a row (D / 4 threads per
// row, a row's threads adjacent), so every partial byte is read once, 16 bytes
// per load; the S lse values of a row are read by all its threads from the
// same addresses (one request per wave and address).  kDepth partials are
// loaded before any is used, so that many loads are in flight per thread.
template <class E>
__global__ __launch_bounds__(256) void merge_states_kernel(const float *o_parts,
                                                           const float *lse_parts,
                                                           typename E::raw *o, float *lse,
                                                           int rows, int n_parts, int d) {
  constexpr int kDepth = 8;
  const int q4 = d / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / q4;
  if (row >= rows) return;
  const int col = 4 * (int)(idx - row * q4);
  const int64_t lstride = rows;                    // between the lse of two partials
  const int64_t ostride = (int64_t)rows * d;       // between two partial outputs
  const float *lrow = lse_parts + row;
  const float *orow = o_parts + row * d + col;
  float mx = -INFINITY;
  for (int s = 0; s < n_parts; ++s) mx = fmaxf(mx, lrow[s * lstride]);
  const float ref = safe_ref(mx);
  float W = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < n_parts; s0 += kDepth) {
    f32x4 x[kDepth];
    float w[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int s = min(s0 + k, n_parts - 1);
      x[k] = *reinterpret_cast<const f32x4 *>(orow + s * ostride);
      w[k] = s0 + k < n_parts ? fast_exp2((lrow[s * lstride] - ref) * kLog2e) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      W += w[k];
      if (w[k] > 0.0f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[k], x[k][e], acc[e]);
      }
    }
  }
  const bool any = W > 0.0f;
  const f32x4 o4 = any ? acc / W : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  store4<E>(o + row * d + col, o4);
  if (col == 0 && lse) lse[row] = any ? mx + fast_log2(W) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------- schedule hook
//
// Test-only: the unit each work index runs, from find_unit, 8 int32 per index:
// b (-1 past the real count), c, n_units, L, u0, page base, row0 low, row0 high.
__global__ __launch_bounds__(256) void schedule_kernel(const DecodeParams p, int32_t *out) {
  UnitInfo u;
  const bool ok = find_unit<true>(p, blockIdx.x, u);
  if (threadIdx.x != 0) return;
  int32_t *o = out + 8 * (int64_t)blockIdx.x;
  if (!ok) {
    o[0] = -1;
    for (int i = 1; i < 8; ++i) o[i] = 0;
    return;
  }
  o[0] = u.b;
  o[1] = u.c;
  o[2] = u.n_units;
  o[3] = u.L;
  o[4] = u.u0;
  o[5] = u.page_base;
  o[6] = u.row0;
  o[7] = 0;
}

// -------------------------------------------------------------- KV append
//
// Decode-time append (baracuda-kernels 0.0.1-alpha.68, batch_paged_decode.rs,
// module doc "Companion plans": the new K/V slices are written into the paged
// store before decode).  The page table passed in already counts the new
// token, so request b's new row is its last valid row L_b - 1; L_b = 0 writes
// nothing.  One 64-lane workgroup per (request, KV head), 16 bytes per lane
// (a row is 128 to 1024 bytes).  Page ids are clamped like every other read of
// the table, so a broken table cannot send a write outside the K/V buffers.
__global__ __launch_bounds__(64) void append_kernel(const DecodeParams p, const char *k_new,
                                                    const char *v_new, char *k_data,
                                                    char *v_data, int elem_bytes) {
  const int b = blockIdx.x / p.num_kv_heads;
  const int g = blockIdx.x - b * p.num_kv_heads;
  const Request r = request_of(p, b);
  if (r.L == 0) return;
  const int row_bytes = p.head_dim * elem_bytes;
  const int64_t dst = kv_row_offset(p, r.p0, g, r.L - 1) * elem_bytes;
  const int64_t src = ((int64_t)b * p.num_kv_heads + g) * row_bytes;
  for (int i = threadIdx.x * 16; i < row_bytes; i += 64 * 16) {
    *reinterpret_cast<uint4 *>(k_data + dst + i) = *reinterpret_cast<const uint4 *>(k_new + src + i);
    *reinterpret_cast<uint4 *>(v_data + dst + i) = *reinterpret_cast<const uint4 *>(v_new + src + i);
  }
}

// --------------------------------------------------------- counter check
//
// Test-only: how many of a workspace's counters (n arrival counters kStride
// words apart, then the work-ticket counter) carry the rest mark with a
// non-zero count, i.e. were left part counted.  A call on a workspace leaves
// every counter it used at rest; one left part counted would make the next
// call's merge start early.  One workgroup; out[0] = the count.
__global__ __launch_bounds__(256) void counter_check_kernel(const uint64_t *arrivals, int64_t n,
                                                            const uint64_t *ticket,
                                                            int32_t *out) {
  __shared__ int s_count;
  if (threadIdx.x == 0) s_count = 0;
  __syncthreads();
  int mine = 0;
  for (int64_t i = threadIdx.x; i <= n; i += blockDim.x) {
    const uint64_t c = i < n ? arrivals[i * kArrivalStride] : ticket[0];
    const uint64_t count = c & ((1ull << kCountBits) - 1);
    mine += (c >> kCountBits) == kArrivalMark && count != 0;
  }
  atomicAdd(&s_count, mine);
  __syncthreads();
  if (threadIdx.x == 0) out[0] = s_count;
}

// ------------------------------------------------------------- read probe
//
// Measurement only: streams a buffer of whole 8 KiB blocks with the decode
// kernels' load shape (each wave instruction reads 1 KiB contiguous, 16 bytes
// per lane, non-temporal), eight instructions in flight per wave, so a
// benchmark can state the read bandwidth this shape reaches on the device.
// The loaded words are folded into one value that is stored only if it equals
// a fixed constant, which keeps the loads without writing anything.
constexpr int kProbeBlock = 8192;
__global__ __launch_bounds__(256) void read_probe_kernel(const char *buf, int64_t n_blocks,
                                                         uint32_t *sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x / kWave);
  const int64_t n_waves = (int64_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (int64_t bi = wave; bi < n_blocks; bi += n_waves) {
    const char *blk = buf + bi * kProbeBlock + lane * 16;
    uint4 r[kProbeBlock / 1024];
#pragma unroll
    for (int i = 0; i < kProbeBlock / 1024; ++i) r[i] = load16_stream(blk + i * 1024);
#pragma unroll
    for (int i = 0; i < kProbeBlock / 1024; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace fa
