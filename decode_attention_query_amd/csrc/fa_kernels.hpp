// fa_kernels.hpp -- split plan, vector-ALU decode, LSE merge and the gather hook.
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

// ------------------------------------------------------------------ plan
//
// One workgroup.  For every request: L_b from the page table (clamped so a
// table that breaks its contract cannot send a later kernel outside the
// buffers) and its number of split units; then one descriptor per split unit
// (request, index, count, L_b, page base, first unit), so a decode workgroup
// finds everything about its unit with a single scalar load.  baracuda-kernels
// 0.0.1-alpha.68, src/attention/batch_paged_decode.rs, module doc "Layout":
// request b owns pages indices[indptr[b] .. indptr[b+1]), its last page holds
// last_page_len[b] rows.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const DecodeParams p) {
  // split-merge arrival counters start every call at zero
  for (int i = threadIdx.x; i < p.batch * p.num_qo_heads; i += kPlanThreads) p.arrivals[i] = 0;
  if (p.contig) return;  // a contiguous cache's single length is known on the host
  // Work order: every request's full-length units first, then the shorter
  // last units, so the short work fills the tail of the launch (longest
  // first).  Partial results use a separate numbering, contiguous per request
  // (slot = first slot of the request + index of the unit).
  __shared__ int s_full[kPlanThreads];
  __shared__ int s_part[kPlanThreads];
  __shared__ long long s_rows[kPlanThreads];
  __shared__ int s_carry_full, s_carry_part;
  __shared__ long long s_carry_rows;
  const int tid = threadIdx.x;
  const int T = p.total_used_pages;
  // pass 0 counts the full units of the whole batch (where the partial ones
  // start); pass 1 writes the descriptors
  int total_full = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (tid == 0) {
      s_carry_full = 0;
      s_carry_part = 0;
      s_carry_rows = 0;
    }
    __syncthreads();
    for (int base = 0; base < p.batch; base += kPlanThreads) {
      const int b = base + tid;
      int L = 0, full = 0, part = 0, p0 = 0;
      if (b < p.batch) {
        p0 = min(max(p.indptr[b], 0), T);
        const int p1 = min(max(p.indptr[b + 1], p0), T);
        const int n = p1 - p0;
        const int lpl = min(max(p.last_page_len[b], 0), p.page_size);
        L = n == 0 ? 0 : (n - 1) * p.page_size + lpl;  // < 2^31: host checks T * P
        full = L / p.chunk;
        part = (L % p.chunk != 0 || L == 0) ? 1 : 0;  // an empty request is one empty unit
      }
      // inclusive scans (Hillis-Steele)
      s_full[tid] = full;
      s_part[tid] = part;
      s_rows[tid] = L;
      __syncthreads();
      for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int f = tid >= off ? s_full[tid - off] : 0;
        const int q = tid >= off ? s_part[tid - off] : 0;
        const long long r = tid >= off ? s_rows[tid - off] : 0;
        __syncthreads();
        s_full[tid] += f;
        s_part[tid] += q;
        s_rows[tid] += r;
        __syncthreads();
      }
      if (pass == 1 && b < p.batch) {
        const int first_full = s_carry_full + s_full[tid] - full;
        const int first_part = s_carry_part + s_part[tid] - part;
        const int units = full + part;
        const int slot0 = first_full + first_part;  // units of earlier requests
        p.row_prefix[b] = s_carry_rows + s_rows[tid] - L;
        for (int i = 0; i < full; ++i) {
          const int w = first_full + i;
          if (w < p.units_bound) p.unit_desc[w] = UnitDesc{b, i, units, L, p0, slot0, 0, 0};
        }
        if (part) {
          const int w = total_full + first_part;
          if (w < p.units_bound) p.unit_desc[w] = UnitDesc{b, full, units, L, p0, slot0, 0, 0};
        }
      }
      __syncthreads();
      if (tid == kPlanThreads - 1) {
        s_carry_full += s_full[tid];
        s_carry_part += s_part[tid];
        s_carry_rows += s_rows[tid];
      }
      __syncthreads();
    }
    total_full = s_carry_full;
    __syncthreads();  // everyone has read the carry before pass 1 resets it
  }
  // units past the real count exit at once
  for (int w = s_carry_full + s_carry_part + tid; w < p.units_bound; w += kPlanThreads)
    p.unit_desc[w] = UnitDesc{-1, 0, 0, 0, 0, 0, 0, 0};
  if (tid == 0) p.row_prefix[p.batch] = s_carry_rows;
}

// A split unit: (request, unit within request, units of the request, L_b,
// first partial-result slot of the request, page base).
struct UnitInfo {
  int b, c, n_units, L;
  int u0;
  int32_t page_base;
};

// Returns false for units past the real count.
__device__ inline bool resolve_unit(const DecodeParams &p, int unit, UnitInfo &u) {
  if (p.contig) {
    if (unit >= p.contig_units) return false;
    u.b = 0;
    u.c = unit;
    u.u0 = 0;
    u.n_units = p.contig_units;
    u.L = p.contig_len;
    u.page_base = 0;
    return true;
  }
  typedef const __attribute__((address_space(4))) UnitDesc cdesc;
  const cdesc *d = (cdesc *)p.unit_desc + unit;  // written by the plan kernel
  u.b = d->b;
  u.c = d->c;
  u.n_units = d->n_units;
  u.L = d->L;
  u.page_base = d->page_base;
  u.u0 = d->u0;
  return u.b >= 0;
}

// Writes the combined result of one (request, query head, feature) of a unit:
// the final o / lse if the request has a single unit, else the partial.
template <class E>
__device__ inline void emit(const DecodeParams &p, const UnitInfo &u, int h, int d, float m2,
                            float l, float a) {
  const bool any = l > 0.0f;
  if (u.n_units == 1) {
    const int64_t row = (int64_t)u.b * p.num_qo_heads + h;
    static_cast<typename E::raw *>(p.o)[row * p.head_dim + d] = E::narrow(any ? a / l : 0.0f);
    if (d == 0 && p.lse) p.lse[row] = any ? (m2 + fast_log2(l)) * kLn2 : -INFINITY;
  } else {
    // Partials are read by whichever workgroup merges the request, possibly on
    // another XCD: store them device-coherent (agent-scope atomic stores write
    // through to memory) so no L2 write-back of the whole cache is needed.
    const int64_t row = (int64_t)(u.u0 + u.c) * p.num_qo_heads + h;
    __hip_atomic_store(p.part_o + row * p.head_dim + d, any ? a / l : 0.0f, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0)
      __hip_atomic_store(p.part_lse + row, any ? m2 + fast_log2(l) : -INFINITY,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------- LSE merge

// Device-coherent load of data another workgroup wrote (see finish_split).
__device__ inline float coherent_load(const float *ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
//
// Combines request b's split partials (o_s normalised over its rows, lse_s in
// base 2) for query heads h0 .. h0 + gt - 1; every thread of the 256-thread
// workgroup takes part.  Per head:
//   M = max_s lse_s,  W = sum_s 2^(lse_s - M),
//   o = sum_s 2^(lse_s - M) o_s / W,  lse = (M + log2 W) * ln 2,
// with s running over the request's units in order (one wave per head for M
// and W, fixed butterfly order), so the result is reproducible bit for bit.
template <class E>
__device__ void merge_partials(const DecodeParams &p, int b, int u0, int n, int h0, int gt,
                               float *s_stat /* LDS [32] */) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int hq = p.num_qo_heads;
  for (int g = wave; g < gt; g += 4) {
    float mx = -INFINITY;
    for (int s = lane; s < n; s += kWave) mx = fmaxf(mx, coherent_load(p.part_lse + (int64_t)(u0 + s) * hq + h0 + g));
    mx = wave_max(mx);
    const float ref = safe_ref(mx);
    float w = 0.0f;
    for (int s = lane; s < n; s += kWave)
      w += fast_exp2(coherent_load(p.part_lse + (int64_t)(u0 + s) * hq + h0 + g) - ref);
    w = wave_sum(w);
    if (lane == 0) {
      s_stat[g] = mx;
      s_stat[16 + g] = w;
    }
  }
  __syncthreads();
  const int D = p.head_dim;
  for (int idx = tid; idx < gt * D; idx += 4 * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    const int h = h0 + g;
    const float mx = s_stat[g];
    const float W = s_stat[16 + g];
    const float ref = safe_ref(mx);
    float a = 0.0f;
#pragma unroll 8
    for (int s = 0; s < n; ++s) {
      const int64_t row = (int64_t)(u0 + s) * hq + h;
      a = fmaf(fast_exp2(coherent_load(p.part_lse + row) - ref), coherent_load(p.part_o + row * D + d), a);
    }
    const bool any = W > 0.0f;
    const int64_t orow = (int64_t)b * hq + h;
    static_cast<typename E::raw *>(p.o)[orow * D + d] = E::narrow(any ? a / W : 0.0f);
    if (d == 0 && p.lse) p.lse[orow] = any ? (mx + fast_log2(W)) * kLn2 : -INFINITY;
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
template <class E>
__device__ void finish_split(const DecodeParams &p, const UnitInfo &u, int plane, int h0, int gt,
                             float *s_stat, int *s_last) {
  if (u.n_units <= 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t *counter = p.arrivals + (int64_t)u.b * p.num_qo_heads + plane;
  if (threadIdx.x == 0) *s_last = atomicAdd(counter, 1) == u.n_units - 1;
  __syncthreads();
  if (!*s_last) return;
  merge_partials<E>(p, u.b, u.u0, u.n_units, h0, gt, s_stat);
  if (threadIdx.x == 0) *counter = 0;
}

// ------------------------------------------------------ vector-ALU decode
//
// 4 waves.  A wave reads TPW = 64 / LPT KV rows per step, LPT lanes per row,
// 16 bytes per lane (one global_load_dwordx4), U steps per tile.  Each lane
// keeps, for its row slot, an online-softmax state per query head: running
// max m (base 2), normaliser l and its D / LPT accumulator features
// (ferrox-cuda 0.15.2, src/attn.rs, kernel gqa_decode: the running-max
// rescale of the normaliser and the accumulator; here once per tile instead
// of once per row).  Slots and waves are merged at the end.
template <class E, int D, int GT>
__global__ __launch_bounds__(256) void decode_valu_kernel(const DecodeParams p) {
  constexpr int VEC = 16 / E::kBytes;  // elements per 16-byte lane load
  constexpr int LPT = D / VEC;         // lanes per KV row
  constexpr int TPW = kWave / LPT;     // KV rows per wave step
  constexpr int NW = 4;
  constexpr int U = GT >= 8 ? 2 : 4;   // steps per tile
  constexpr int TILE = NW * TPW * U;   // rows per workgroup iteration
  static_assert(LPT >= 1 && LPT <= kWave && TPW * LPT == kWave, "row split");

  __shared__ float s_acc[NW][GT][D];
  __shared__ float s_m[NW][GT];
  __shared__ float s_l[NW][GT];

  UnitInfo u;
  if (!resolve_unit(p, blockIdx.x, u)) return;
  const int kvh = blockIdx.y / p.n_gblocks;
  const int h0 = kvh * p.group + (blockIdx.y % p.n_gblocks) * GT;
  const int t_begin = u.c * p.chunk;
  const int t_end = min(u.L, t_begin + p.chunk);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int slot = lane / LPT;
  const int vi = lane % LPT;

  float qf[GT][VEC];
  {
    const char *qb = static_cast<const char *>(p.q) +
                     (((int64_t)u.b * p.num_qo_heads + h0) * D + vi * VEC) * E::kBytes;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const uint4 r = *reinterpret_cast<const uint4 *>(qb + (int64_t)g * D * E::kBytes);
      E::widen(r, qf[g]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) qf[g][i] *= p.scale_log2;
    }
  }

  float m[GT], l[GT], acc[GT][VEC];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[g][i] = 0.0f;
  }

  const char *kb = static_cast<const char *>(p.k) + (int64_t)vi * VEC * E::kBytes;
  const char *vb = static_cast<const char *>(p.v) + (int64_t)vi * VEC * E::kBytes;

  for (int t0 = t_begin + wave * TPW * U; t0 < t_end; t0 += TILE) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const int t = t0 + s * TPW + slot;
      valid[s] = t < t_end;
      const int64_t off = kv_row_offset(p, u.page_base, kvh, valid[s] ? t : t_end - 1);
      kr[s] = load16_stream(kb + off * E::kBytes);
      vr[s] = load16_stream(vb + off * E::kBytes);
    }
    float sc[U][GT];
#pragma unroll
    for (int s = 0; s < U; ++s) {
      float kf[VEC];
      E::widen(kr[s], kf);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) dot = fmaf(qf[g][i], kf[i], dot);
        sc[s][g] = dot;
      }
    }
#pragma unroll
    for (int off = 1; off < LPT; off <<= 1) {
#pragma unroll
      for (int s = 0; s < U; ++s)
#pragma unroll
        for (int g = 0; g < GT; ++g) sc[s][g] += __shfl_xor(sc[s][g], off);
    }
    float vf[U][VEC];
#pragma unroll
    for (int s = 0; s < U; ++s) E::widen(vr[s], vf[s]);
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mt = -INFINITY;
#pragma unroll
      for (int s = 0; s < U; ++s) {
        if (!valid[s]) sc[s][g] = -INFINITY;
        mt = fmaxf(mt, sc[s][g]);
      }
      const float mn = fmaxf(m[g], mt);
      const float ref = safe_ref(mn);
      const float alpha = fast_exp2(m[g] - ref);
      float pw[U];
      float psum = 0.0f;
#pragma unroll
      for (int s = 0; s < U; ++s) {
        pw[s] = fast_exp2(sc[s][g] - ref);
        psum += pw[s];
      }
      l[g] = l[g] * alpha + psum;
      m[g] = mn;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        float a = acc[g][i] * alpha;
#pragma unroll
        for (int s = 0; s < U; ++s) a = fmaf(pw[s], vf[s][i], a);
        acc[g][i] = a;
      }
    }
  }

  // merge the row slots of the wave (lanes LPT, 2 LPT, ... apart)
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float ref = safe_ref(mn);
      const float a = fast_exp2(m[g] - ref);
      const float bw = fast_exp2(mo - ref);
      l[g] = l[g] * a + lo * bw;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[g][i] = acc[g][i] * a + __shfl_xor(acc[g][i], off) * bw;
      m[g] = mn;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) s_acc[wave][g][vi * VEC + i] = acc[g][i];
      if (vi == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  // merge the waves; one thread per (query head, feature)
  for (int idx = tid; idx < GT * D; idx += NW * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    const float ref = safe_ref(M);
    float lsum = 0.0f, a = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sw = fast_exp2(s_m[w][g] - ref);
      lsum += s_l[w][g] * sw;
      a += s_acc[w][g][d] * sw;
    }
    emit<E>(p, u, h0 + g, d, M, lsum, a);
  }
  __shared__ float s_stat[32];
  __shared__ int s_last;
  finish_split<E>(p, u, blockIdx.y, h0, GT, s_stat, &s_last);
}

// ------------------------------------------------------------ gather hook
//
// Test-only: copies every valid row of one KV head of one split unit to
// out[(row_prefix[b] + t) * Hkv + kvh, :], using kv_row_offset, the same
// address code as the decode kernels.  16 bytes per lane.
__global__ __launch_bounds__(256) void gather_kernel(const DecodeParams p, void *out,
                                                     int64_t out_rows, int elem_bytes) {
  UnitInfo u;
  if (!resolve_unit(p, blockIdx.x, u)) return;
  const int kvh = blockIdx.y;
  const int t_begin = u.c * p.chunk;
  const int t_end = min(u.L, t_begin + p.chunk);
  const int vecs = p.head_dim * elem_bytes / 16;  // 16-byte vectors per row
  for (int idx = threadIdx.x; idx < (t_end - t_begin) * vecs; idx += blockDim.x) {
    const int t = t_begin + idx / vecs;
    const int vi = idx % vecs;
    const int64_t orow = p.row_prefix[u.b] + t;
    if (orow >= out_rows) continue;
    const int64_t off = kv_row_offset(p, u.page_base, kvh, t);
    const uint4 r =
        *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.k) + off * elem_bytes + vi * 16);
    *reinterpret_cast<uint4 *>(static_cast<char *>(out) +
                               ((orow * p.num_kv_heads + kvh) * p.head_dim) * elem_bytes + vi * 16) = r;
  }
}

}  // namespace fa
