// fa_kernels.hpp -- split plan, vector-ALU decode, LSE merge and the gather hook.
//
// Work decomposition (all kernels): a *split unit* is one request's KV rows
// [c * chunk, min(L_b, (c + 1) * chunk)).  A decode workgroup handles one split
// unit for one KV head and a block of GT query heads of that head's group, so
// every K/V byte of the unit is read from HBM once for all GT heads.  A request
// with one unit writes o and lse directly; otherwise each unit writes a
// normalised partial output and its base-2 log-sum-exp, and the merge kernel
// combines them in a fixed order.
#pragma once

#include "fa_common.hpp"

namespace fa {

// ------------------------------------------------------------------ plan
//
// One workgroup.  For every request: L_b from the page table (clamped so a
// table that breaks its contract cannot send a later kernel outside the
// buffers), its number of split units, and the prefix sums that map a split
// unit back to its request.  baracuda-kernels 0.0.1-alpha.68,
// src/attention/batch_paged_decode.rs, module doc "Layout": request b owns
// pages indices[indptr[b] .. indptr[b+1]), its last page holds
// last_page_len[b] rows.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const DecodeParams p) {
  __shared__ int s_units[kPlanThreads];
  __shared__ long long s_rows[kPlanThreads];
  __shared__ int s_carry_units;
  __shared__ long long s_carry_rows;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_carry_units = 0;
    s_carry_rows = 0;
  }
  __syncthreads();
  const int T = p.total_used_pages;
  for (int base = 0; base < p.batch; base += kPlanThreads) {
    const int b = base + tid;
    int L = 0, units = 0, p0 = 0;
    if (b < p.batch) {
      p0 = min(max(p.indptr[b], 0), T);
      const int p1 = min(max(p.indptr[b + 1], p0), T);
      const int n = p1 - p0;
      const int lpl = min(max(p.last_page_len[b], 0), p.page_size);
      L = n == 0 ? 0 : (n - 1) * p.page_size + lpl;  // < 2^31: host checks T * P
      units = L == 0 ? 1 : (L + p.chunk - 1) / p.chunk;
      p.seq_len[b] = L;
      p.page_base[b] = p0;
    }
    // inclusive scans (Hillis-Steele) of the unit counts and row counts
    s_units[tid] = units;
    s_rows[tid] = L;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int u = tid >= off ? s_units[tid - off] : 0;
      const long long r = tid >= off ? s_rows[tid - off] : 0;
      __syncthreads();
      s_units[tid] += u;
      s_rows[tid] += r;
      __syncthreads();
    }
    const int first_unit = s_carry_units + s_units[tid] - units;
    const long long first_row = s_carry_rows + s_rows[tid] - L;
    if (b < p.batch) {
      p.unit_prefix[b] = min(first_unit, p.units_bound);
      p.row_prefix[b] = first_row;
      for (int i = 0; i < units; ++i) {
        const int u = first_unit + i;
        if (u < p.units_bound) p.unit_req[u] = b;
      }
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) {
      s_carry_units += s_units[tid];
      s_carry_rows += s_rows[tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    p.unit_prefix[p.batch] = min(s_carry_units, p.units_bound);
    p.row_prefix[p.batch] = s_carry_rows;
  }
}

// Resolves split unit blockIdx.x to (request, unit within request, units of
// the request, L_b, page base).  Returns false for units past the real count.
struct UnitInfo {
  int b, c, n_units, L;
  int32_t page_base;
};

__device__ inline bool resolve_unit(const DecodeParams &p, int unit, UnitInfo &u) {
  if (p.contig) {
    if (unit >= p.contig_units) return false;
    u.b = 0;
    u.c = unit;
    u.n_units = p.contig_units;
    u.L = p.contig_len;
    u.page_base = 0;
    return true;
  }
  if (unit >= p.unit_prefix[p.batch]) return false;
  u.b = p.unit_req[unit];
  const int u0 = p.unit_prefix[u.b];
  u.c = unit - u0;
  u.n_units = p.unit_prefix[u.b + 1] - u0;
  u.L = p.seq_len[u.b];
  u.page_base = p.page_base[u.b];
  return true;
}

// Writes the combined result of one (request, query head, feature) of a unit:
// the final o / lse if the request has a single unit, else the partial.
template <class E>
__device__ inline void emit(const DecodeParams &p, const UnitInfo &u, int unit, int h, int d,
                            float m2, float l, float a) {
  const bool any = l > 0.0f;
  if (u.n_units == 1) {
    const int64_t row = (int64_t)u.b * p.num_qo_heads + h;
    static_cast<typename E::raw *>(p.o)[row * p.head_dim + d] = E::narrow(any ? a / l : 0.0f);
    if (d == 0 && p.lse) p.lse[row] = any ? (m2 + fast_log2(l)) * kLn2 : -INFINITY;
  } else {
    const int64_t row = (int64_t)unit * p.num_qo_heads + h;
    p.part_o[row * p.head_dim + d] = any ? a / l : 0.0f;
    if (d == 0) p.part_lse[row] = any ? m2 + fast_log2(l) : -INFINITY;
  }
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
    emit<E>(p, u, blockIdx.x, h0 + g, d, M, lsum, a);
  }
}

// ------------------------------------------------------------- LSE merge
//
// One wave per (request, query head).  Combines the request's split partials
// (o_s normalised over its rows, lse_s in base 2):
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
//   lse = (M + log2 sum_s w_s) * ln 2,
// summing over s in increasing order (fixed, so the result is reproducible).
// Requests with a single unit were written by the decode kernel and are left.
template <class E>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeParams p) {
  const int item = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (item >= p.batch * p.num_qo_heads) return;
  const int b = item / p.num_qo_heads;
  const int h = item % p.num_qo_heads;
  int u0, n;
  if (p.contig) {
    u0 = 0;
    n = p.contig_units;
  } else {
    u0 = p.unit_prefix[b];
    n = p.unit_prefix[b + 1] - u0;
  }
  if (n <= 1) return;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, p.part_lse[(int64_t)(u0 + s) * p.num_qo_heads + h]);
  const float ref = safe_ref(M);
  constexpr int kMaxPerLane = 256 / kWave;
  float a[kMaxPerLane] = {0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
  for (int s = 0; s < n; ++s) {
    const int64_t row = (int64_t)(u0 + s) * p.num_qo_heads + h;
    const float w = fast_exp2(p.part_lse[row] - ref);
    wsum += w;
    const float *po = p.part_o + row * p.head_dim;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int d = lane + j * kWave;
      if (d < p.head_dim) a[j] = fmaf(w, po[d], a[j]);
    }
  }
  const int64_t out_row = (int64_t)b * p.num_qo_heads + h;
  const bool any = wsum > 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int d = lane + j * kWave;
    if (d < p.head_dim)
      static_cast<typename E::raw *>(p.o)[out_row * p.head_dim + d] =
          E::narrow(any ? a[j] / wsum : 0.0f);
  }
  if (lane == 0 && p.lse) p.lse[out_row] = any ? (M + fast_log2(wsum)) * kLn2 : -INFINITY;
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
