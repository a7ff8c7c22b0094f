// fa_decode.hip -- the C ABI of the decode library: workspace carve-up, kernel
// dispatch and the entry points (argument checks and the launch plan are in
// fa_plan.hpp).  See include/fa_decode.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/fa_decode.h"
#include "../../include/fa_decode_debug.h"
#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_mfma.hpp"
#include "fa_plan.hpp"

namespace {

using fa::DecodeParams;

using namespace fa_plan;

void carve(DecodeParams &p, const HostPlan &hp, void *ws) {
  char *w = static_cast<char *>(ws);
  p.part_lse = reinterpret_cast<float *>(w + hp.part_lse);
  p.part_o = reinterpret_cast<float *>(w + hp.part_o);
  p.arrivals = reinterpret_cast<uint64_t *>(w + hp.arrivals);
  p.tickets = reinterpret_cast<uint64_t *>(w + hp.tickets);
}

// ------------------------------------------------------------------ timing

struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<std::array<hipEvent_t, 4>> recorded;  // call start, main start, main end, call end
  std::vector<hipEvent_t> pool;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Timing &timing() {
  static Timing t;
  return t;
}

// Event quad of one call while timing is on (all null otherwise).
struct CallEvents {
  std::array<hipEvent_t, 4> ev{};
  bool on = false;
  explicit CallEvents(hipStream_t s) {
    Timing &t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (!t.enabled) return;
    for (auto &e : ev) e = t.get();
    on = std::all_of(ev.begin(), ev.end(), [](hipEvent_t e) { return e != nullptr; });
    if (on) (void)hipEventRecord(ev[0], s);
  }
  void mark(int i, hipStream_t s) {
    if (on) (void)hipEventRecord(ev[i], s);
  }
  void finish(hipStream_t s) {
    if (!on) return;
    (void)hipEventRecord(ev[3], s);
    Timing &t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    t.recorded.push_back(ev);
  }
};

// --------------------------------------------------------------- dispatch

// Workgroups of the first resident round (per_cu per compute unit) take
// their work item from their launch index; the rest of a launch of n draw
// theirs from a counter.  The compute-unit count is read once per device.
int first_round(int64_t n, int per_cu) {
  static std::atomic<int> cus_of[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return int(n);
  int cus = cus_of[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return int(n);
    cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  const int64_t r = int64_t(per_cu) * int64_t(cus);
  if (n <= r || n - r >= (int64_t(1) << fa::kCountBits)) return int(n);
  return int(r);
}

template <class E, int D, int NB>
hipError_t launch_mfma_nb(const DecodeParams &p, bool mods, dim3 grid, dim3 block,
                          hipStream_t s) {
  if (p.nhd) {
    if (mods)
      hipLaunchKernelGGL((fa::decode_mfma_kernel<E, D, true, true, NB>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((fa::decode_mfma_kernel<E, D, true, false, NB>), grid, block, 0, s, p);
  } else {
    if (mods)
      hipLaunchKernelGGL((fa::decode_mfma_kernel<E, D, false, true, NB>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((fa::decode_mfma_kernel<E, D, false, false, NB>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

// Workgroups of the kernel instance for (E, D, NB) that one compute unit
// holds at once (two at D = 128 and 256, three at D = 64), from the runtime's
// occupancy calculator; read once per instance (the same on every device of
// one architecture), 2 if the query fails.
template <class E, int D, int NB>
int resident_per_cu(dim3 block) {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&fa::decode_mfma_kernel<E, D, false, false, NB>),
            int(block.x), 0) != hipSuccess ||
        n <= 0)
      n = 2;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class E, int D>
hipError_t launch_mfma(const DecodeParams &params, const HostPlan &hp, hipStream_t s) {
  dim3 grid(unsigned(hp.units_bound) * unsigned(hp.planes));
  dim3 block(fa::MfmaGeom<E, D>::NW * 64);
  DecodeParams p = params;
  const int per_cu = hp.nb == 2 ? resident_per_cu<E, D, 2>(block) : resident_per_cu<E, D, 1>(block);
  p.ticket_from = first_round(int64_t(hp.units_bound) * hp.planes, per_cu);
  const bool mods = p.window > 0 || p.softcap2 > 0.0f || p.alibi != nullptr || p.mask != nullptr;
  if (hp.nb == 2)
    return launch_mfma_nb<E, D, 2>(p, mods, grid, block, s);
  return launch_mfma_nb<E, D, 1>(p, mods, grid, block, s);
}

template <class E>
hipError_t launch_decode_mfma(const DecodeParams &p, const HostPlan &hp, hipStream_t s) {
  switch (p.head_dim) {
    case 64: return launch_mfma<E, 64>(p, hp, s);
    case 128: return launch_mfma<E, 128>(p, hp, s);
    default: return launch_mfma<E, 256>(p, hp, s);
  }
}

hipError_t dispatch_decode(fa_dtype_t dt, const DecodeParams &p, const HostPlan &hp,
                           hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return launch_decode_mfma<fa::F32>(p, hp, s);
    case FA_DTYPE_F16: return launch_decode_mfma<fa::F16>(p, hp, s);
    default: return launch_decode_mfma<fa::BF16>(p, hp, s);
  }
}

DecodeParams base_params(int batch, int hq, int hkv, int d, int page_size, int pages,
                         int total_used_pages, float scale, const HostPlan &hp) {
  DecodeParams p{};
  p.batch = batch;
  p.num_qo_heads = hq;
  p.num_kv_heads = hkv;
  p.head_dim = d;
  p.page_size = page_size;
  p.num_total_pages = pages;
  p.total_used_pages = total_used_pages;
  p.group = hp.group;
  p.n_gblocks = hp.n_gblocks;
  p.heads_per_unit = hp.gt;
  p.planes = hp.planes;
  p.scale_log2 = scale * fa::kLog2e;
  p.page_div = fa::make_fastdiv(uint32_t(page_size));
  p.uniform_blocks = page_size % 16 == 0;
  p.chunk = hp.chunk;
  p.units_bound = hp.units_bound;
  return p;
}


void apply_variant(DecodeParams &p, const Variant &v) {
  p.nhd = v.nhd;
  p.window = v.window;
  p.alibi = v.alibi;
  p.mask = v.mask;
  p.mask_bytes = v.mask_bytes;
  if (v.softcap > 0.0f) {
    p.softcap2 = v.softcap * fa::kLog2e;  // capping commutes with the base-2 scale
    p.softcap2_inv = 1.0f / p.softcap2;
  }
}

fa_status_t decode_contig(const Variant &var, fa_dtype_t dtype, int num_qo_heads,
                          int num_kv_heads, int head_dim, int max_kv_len, int valid_kv_len,
                          float scale, const void *q, const void *k_cache, const void *v_cache,
                          void *o, float *lse, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const fa_status_t st = contig_checks(dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
                                       valid_kv_len, q, k_cache, v_cache, o, lse, workspace);
  if (st != FA_OK) return st;
  const size_t need = workspace_size(1, num_qo_heads, num_kv_heads, head_dim, max_kv_len, 1);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;

  // Sized like the workspace query (a single page of max_kv_len rows) so the
  // split units fit what the caller allocated.
  const HostPlan hp = make_plan(1, num_qo_heads, num_kv_heads, head_dim, max_kv_len, 1,
                                /*contig=*/true);
  DecodeParams p = base_params(1, num_qo_heads, num_kv_heads, head_dim, max_kv_len, 1, 1,
                               scale, hp);
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o = o;
  p.lse = lse;
  p.contig = 1;
  apply_variant(p, var);
  p.uniform_blocks = 1;
  p.contig_len = valid_kv_len;
  p.contig_start =
      (var.window > 0 && valid_kv_len > var.window) ? valid_kv_len - var.window : 0;
  p.contig_lo = p.contig_start & ~15;
  const int rows = valid_kv_len - p.contig_lo;
  p.contig_units = rows == 0 ? 1 : int((int64_t(rows) + hp.chunk - 1) / hp.chunk);
  carve(p, hp, workspace);

  CallEvents ev(stream);
  ev.mark(1, stream);
  if (dispatch_decode(dtype, p, hp, stream) != hipSuccess) return FA_ERR_LAUNCH;
  ev.mark(2, stream);
  ev.finish(stream);
  return FA_OK;
}

fa_status_t decode_paged(const Variant &var, fa_dtype_t dtype, int batch, int num_qo_heads,
                         int num_kv_heads, int head_dim, int page_size, int num_total_pages,
                         int total_used_pages, float sm_scale, const void *q,
                         const void *k_data, const void *v_data, const int32_t *indices,
                         const int32_t *indptr, const int32_t *last_page_len, void *o,
                         float *lse, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const fa_status_t st = paged_checks(dtype, batch, num_qo_heads, num_kv_heads, head_dim,
                                      page_size, num_total_pages, total_used_pages, q, k_data,
                                      v_data, indices, indptr, last_page_len, o, lse, workspace);
  if (st != FA_OK) return st;
  const HostPlan hp = make_plan(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                total_used_pages, false);
  const size_t need = workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                     total_used_pages);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;

  DecodeParams p = base_params(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                               num_total_pages, total_used_pages, sm_scale, hp);
  p.q = q;
  p.k = k_data;
  p.v = v_data;
  p.o = o;
  p.lse = lse;
  p.indices = indices;
  p.indptr = indptr;
  p.last_page_len = last_page_len;
  apply_variant(p, var);
  carve(p, hp, workspace);

  CallEvents ev(stream);
  ev.mark(1, stream);
  if (dispatch_decode(dtype, p, hp, stream) != hipSuccess) return FA_ERR_LAUNCH;
  ev.mark(2, stream);
  ev.finish(stream);
  return FA_OK;
}

fa_status_t append_paged(int nhd, fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                         int page_size, int num_total_pages, int total_used_pages,
                         const void *k_new, const void *v_new, const int32_t *indices,
                         const int32_t *indptr, const int32_t *last_page_len, void *k_data,
                         void *v_data, hipStream_t stream) {
  const fa_status_t st = append_checks(dtype, batch, num_kv_heads, head_dim, page_size,
                                       num_total_pages, total_used_pages, k_new, v_new,
                                       indices, indptr, last_page_len, k_data, v_data);
  if (st != FA_OK) return st;
  const HostPlan hp = make_plan(batch, num_kv_heads, num_kv_heads, head_dim, page_size,
                                total_used_pages, false);
  DecodeParams p = base_params(batch, num_kv_heads, num_kv_heads, head_dim, page_size,
                               num_total_pages, total_used_pages, 1.0f, hp);
  p.indices = indices;
  p.indptr = indptr;
  p.last_page_len = last_page_len;
  p.nhd = nhd;
  const int elem = dtype == FA_DTYPE_F32 ? 4 : 2;
  hipLaunchKernelGGL(fa::append_kernel, dim3(unsigned(batch) * unsigned(num_kv_heads)),
                     dim3(64), 0, stream, p, static_cast<const char *>(k_new),
                     static_cast<const char *>(v_new), static_cast<char *>(k_data),
                     static_cast<char *>(v_data), elem);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// The gather hook runs the decode kernel's own tile loads (gather_tiles_kernel),
// with the same workgroup size and split units as the decode launch.
template <class E, int D>
hipError_t launch_gather(const DecodeParams &p, const HostPlan &hp, void *out, int64_t out_rows,
                         hipStream_t s) {
  const dim3 grid(unsigned(hp.units_bound) * unsigned(hp.planes));
  const dim3 block(fa::MfmaGeom<E, D>::NW * 64);
  char *dst = static_cast<char *>(out);
  if (p.nhd)
    hipLaunchKernelGGL((fa::gather_tiles_kernel<E, D, true>), grid, block, 0, s, p, dst,
                       out_rows);
  else
    hipLaunchKernelGGL((fa::gather_tiles_kernel<E, D, false>), grid, block, 0, s, p, dst,
                       out_rows);
  return hipGetLastError();
}

template <class E>
hipError_t launch_gather_dim(const DecodeParams &p, const HostPlan &hp, void *out,
                             int64_t out_rows, hipStream_t s) {
  switch (p.head_dim) {
    case 64: return launch_gather<E, 64>(p, hp, out, out_rows, s);
    case 128: return launch_gather<E, 128>(p, hp, out, out_rows, s);
    default: return launch_gather<E, 256>(p, hp, out, out_rows, s);
  }
}

fa_status_t gather_paged(int nhd, fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                         int page_size, int num_total_pages, int total_used_pages,
                         const void *data, const int32_t *indices, const int32_t *indptr,
                         const int32_t *last_page_len, void *out, int64_t out_rows,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const fa_status_t st = gather_checks(dtype, batch, num_kv_heads, head_dim, page_size,
                                       num_total_pages, total_used_pages, data, indices,
                                       indptr, last_page_len, out, out_rows, workspace);
  if (st != FA_OK) return st;
  const size_t need = workspace_size(batch, num_kv_heads, num_kv_heads, head_dim, page_size,
                                     total_used_pages);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  const HostPlan hp = make_plan(batch, num_kv_heads, num_kv_heads, head_dim, page_size,
                                total_used_pages, false);
  DecodeParams p = base_params(batch, num_kv_heads, num_kv_heads, head_dim, page_size,
                               num_total_pages, total_used_pages, 1.0f, hp);
  p.k = data;
  p.v = data;
  p.indices = indices;
  p.indptr = indptr;
  p.last_page_len = last_page_len;
  p.nhd = nhd;
  carve(p, hp, workspace);
  hipError_t e;
  switch (dtype) {
    case FA_DTYPE_F32: e = launch_gather_dim<fa::F32>(p, hp, out, out_rows, stream); break;
    case FA_DTYPE_F16: e = launch_gather_dim<fa::F16>(p, hp, out, out_rows, stream); break;
    default: e = launch_gather_dim<fa::BF16>(p, hp, out, out_rows, stream); break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <class E>
hipError_t launch_merge_states(const float *o_parts, const float *lse_parts, void *o,
                               float *lse, int rows, int n_parts, int d, hipStream_t s) {
  const int64_t threads = int64_t(rows) * (d / 4);
  hipLaunchKernelGGL(fa::merge_states_kernel<E>, dim3(unsigned((threads + 255) / 256)),
                     dim3(256), 0, s, o_parts, lse_parts,
                     static_cast<typename E::raw *>(o), lse, rows, n_parts, d);
  return hipGetLastError();
}

fa_status_t merge_states(fa_dtype_t dtype, int num_rows, int num_parts, int head_dim,
                         const float *o_parts, const float *lse_parts, void *o, float *lse,
                         hipStream_t stream) {
  bool empty = false;
  const fa_status_t st = merge_checks(dtype, num_rows, num_parts, head_dim, o_parts, lse_parts,
                                      o, lse, &empty);
  if (st != FA_OK || empty) return st;
  hipError_t e;
  switch (dtype) {
    case FA_DTYPE_F32:
      e = launch_merge_states<fa::F32>(o_parts, lse_parts, o, lse, num_rows, num_parts,
                                       head_dim, stream);
      break;
    case FA_DTYPE_F16:
      e = launch_merge_states<fa::F16>(o_parts, lse_parts, o, lse, num_rows, num_parts,
                                       head_dim, stream);
      break;
    default:
      e = launch_merge_states<fa::BF16>(o_parts, lse_parts, o, lse, num_rows, num_parts,
                                        head_dim, stream);
      break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

// ------------------------------------------------ allocation-free entry point
//
// The split partials and counters of fa_decode_paged_noalloc live here: one
// copy of this array on every GPU the library runs on, held until the process
// ends.  In host code `scratch` only names the array (a host-side stand-in, not
// a device address): its device address on a GPU comes from
// hipGetSymbolAddress with that GPU current, and only that address is passed
// to kernels.
__device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's copy of `scratch`, looked up on the
// first call on that GPU and kept; nullptr if the lookup fails.
void *scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *addr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (addr) return addr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  addr = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (!addr) {
    void *found = nullptr;
    if (hipGetSymbolAddress(&found, HIP_SYMBOL(scratch)) != hipSuccess || !found)
      return nullptr;
    g_scratch_addr[dev].store(found, std::memory_order_release);
    addr = found;
  }
  return addr;
}

}  // namespace

extern "C" {

size_t fa_decode_workspace_size(int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                                int page_size, int total_used_pages) {
  return workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                        total_used_pages);
}

fa_status_t fa_append_paged(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                            int page_size, int num_total_pages, int total_used_pages,
                            const void *k_new, const void *v_new, const int32_t *indices,
                            const int32_t *indptr, const int32_t *last_page_len, void *k_data,
                            void *v_data, hipStream_t stream) {
  return append_paged(0, dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                      total_used_pages, k_new, v_new, indices, indptr, last_page_len, k_data,
                      v_data, stream);
}

fa_status_t fa_append_paged_nhd(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                                int page_size, int num_total_pages, int total_used_pages,
                                const void *k_new, const void *v_new, const int32_t *indices,
                                const int32_t *indptr, const int32_t *last_page_len,
                                void *k_data, void *v_data, hipStream_t stream) {
  return append_paged(1, dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                      total_used_pages, k_new, v_new, indices, indptr, last_page_len, k_data,
                      v_data, stream);
}

fa_status_t fa_decode_contig(fa_dtype_t dtype, int num_qo_heads, int num_kv_heads,
                             int head_dim, int max_kv_len, int valid_kv_len, float scale,
                             const void *q, const void *k_cache, const void *v_cache, void *o,
                             float *lse, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return decode_contig(Variant{}, dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                       scale, q, k_cache, v_cache, o, lse, workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_contig_nhd(fa_dtype_t dtype, int num_qo_heads, int num_kv_heads,
                                 int head_dim, int max_kv_len, int valid_kv_len, float scale,
                                 const void *q, const void *k_cache, const void *v_cache,
                                 void *o, float *lse, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return decode_contig(Variant{1, 0, 0.0f, nullptr}, dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                       scale, q, k_cache, v_cache, o, lse, workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_paged(fa_dtype_t dtype, int batch, int num_qo_heads, int num_kv_heads,
                            int head_dim, int page_size, int num_total_pages,
                            int total_used_pages, float sm_scale, const void *q,
                            const void *k_data, const void *v_data, const int32_t *indices,
                            const int32_t *indptr, const int32_t *last_page_len, void *o,
                            float *lse, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return decode_paged(Variant{}, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                      num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
                      indptr, last_page_len, o, lse, workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_paged_nhd(fa_dtype_t dtype, int batch, int num_qo_heads,
                                int num_kv_heads, int head_dim, int page_size,
                                int num_total_pages, int total_used_pages, float sm_scale,
                                const void *q, const void *k_data, const void *v_data,
                                const int32_t *indices, const int32_t *indptr,
                                const int32_t *last_page_len, void *o, float *lse,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_paged(Variant{1, 0, 0.0f, nullptr}, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                      num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
                      indptr, last_page_len, o, lse, workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_paged_noalloc(fa_dtype_t dtype, int batch, int num_qo_heads,
                                    int num_kv_heads, int head_dim, int page_size,
                                    int num_total_pages, int total_used_pages, float sm_scale,
                                    const void *q, const void *k_data, const void *v_data,
                                    const int32_t *indices, const int32_t *indptr,
                                    const int32_t *last_page_len, void *o, float *lse,
                                    hipStream_t stream) {
  const fa_status_t st = paged_checks(dtype, batch, num_qo_heads, num_kv_heads, head_dim,
                                      page_size, num_total_pages, total_used_pages, q, k_data,
                                      v_data, indices, indptr, last_page_len, o, lse, nullptr);
  if (st != FA_OK) return st;
  const size_t need = workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                     total_used_pages);
  if (need > size_t(FA_NOALLOC_SCRATCH_BYTES)) return FA_ERR_WORKSPACE_TOO_SMALL;
  void *ws = scratch_address();
  if (!ws) return FA_ERR_LAUNCH;
  return decode_paged(Variant{}, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                      num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
                      indptr, last_page_len, o, lse, ws, size_t(FA_NOALLOC_SCRATCH_BYTES),
                      stream);
}

fa_status_t fa_decode_contig_opts(const fa_decode_options_t *opts, fa_dtype_t dtype,
                                  int num_qo_heads, int num_kv_heads, int head_dim,
                                  int max_kv_len, int valid_kv_len, float scale, const void *q,
                                  const void *k_cache, const void *v_cache, void *o, float *lse,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Variant var;
  const fa_status_t st = read_options(opts, var);
  if (st != FA_OK) return st;
  return decode_contig(var, dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
                       valid_kv_len, scale, q, k_cache, v_cache, o, lse, workspace,
                       workspace_bytes, stream);
}

fa_status_t fa_decode_paged_opts(const fa_decode_options_t *opts, fa_dtype_t dtype, int batch,
                                 int num_qo_heads, int num_kv_heads, int head_dim, int page_size,
                                 int num_total_pages, int total_used_pages, float sm_scale,
                                 const void *q, const void *k_data, const void *v_data,
                                 const int32_t *indices, const int32_t *indptr,
                                 const int32_t *last_page_len, void *o, float *lse,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Variant var;
  const fa_status_t st = read_options(opts, var);
  if (st != FA_OK) return st;
  return decode_paged(var, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                      num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
                      indptr, last_page_len, o, lse, workspace, workspace_bytes, stream);
}

fa_status_t fa_merge_states(fa_dtype_t dtype, int num_rows, int num_parts, int head_dim,
                            const float *o_parts, const float *lse_parts, void *o, float *lse,
                            hipStream_t stream) {
  return merge_states(dtype, num_rows, num_parts, head_dim, o_parts, lse_parts, o, lse, stream);
}

const char *fa_status_string(fa_status_t status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_PROBLEM: return "FA_ERR_INVALID_PROBLEM";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH";
  }
  return "FA_ERR_UNKNOWN";
}

// ------------------------------------------------------------------- hooks

fa_status_t fa_debug_gather_paged(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                                  int page_size, int num_total_pages, int total_used_pages,
                                  const void *data, const int32_t *indices,
                                  const int32_t *indptr, const int32_t *last_page_len,
                                  void *out, int64_t out_rows, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return gather_paged(0, dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                      total_used_pages, data, indices, indptr, last_page_len, out, out_rows,
                      workspace, workspace_bytes, stream);
}

fa_status_t fa_debug_gather_paged_nhd(fa_dtype_t dtype, int batch, int num_kv_heads,
                                      int head_dim, int page_size, int num_total_pages,
                                      int total_used_pages, const void *data,
                                      const int32_t *indices, const int32_t *indptr,
                                      const int32_t *last_page_len, void *out, int64_t out_rows,
                                      void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  return gather_paged(1, dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                      total_used_pages, data, indices, indptr, last_page_len, out, out_rows,
                      workspace, workspace_bytes, stream);
}

fa_status_t fa_debug_schedule(fa_dtype_t dtype, int batch, int num_qo_heads, int num_kv_heads,
                              int head_dim, int page_size, int total_used_pages,
                              const int32_t *indptr, const int32_t *last_page_len,
                              int32_t *out, int64_t out_entries, hipStream_t stream) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!extents_ok(batch, num_qo_heads, num_kv_heads, page_size)) return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (total_used_pages < 0) return FA_ERR_INVALID_PROBLEM;
  if (!indptr || !last_page_len || !out) return FA_ERR_INVALID_PROBLEM;
  if (!all_aligned({}, {indptr, last_page_len, out})) return FA_ERR_INVALID_PROBLEM;
  if (!grid_ok(num_qo_heads, num_kv_heads) || !rows_ok(total_used_pages, page_size))
    return FA_ERR_UNSUPPORTED;
  const HostPlan hp = make_plan(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                total_used_pages, false);
  if (!launch_ok(hp)) return FA_ERR_UNSUPPORTED;
  if (out_entries < 8 * int64_t(hp.units_bound)) return FA_ERR_WORKSPACE_TOO_SMALL;
  DecodeParams p = base_params(batch, num_qo_heads, num_kv_heads, head_dim, page_size, 1,
                               total_used_pages, 1.0f, hp);
  p.indptr = indptr;
  p.last_page_len = last_page_len;
  hipLaunchKernelGGL(fa::schedule_kernel, dim3(hp.units_bound), dim3(256), 0, stream, p, out);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status_t fa_debug_counters_in_use(int batch, int num_qo_heads, int num_kv_heads,
                                     int head_dim, int page_size, int total_used_pages,
                                     const void *workspace, size_t workspace_bytes,
                                     int32_t *out, hipStream_t stream) {
  if (!extents_ok(batch, num_qo_heads, num_kv_heads, page_size) || total_used_pages < 0)
    return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (!out || !all_aligned({workspace}, {out})) return FA_ERR_INVALID_PROBLEM;
  if (!grid_ok(num_qo_heads, num_kv_heads) || !rows_ok(total_used_pages, page_size))
    return FA_ERR_UNSUPPORTED;
  const HostPlan hp = make_plan(batch, num_qo_heads, num_kv_heads, head_dim,
                                page_size, total_used_pages, false);
  if (!launch_ok(hp)) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < hp.total) return FA_ERR_WORKSPACE_TOO_SMALL;
  const char *w = static_cast<const char *>(workspace);
  hipLaunchKernelGGL(fa::counter_check_kernel, dim3(1), dim3(256), 0, stream,
                     reinterpret_cast<const uint64_t *>(w + hp.arrivals),
                     int64_t(batch) * num_qo_heads,
                     reinterpret_cast<const uint64_t *>(w + hp.tickets), out);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status_t fa_debug_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                                hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % fa::kProbeBlock != 0 || !all_aligned({buf}, {sink}))
    return FA_ERR_INVALID_PROBLEM;
  const int64_t n_blocks = int64_t(bytes / fa::kProbeBlock);
  hipLaunchKernelGGL(fa::read_probe_kernel, dim3(8192), dim3(256), 0, stream,
                     static_cast<const char *>(buf), n_blocks, sink);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status_t fa_debug_timing_enable(int enable) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.enabled = enable != 0;
  return FA_OK;
}

fa_status_t fa_debug_timing_read(double *main_kernel_ms, double *whole_call_ms, int *calls) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  double main_ms = 0.0, call_ms = 0.0;
  bool ok = true;
  for (auto &ev : t.recorded) {
    float a = 0.0f, b = 0.0f;
    if (hipEventSynchronize(ev[3]) != hipSuccess ||
        hipEventElapsedTime(&a, ev[1], ev[2]) != hipSuccess ||
        hipEventElapsedTime(&b, ev[0], ev[3]) != hipSuccess)
      ok = false;
    main_ms += a;
    call_ms += b;
    for (hipEvent_t e : ev) t.pool.push_back(e);
  }
  const int n = int(t.recorded.size());
  t.recorded.clear();
  if (main_kernel_ms) *main_kernel_ms = main_ms;
  if (whole_call_ms) *whole_call_ms = call_ms;
  if (calls) *calls = n;
  return ok ? FA_OK : FA_ERR_LAUNCH;
}

fa_status_t fa_debug_plan(fa_dtype_t dtype, int batch, int num_qo_heads, int num_kv_heads,
                          int head_dim, int page_size, int total_used_pages, int *chunk_rows,
                          int *units_bound, int *heads_per_unit_out, int *kernel_kind) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!extents_ok(batch, num_qo_heads, num_kv_heads, page_size) || total_used_pages < 0)
    return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  const HostPlan hp = make_plan(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                total_used_pages, false);
  if (chunk_rows) *chunk_rows = hp.chunk;
  if (units_bound) *units_bound = hp.units_bound;
  if (heads_per_unit_out) *heads_per_unit_out = std::min(hp.group, hp.gt * hp.nb);
  if (kernel_kind) *kernel_kind = hp.kind;
  return FA_OK;
}

}  // extern "C"
