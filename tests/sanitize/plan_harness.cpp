// Host-side checks and launch plan of the decode library (fa_plan.hpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: every entry
// point's argument checks over random, extreme and edge-case arguments
// (signed overflow in a size product, say, aborts the run), and the plan's
// invariants for every valid problem drawn:
//   - the split size is a positive multiple of 128 rows, and a unit of a
//     paged call whose page size is a multiple of 16 spans at most
//     kPageTable page slots;
//   - the unit bound covers any split of the rows the page table allows
//     (requests of random lengths summing to at most total_used_pages pages);
//   - the workspace regions are 256-byte aligned, in order, do not overlap
//     and end at the reported total, which fa_decode_workspace_size returns.
// Prints "plan harness OK" and exits 0, or reports the first broken case.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../decode_attention_query_amd/csrc/fa_plan.hpp"

using namespace fa_plan;

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

uint64_t next_u64() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}

int pick(std::initializer_list<int> v) {
  const int i = int(next_u64() % v.size());
  return *(v.begin() + i);
}

int rand_int(int lo, int hi) {  // inclusive
  return lo + int(next_u64() % uint64_t(int64_t(hi) - lo + 1));
}

// placeholder pointers: never dereferenced by the checks
const void *ptr_kind(int k) {
  switch (k) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<const void *>(uintptr_t(0x1002));  // 2-byte aligned
    case 2: return reinterpret_cast<const void *>(uintptr_t(0x1008));  // 8-byte aligned
    default: return reinterpret_cast<const void *>(uintptr_t(0x10000));
  }
}

const void *mostly_good() { return ptr_kind(next_u64() % 8 == 0 ? int(next_u64() % 3) : 3); }

int g_failures = 0;

void fail(const char *what, int a, int b, int c, int d, int e, int f) {
  if (g_failures++ < 10)
    std::fprintf(stderr, "FAIL %s: %d %d %d %d %d %d\n", what, a, b, c, d, e, f);
}

bool status_known(fa_status_t st) {
  return st == FA_OK || st == FA_ERR_INVALID_PROBLEM || st == FA_ERR_UNSUPPORTED ||
         st == FA_ERR_WORKSPACE_TOO_SMALL || st == FA_ERR_LAUNCH;
}

int extreme() {
  return pick({-(1 << 30), -1, 0, 1, 2, 3, 7, 16, 17, 64, 1000, 65535, 65536, 1 << 20,
               (1 << 30), 0x7fffffff});
}

void check_plan(int batch, int hq, int hkv, int d, int page, int used) {
  const HostPlan hp = make_plan(batch, hq, hkv, d, page, used, false);
  if (hp.chunk <= 0 || hp.chunk % 128 != 0) fail("chunk", batch, hq, hkv, d, page, used);
  if (page % 16 == 0 && int64_t(hp.chunk) / page + 2 > fa::kPageTable)
    fail("page slots per unit", batch, hq, hkv, d, page, used);
  // random request lengths within the table's rows
  const int64_t total_rows = int64_t(used) * page;
  int64_t units = 0, rows_left = total_rows;
  for (int b = 0; b < batch && b < 4096; ++b) {
    int64_t L = 0;
    if (rows_left > 0 && next_u64() % 4 != 0) L = int64_t(next_u64() % uint64_t(rows_left + 1));
    if (b == batch - 1 || b == 4095) L = rows_left;  // the last takes the rest
    rows_left -= L;
    units += L == 0 ? 1 : (L + hp.chunk - 1) / hp.chunk;
  }
  if (batch > 4096) units += batch - 4096;  // the other requests: empty, one unit each
  if (units > hp.units_bound) fail("units bound", batch, hq, hkv, d, page, used);
  const size_t need = size_t(hp.units_bound) * hq;
  bool ok = hp.part_lse == 0 && hp.part_o >= hp.part_lse + sizeof(float) * need &&
            hp.arrivals >= hp.part_o + sizeof(float) * need * size_t(d) &&
            hp.tickets >= hp.arrivals + sizeof(uint64_t) * fa::kArrivalStride * size_t(batch) * hq &&
            hp.total >= hp.tickets + sizeof(uint64_t) * fa::kArrivalStride;
  for (size_t off : {hp.part_lse, hp.part_o, hp.arrivals, hp.tickets, hp.total})
    ok = ok && off % kAlign == 0;
  if (!ok) fail("workspace layout", batch, hq, hkv, d, page, used);
  if (workspace_size(batch, hq, hkv, d, page, used) != hp.total)
    fail("workspace size", batch, hq, hkv, d, page, used);
}

}  // namespace

int main() {
  int valid = 0;
  for (int trial = 0; trial < 1000000; ++trial) {
    int batch, hq, hkv, d, page, pages, used;
    if (trial % 3 == 0) {  // extremes
      batch = extreme(); hkv = extreme(); hq = extreme(); d = pick({-1, 0, 64, 96, 128, 256, 512});
      page = extreme(); pages = extreme(); used = extreme();
    } else {  // plausible problems
      batch = rand_int(1, 4096);
      hkv = pick({1, 2, 3, 4, 8, 16});
      hq = hkv * pick({1, 2, 3, 4, 7, 8, 16, 24, 32, 48, 64});
      d = pick({64, 128, 256});
      page = pick({1, 3, 5, 16, 32, 48, 64, 256, 1024});
      used = rand_int(0, 1 << 16);
      pages = used + rand_int(1, 1000);
    }
    const fa_dtype_t dt = fa_dtype_t(pick({0, 1, 2, 3, -1}));
    const void *q = mostly_good(), *k = mostly_good(), *v = mostly_good(), *o = mostly_good();
    const auto *ind = static_cast<const int32_t *>(mostly_good());
    const auto *ptr = static_cast<const int32_t *>(mostly_good());
    const auto *lpl = static_cast<const int32_t *>(mostly_good());
    const auto *lse = static_cast<const float *>(mostly_good());
    const void *ws = mostly_good();
    const fa_status_t sp = paged_checks(dt, batch, hq, hkv, d, page, pages, used, q, k, v, ind,
                                        ptr, lpl, o, lse, ws);
    const int valid_len = int(std::max<int64_t>(
        -2, std::min<int64_t>(int64_t(page) + rand_int(-3, 2), 0x7fffffff)));
    const fa_status_t sc = contig_checks(dt, hq, hkv, d, page, valid_len, q, k, v, o, lse, ws);
    const fa_status_t sa = append_checks(dt, batch, hkv, d, page, pages, used, q, k, ind, ptr,
                                         lpl, o, v);
    const fa_status_t sg = gather_checks(dt, batch, hkv, d, page, pages, used, k, ind, ptr, lpl,
                                         o, int64_t(extreme()), ws);
    bool empty = false;
    const fa_status_t sm = merge_checks(dt, extreme(), extreme(), d, static_cast<const float *>(q),
                                        lse, o, lse, &empty);
    for (fa_status_t st : {sp, sc, sa, sg, sm})
      if (!status_known(st)) fail("unknown status", batch, hq, hkv, d, page, used);
    const size_t wsz = workspace_size(batch, hq, hkv, d, page, used);
    if (sp == FA_OK) {
      ++valid;
      if (wsz == 0) fail("valid problem without workspace", batch, hq, hkv, d, page, used);
      check_plan(batch, hq, hkv, d, page, used);
    }
    if (sc == FA_OK) {
      const HostPlan hc = make_plan(1, hq, hkv, d, page, 1, true);
      if (hc.units_bound < 1 || int64_t(hc.units_bound) * hc.chunk < page)
        fail("contig units", 1, hq, hkv, d, page, 1);
    }
    fa_decode_options_t opts{pick({-1, 0, 1, 2}), extreme(),
                             float(pick({-1, 0, 30})) * (next_u64() % 7 == 0 ? 1e38f : 1.0f),
                             static_cast<const float *>(mostly_good()),
                             static_cast<const uint8_t *>(mostly_good()),
                             size_t(next_u64() % 3) << (next_u64() % 40)};
    Variant var;
    if (!status_known(read_options(&opts, var))) fail("options", 0, 0, 0, 0, 0, 0);
  }
  if (valid < 50000) {
    std::fprintf(stderr, "too few valid problems drawn: %d\n", valid);
    return 1;
  }
  if (g_failures) {
    std::fprintf(stderr, "%d failures\n", g_failures);
    return 1;
  }
  std::printf("plan harness OK (%d valid problems)\n", valid);
  return 0;
}
