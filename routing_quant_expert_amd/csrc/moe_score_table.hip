// The glibc score mode: the host's own libm defines the scores
// [device_route.rs, module doc: the selection bit for bit with glibc-exact
// softplus; moe_v41.rs, fn softplus, fn route_from_logits: f32 exp, ln_1p and
// sqrt of the host]. The device keeps its correctly rounded chain (score_of)
// and replaces its result by glibc's on the inputs where the two differ; this
// file finds those inputs by sweeping every f32 z <= 20 once per process and
// keeps the per-device registration of the table the caller uploads.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "moe_host.h"
#include "moe_internal.h"

namespace moe {
namespace {

// The chain as the host computes it: f32 expf, log1pf and sqrtf of the C
// library, with the cut at 20 of the correctly rounded chain.
float glibc_score(float z) { return z > 20.0f ? sqrtf(z) : sqrtf(log1pf(expf(z))); }

struct HostTable {
  std::vector<uint32_t> keys, vals, index;
};

HostTable* g_host = nullptr;
std::once_flag g_host_once;

int sweep_threads() {
  unsigned n = std::thread::hardware_concurrency();
  if (const char* e = std::getenv("OMP_NUM_THREADS")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v > 0 && (unsigned long)v < n) n = (unsigned)v;
  }
  return n < 1 ? 1 : (n > 64 ? 64 : (int)n);
}

// Every non-NaN input z <= 20, in chunks of 2^20 bit patterns taken in turn
// by the threads; each chunk's exceptions are kept apart and joined in chunk
// order, which is ascending bit order.
void build_host_table() {
  constexpr int kChunkBits = 20;
  constexpr int kChunks = 1 << (32 - kChunkBits);
  std::vector<std::vector<uint32_t>> ck(kChunks), cv(kChunks);
  std::atomic<int> next{0};
  auto work = [&]() {
    for (int c; (c = next.fetch_add(1)) < kChunks;) {
      const uint64_t lo = (uint64_t)c << kChunkBits, hi = lo + ((uint64_t)1 << kChunkBits);
      for (uint64_t b = lo; b < hi; ++b) {
        const float z = __builtin_bit_cast(float, (uint32_t)b);
        if (!(z <= 20.0f)) continue;
        const float g = glibc_score(z), s = score_of(z, 1.0f);
        const uint32_t gb = __builtin_bit_cast(uint32_t, g);
        if (gb != __builtin_bit_cast(uint32_t, s)) {
          ck[c].push_back((uint32_t)b);
          cv[c].push_back(gb);
        }
      }
    }
  };
  const int nt = sweep_threads();
  std::vector<std::thread> pool;
  for (int t = 1; t < nt; ++t) pool.emplace_back(work);
  work();
  for (auto& t : pool) t.join();

  HostTable* h = new HostTable;
  size_t total = 0;
  for (int c = 0; c < kChunks; ++c) total += ck[c].size();
  h->keys.reserve(total);
  h->vals.reserve(total);
  for (int c = 0; c < kChunks; ++c) {
    h->keys.insert(h->keys.end(), ck[c].begin(), ck[c].end());
    h->vals.insert(h->vals.end(), cv[c].begin(), cv[c].end());
    std::vector<uint32_t>().swap(ck[c]);
    std::vector<uint32_t>().swap(cv[c]);
  }
  h->index.assign(MOE_SCORE_INDEX_LEN, 0);
  size_t i = 0;
  for (uint32_t p = 0; p < (1u << 24); ++p) {
    while (i < total && (h->keys[i] >> kScorePrefixShift) < p) ++i;
    h->index[p] = (uint32_t)i;
  }
  h->index[1u << 24] = (uint32_t)total;
  g_host = h;
}

constexpr int kMaxDevices = 64;
std::mutex g_reg_mu;
ScoreTable g_reg[kMaxDevices] = {};

}  // namespace

ScoreTable score_table_for(const moe_cfg& c) {
  if (c.score_mode != MOE_SCORE_GLIBC) return ScoreTable{nullptr, nullptr, nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ScoreTable{nullptr, nullptr, nullptr};
  std::lock_guard<std::mutex> lk(g_reg_mu);
  return g_reg[dev];
}

ScoreTable host_score_table() {
  std::call_once(g_host_once, build_host_table);
  return ScoreTable{g_host->keys.data(), g_host->vals.data(), g_host->index.data()};
}

int check_score_mode(const moe_cfg& c) {
  if (c.score_mode == MOE_SCORE_CR) return MOE_OK;
  if (!score_table_for(c).keys)
    return fail(MOE_EINVAL, "score_mode MOE_SCORE_GLIBC needs moe_set_score_table on the current device first%s%lld");
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

static int moe_glibc_score_table_body(uint32_t* keys, uint32_t* vals, uint32_t* index, int64_t cap, int64_t* n) {
  if (!n) return fail(MOE_EINVAL, "n is NULL%s%lld");
  std::call_once(g_host_once, build_host_table);
  const int64_t total = (int64_t)g_host->keys.size();
  *n = total;
  if (!keys) return MOE_OK;
  if (!vals || !index || cap < total)
    return fail(MOE_EINVAL, "score table: keys, vals of cap >= %s%lld entries and index are needed", "",
                (long long)total);
  std::memcpy(keys, g_host->keys.data(), sizeof(uint32_t) * total);
  std::memcpy(vals, g_host->vals.data(), sizeof(uint32_t) * total);
  std::memcpy(index, g_host->index.data(), sizeof(uint32_t) * MOE_SCORE_INDEX_LEN);
  return MOE_OK;
}

int moe_set_score_table(const uint32_t* keys, const uint32_t* vals, const uint32_t* index, int64_t n) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "set_score_table");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device index %s%lld beyond the table registry", "", dev);
  if (keys && (!vals || !index || n < 0))
    return fail(MOE_EINVAL, "score table: keys, vals and index must all be given%s%lld");
  std::lock_guard<std::mutex> lk(g_reg_mu);
  g_reg[dev] = keys ? ScoreTable{keys, vals, index} : ScoreTable{nullptr, nullptr, nullptr};
  return MOE_OK;
}

int moe_glibc_score_table(uint32_t* keys, uint32_t* vals, uint32_t* index, int64_t cap, int64_t* n) {
  return guarded([&] { return moe_glibc_score_table_body(keys, vals, index, cap, n); });
}

}  // extern "C"
