// Delta residency manager: decides which variants' compressed deltas stay in device memory, and
// ties a load's completion to the HIP event the upload recorded.  It follows the BitDelta post,
// "Infrastructure details": the variants with the most requests stay pinned (the top few by
// volume are always resident), the others share the rest of the space with least-recently-used
// eviction; a request for a variant that is not resident starts a load (cold start); requests for
// a variant whose load is in flight wait for it instead of starting another (request routing).
//
// Request rate is the number of requests seen so far; the pinned set is the num_pinned variants
// with the highest counts (ties to the smaller id) among those requested at least once, counting
// the current request.  Loading variants are neither evicted nor loaded twice; pinned variants
// and variants held by requests in flight are never evicted; eviction takes the least recently
// requested evictable variant first (ties to the smaller id) until the new delta fits; a request
// that cannot be made to fit changes nothing but the request counts and is answered NO_ROOM.
// A request may hold its variant (the answer HIT, LOAD or QUEUED then counts one more holder);
// the caller releases it when the work that reads the variant's memory has drained.  The caller
// moves the bytes (bitdelta_upload_variant on its stream, say); it reports the end of a load
// with load_done, or attaches the event recorded after the upload and lets poll find it done.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include "../../include/bitdelta.h"

namespace bd {
bitdelta_status status_of_hip(hipError_t e);  // records e for bitdelta_last_hip_error
}

struct bitdelta_residency {
  std::vector<int64_t> size;
  std::vector<int64_t> count;
  std::vector<uint64_t> last;    // time of the latest request, 0 = never
  std::vector<uint8_t> state;    // BITDELTA_VARIANT_*
  std::vector<int64_t> holds;    // requests holding the variant (not yet released)
  std::vector<hipEvent_t> done;  // event of a loading variant's upload, or null
  int64_t cap = 0;
  int64_t used = 0;
  int32_t num_pinned = 0;
  uint64_t clock = 0;
  std::mutex mu;
};

namespace {

constexpr int32_t kMaxResidencyVariants = 4096;

std::vector<uint8_t> pinned_set(const bitdelta_residency& r) {
  const int n = (int)r.size.size();
  std::vector<int32_t> ids(n);
  std::iota(ids.begin(), ids.end(), 0);
  const int k = std::min<int>(r.num_pinned, n);
  std::partial_sort(ids.begin(), ids.begin() + k, ids.end(), [&](int32_t a, int32_t b) {
    return r.count[a] != r.count[b] ? r.count[a] > r.count[b] : a < b;
  });
  std::vector<uint8_t> pin(n, 0);
  for (int i = 0; i < k; ++i)
    if (r.count[ids[i]] > 0) pin[ids[i]] = 1;
  return pin;
}

}  // namespace

extern "C" {

bitdelta_status bitdelta_residency_create(int32_t num_variants, const int64_t* variant_bytes,
                                          int64_t capacity_bytes, int32_t num_pinned,
                                          bitdelta_residency** out) {
  if (!out) return BITDELTA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_variants <= 0 || num_variants > kMaxResidencyVariants || !variant_bytes ||
      capacity_bytes <= 0 || num_pinned < 0)
    return BITDELTA_ERR_INVALID_ARG;
  for (int32_t v = 0; v < num_variants; ++v)
    if (variant_bytes[v] <= 0) return BITDELTA_ERR_INVALID_ARG;
  bitdelta_residency* r = new (std::nothrow) bitdelta_residency;
  if (!r) return BITDELTA_ERR_UNSUPPORTED;
  r->size.assign(variant_bytes, variant_bytes + num_variants);
  r->count.assign(num_variants, 0);
  r->last.assign(num_variants, 0);
  r->state.assign(num_variants, BITDELTA_VARIANT_ABSENT);
  r->holds.assign(num_variants, 0);
  r->done.assign(num_variants, nullptr);
  r->cap = capacity_bytes;
  r->num_pinned = num_pinned;
  *out = r;
  return BITDELTA_OK;
}

void bitdelta_residency_destroy(bitdelta_residency* r) { delete r; }

bitdelta_status bitdelta_residency_request(bitdelta_residency* r, int32_t variant, int32_t hold,
                                           int32_t* action, int32_t* evicted,
                                           int32_t* num_evicted) {
  if (!r || !action || !evicted || !num_evicted || (hold != 0 && hold != 1))
    return BITDELTA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(r->mu);
  const int n = (int)r->size.size();
  if (variant < 0 || variant >= n) return BITDELTA_ERR_INVALID_ARG;
  *num_evicted = 0;
  r->count[variant] += 1;
  r->last[variant] = ++r->clock;
  if (r->state[variant] == BITDELTA_VARIANT_RESIDENT) {
    *action = BITDELTA_RESIDENCY_HIT;
    r->holds[variant] += hold;
    return BITDELTA_OK;
  }
  if (r->state[variant] == BITDELTA_VARIANT_LOADING) {
    *action = BITDELTA_RESIDENCY_QUEUED;
    r->holds[variant] += hold;
    return BITDELTA_OK;
  }
  const std::vector<uint8_t> pin = pinned_set(*r);
  std::vector<int32_t> cand;
  int64_t freeable = 0;
  for (int u = 0; u < n; ++u)
    if (u != variant && r->state[u] == BITDELTA_VARIANT_RESIDENT && !pin[u] && r->holds[u] == 0) {
      cand.push_back(u);
      freeable += r->size[u];
    }
  int64_t need = r->used + r->size[variant] - r->cap;
  if (need > freeable) {
    *action = BITDELTA_RESIDENCY_NO_ROOM;
    return BITDELTA_OK;
  }
  std::sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) {
    return r->last[a] != r->last[b] ? r->last[a] < r->last[b] : a < b;
  });
  int32_t ne = 0;
  for (int32_t u : cand) {
    if (need <= 0) break;
    r->state[u] = BITDELTA_VARIANT_ABSENT;
    r->used -= r->size[u];
    need -= r->size[u];
    evicted[ne++] = u;
  }
  r->state[variant] = BITDELTA_VARIANT_LOADING;
  r->done[variant] = nullptr;
  r->used += r->size[variant];
  r->holds[variant] += hold;
  *num_evicted = ne;
  *action = BITDELTA_RESIDENCY_LOAD;
  return BITDELTA_OK;
}

bitdelta_status bitdelta_residency_release(bitdelta_residency* r, int32_t variant) {
  if (!r) return BITDELTA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(r->mu);
  if (variant < 0 || variant >= (int)r->size.size() || r->holds[variant] == 0)
    return BITDELTA_ERR_INVALID_ARG;
  r->holds[variant] -= 1;
  return BITDELTA_OK;
}

int64_t bitdelta_residency_holds(bitdelta_residency* r, int32_t variant) {
  if (!r) return -1;
  std::lock_guard<std::mutex> lock(r->mu);
  if (variant < 0 || variant >= (int)r->size.size()) return -1;
  return r->holds[variant];
}

bitdelta_status bitdelta_residency_load_done(bitdelta_residency* r, int32_t variant) {
  if (!r) return BITDELTA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(r->mu);
  if (variant < 0 || variant >= (int)r->size.size() ||
      r->state[variant] != BITDELTA_VARIANT_LOADING)
    return BITDELTA_ERR_INVALID_ARG;
  r->state[variant] = BITDELTA_VARIANT_RESIDENT;
  r->done[variant] = nullptr;
  return BITDELTA_OK;
}

bitdelta_status bitdelta_residency_load_enqueued(bitdelta_residency* r, int32_t variant,
                                                 bitdelta_event event) {
  if (!r || !event) return BITDELTA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(r->mu);
  if (variant < 0 || variant >= (int)r->size.size() ||
      r->state[variant] != BITDELTA_VARIANT_LOADING)
    return BITDELTA_ERR_INVALID_ARG;
  r->done[variant] = static_cast<hipEvent_t>(event);
  return BITDELTA_OK;
}

bitdelta_status bitdelta_residency_poll(bitdelta_residency* r, int32_t* completed,
                                        int32_t* num_completed) {
  if (!r || !completed || !num_completed) return BITDELTA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(r->mu);
  int32_t nc = 0;
  for (int v = 0; v < (int)r->size.size(); ++v) {
    if (r->state[v] != BITDELTA_VARIANT_LOADING || !r->done[v]) continue;
    const hipError_t e = hipEventQuery(r->done[v]);
    if (e == hipErrorNotReady) continue;
    if (e != hipSuccess) {
      *num_completed = nc;
      return bd::status_of_hip(e);
    }
    r->state[v] = BITDELTA_VARIANT_RESIDENT;
    r->done[v] = nullptr;
    completed[nc++] = v;
  }
  *num_completed = nc;
  return BITDELTA_OK;
}

int32_t bitdelta_residency_state(bitdelta_residency* r, int32_t variant) {
  if (!r) return -1;
  std::lock_guard<std::mutex> lock(r->mu);
  if (variant < 0 || variant >= (int)r->size.size()) return -1;
  return r->state[variant];
}

int64_t bitdelta_residency_used_bytes(bitdelta_residency* r) {
  if (!r) return -1;
  std::lock_guard<std::mutex> lock(r->mu);
  return r->used;
}

}  // extern "C"
