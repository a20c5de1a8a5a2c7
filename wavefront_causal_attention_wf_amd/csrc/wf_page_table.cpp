// Host page table for one request's attention pages.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", full text:
// Appendix B.3 (the live store page becomes retained history after the round;
// the first clean chunk may be kept as a persistent anchor) and Appendix B.8 /
// Eq. (13) (fixed-capacity K/V arrays, history bounded independently of video
// length). The pages give no allocation policy; this one is FIFO so that page
// tables are a unique function of the call sequence:
//   alloc  : pop ceil(T/P) ids from the front of the free list;
//   commit : append the live chunk to history; if history exceeds the window,
//            remove the oldest chunk (the oldest after the anchor when pinned)
//            and append its ids, in page order, to the back of the free list.
//
// Pure host C++ (no HIP), so it also builds with g++ for sanitizer runs.
#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "wf_attn.h"
#include "wf_error.h"

struct wf_page_table {
  int32_t num_pages = 0;
  int32_t page_size = 0;
  int32_t chunk_tokens = 0;
  int32_t window = 0;
  bool pin_anchor = false;
  int32_t ppc = 0;
  // Free list as a ring buffer of capacity num_pages: ids at [head, head+count).
  std::vector<int32_t> ring;
  int32_t head = 0;
  int32_t count = 0;
  std::vector<std::vector<int32_t>> history;  // oldest first
  std::vector<int32_t> live;                  // allocated store chunk, empty if none
  bool has_live = false;

  int32_t pop_front() {
    int32_t id = ring[head];
    head = (head + 1) % num_pages;
    --count;
    return id;
  }
  void push_back(int32_t id) {
    ring[(head + count) % num_pages] = id;
    ++count;
  }
};

namespace {
constexpr int64_t kMaxPages = int64_t(1) << 30;
}

extern "C" wf_status wf_page_table_create(int32_t num_pages, int32_t page_size,
                                          int32_t chunk_tokens, int32_t window_chunks,
                                          int32_t pin_anchor, const int32_t* initial_free_order,
                                          wf_page_table** out) {
  try {
    if (!out) return wf::fail(WF_EINVAL, "wf_page_table_create: out is NULL");
    if (num_pages <= 0 || num_pages > kMaxPages || page_size <= 0 || chunk_tokens <= 0 ||
        window_chunks <= 0)
      return wf::fail(WF_EINVAL,
                      "wf_page_table_create: sizes must be positive (num_pages=%d page_size=%d "
                      "chunk_tokens=%d window_chunks=%d)",
                      num_pages, page_size, chunk_tokens, window_chunks);
    if (pin_anchor && window_chunks < 2)
      return wf::fail(WF_EINVAL, "wf_page_table_create: a pinned anchor needs window_chunks >= 2");
    auto* pt = new wf_page_table();
    pt->num_pages = num_pages;
    pt->page_size = page_size;
    pt->chunk_tokens = chunk_tokens;
    pt->window = window_chunks;
    pt->pin_anchor = pin_anchor != 0;
    pt->ppc = int32_t((int64_t(chunk_tokens) + page_size - 1) / page_size);
    pt->ring.resize(size_t(num_pages));
    if (initial_free_order) {
      std::vector<char> seen(size_t(num_pages), 0);
      for (int32_t i = 0; i < num_pages; ++i) {
        int32_t id = initial_free_order[i];
        if (id < 0 || id >= num_pages || seen[size_t(id)]) {
          delete pt;
          return wf::fail(WF_EINVAL,
                          "wf_page_table_create: initial_free_order is not a permutation of "
                          "0..%d (entry %d = %d)",
                          num_pages - 1, i, id);
        }
        seen[size_t(id)] = 1;
        pt->ring[size_t(i)] = id;
      }
    } else {
      for (int32_t i = 0; i < num_pages; ++i) pt->ring[size_t(i)] = i;
    }
    pt->count = num_pages;
    *out = pt;
    return WF_OK;
  } catch (const std::bad_alloc&) {
    return wf::fail(WF_ENOMEM, "wf_page_table_create: host allocation failed");
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_page_table_create: internal error");
  }
}

extern "C" void wf_page_table_destroy(wf_page_table* pt) { delete pt; }

extern "C" wf_status wf_page_table_pages_per_chunk(const wf_page_table* pt, int32_t* out) {
  if (!pt || !out) return wf::fail(WF_EINVAL, "wf_page_table_pages_per_chunk: NULL argument");
  *out = pt->ppc;
  return WF_OK;
}

extern "C" wf_status wf_page_table_alloc_chunk(wf_page_table* pt, int32_t* out_ids,
                                               int32_t capacity) {
  try {
    if (!pt || !out_ids) return wf::fail(WF_EINVAL, "wf_page_table_alloc_chunk: NULL argument");
    if (capacity < pt->ppc)
      return wf::fail(WF_EINVAL, "wf_page_table_alloc_chunk: capacity %d < pages per chunk %d",
                      capacity, pt->ppc);
    if (pt->has_live)
      return wf::fail(WF_ESTATE, "wf_page_table_alloc_chunk: a live chunk is already allocated");
    if (pt->count < pt->ppc)
      return wf::fail(WF_ENOMEM, "wf_page_table_alloc_chunk: %d free pages, %d needed", pt->count,
                      pt->ppc);
    pt->live.reserve(size_t(pt->ppc));  // may throw before any state changes
    pt->live.clear();
    for (int32_t i = 0; i < pt->ppc; ++i) {
      int32_t id = pt->pop_front();
      pt->live.push_back(id);
      out_ids[i] = id;
    }
    pt->has_live = true;
    return WF_OK;
  } catch (const std::bad_alloc&) {
    return wf::fail(WF_ENOMEM, "wf_page_table_alloc_chunk: host allocation failed");
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_page_table_alloc_chunk: internal error");
  }
}

extern "C" wf_status wf_page_table_commit(wf_page_table* pt, int32_t* evicted_ids,
                                          int32_t capacity, int32_t* n_evicted) {
  try {
    if (!pt || !n_evicted) return wf::fail(WF_EINVAL, "wf_page_table_commit: NULL argument");
    if (!pt->has_live)
      return wf::fail(WF_ESTATE, "wf_page_table_commit: no live chunk to promote");
    const bool will_evict = int32_t(pt->history.size()) + 1 > pt->window;
    if (will_evict && (capacity < pt->ppc || !evicted_ids) && capacity != 0)
      return wf::fail(WF_EINVAL, "wf_page_table_commit: evicted_ids capacity %d < %d", capacity,
                      pt->ppc);
    pt->history.reserve(pt->history.size() + 1);  // may throw before any state changes
    pt->history.push_back(pt->live);
    pt->live.clear();
    pt->has_live = false;
    *n_evicted = 0;
    if (will_evict) {
      size_t idx = pt->pin_anchor ? 1 : 0;
      std::vector<int32_t> gone = std::move(pt->history[idx]);
      pt->history.erase(pt->history.begin() + std::ptrdiff_t(idx));
      for (size_t i = 0; i < gone.size(); ++i) {
        pt->push_back(gone[i]);
        if (evicted_ids && capacity >= pt->ppc) evicted_ids[i] = gone[i];
      }
      *n_evicted = int32_t(gone.size());
    }
    return WF_OK;
  } catch (const std::bad_alloc&) {
    return wf::fail(WF_ENOMEM, "wf_page_table_commit: host allocation failed");
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_page_table_commit: internal error");
  }
}

extern "C" wf_status wf_page_table_export(const wf_page_table* pt, int32_t* out,
                                          int32_t capacity, int32_t* n_hist_chunks) {
  if (!pt || !n_hist_chunks) return wf::fail(WF_EINVAL, "wf_page_table_export: NULL argument");
  const int64_t need = int64_t(pt->history.size()) * pt->ppc;
  if (need > 0 && (!out || capacity < need))
    return wf::fail(WF_EINVAL, "wf_page_table_export: capacity %d < %lld", capacity,
                    static_cast<long long>(need));
  int64_t o = 0;
  for (const auto& c : pt->history)
    for (int32_t id : c) out[o++] = id;
  *n_hist_chunks = int32_t(pt->history.size());
  return WF_OK;
}

extern "C" wf_status wf_page_table_num_free(const wf_page_table* pt, int32_t* out) {
  if (!pt || !out) return wf::fail(WF_EINVAL, "wf_page_table_num_free: NULL argument");
  *out = pt->count;
  return WF_OK;
}
