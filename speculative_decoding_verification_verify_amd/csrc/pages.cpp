// Host-side KV page list with provisional pages for the verify window.
//
// Verification extends each sequence's KV cache by the window before the
// verifier knows how much of it survives; the pages that only a rejected
// tail used must go back to the pool (AI Engineering from Scratch,
// "Speculative decoding and EAGLE-3", "Rolling back the KV cache";
// sglang_spec_decode README, the provisional KV layer).
//
// A sequence owns pages for positions [0, 16 * npages).  reserve() grows
// that range for the next window (the new pages are provisional), commit()
// frees every page whose first position lies at or past the committed
// length and keeps the rest, release() frees all of them.  The lowest-
// numbered free page is always handed out first (a min-heap), so the block
// tables are reproducible.  Every page has one owner entry (a sequence or
// free): a page freed twice, or freed by a sequence that does not own it, is
// reported instead of corrupting the pool.  Not thread-safe: one pool per
// scheduler thread, or a lock around the calls.

#include <algorithm>
#include <functional>
#include <new>
#include <queue>
#include <vector>

#include "specverify.h"

struct sv_page_pool {
  int num_blocks = 0, max_seqs = 0, mbps = 0;
  std::priority_queue<int, std::vector<int>, std::greater<int>> free_heap;
  std::vector<int> owner;                  // per page: owning sequence, or -1 when free
  std::vector<std::vector<int>> pages;     // per sequence, in position order
  std::vector<int32_t> table;              // [max_seqs, mbps], unused entries 0
};

namespace {

constexpr int kPage = SV_BLOCK_SIZE;

int pages_for(long long len) { return (int)((len + kPage - 1) / kPage); }

bool seq_ok(const sv_page_pool* p, int seq) { return p && seq >= 0 && seq < p->max_seqs; }

// Frees pages [keep, end) of a sequence, newest first.
int drop_tail(sv_page_pool* p, int seq, int keep) {
  std::vector<int>& pg = p->pages[seq];
  for (int k = (int)pg.size() - 1; k >= keep; --k) {
    const int blk = pg[k];
    if (blk < 0 || blk >= p->num_blocks || p->owner[blk] != seq) return SV_ERR_INVALID_ARG;
    p->owner[blk] = -1;
    p->free_heap.push(blk);
    p->table[(size_t)seq * p->mbps + k] = 0;
  }
  pg.resize(keep);
  return SV_OK;
}

}  // namespace

extern "C" sv_page_pool* spec_pages_create(int num_blocks, int max_seqs, int max_blocks_per_seq) {
  if (num_blocks < 1 || max_seqs < 1 || max_blocks_per_seq < 1) return nullptr;
  sv_page_pool* p = new (std::nothrow) sv_page_pool;
  if (!p) return nullptr;
  try {
    p->num_blocks = num_blocks;
    p->max_seqs = max_seqs;
    p->mbps = max_blocks_per_seq;
    p->owner.assign(num_blocks, -1);
    p->pages.assign(max_seqs, {});
    p->table.assign((size_t)max_seqs * max_blocks_per_seq, 0);
    std::vector<int> all(num_blocks);
    for (int i = 0; i < num_blocks; ++i) all[i] = i;
    p->free_heap = decltype(p->free_heap)(std::greater<int>(), std::move(all));
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

extern "C" void spec_pages_destroy(sv_page_pool* pool) { delete pool; }

extern "C" int spec_pages_reserve(sv_page_pool* p, int seq, int total_len) {
  if (!seq_ok(p, seq) || total_len < 0) return SV_ERR_INVALID_ARG;
  const int need = pages_for(total_len);
  if (need > p->mbps) return SV_ERR_INVALID_ARG;
  std::vector<int>& pg = p->pages[seq];
  const int extra = need - (int)pg.size();
  if (extra <= 0) return SV_OK;
  if (extra > (int)p->free_heap.size()) return SV_ERR_NO_PAGES;    // nothing taken
  for (int k = 0; k < extra; ++k) {
    const int blk = p->free_heap.top();
    p->free_heap.pop();
    p->owner[blk] = seq;
    p->table[(size_t)seq * p->mbps + pg.size()] = blk;
    pg.push_back(blk);
  }
  return SV_OK;
}

extern "C" int spec_pages_commit(sv_page_pool* p, int seq, int committed_len) {
  if (!seq_ok(p, seq) || committed_len < 0) return SV_ERR_INVALID_ARG;
  const int keep = pages_for(committed_len);
  if (keep > (int)p->pages[seq].size()) return SV_ERR_INVALID_ARG;
  return drop_tail(p, seq, keep);
}

extern "C" int spec_pages_release(sv_page_pool* p, int seq) {
  if (!seq_ok(p, seq)) return SV_ERR_INVALID_ARG;
  return drop_tail(p, seq, 0);
}

extern "C" int spec_pages_free_count(const sv_page_pool* p) {
  return p ? (int)p->free_heap.size() : SV_ERR_INVALID_ARG;
}

extern "C" int spec_pages_seq_blocks(const sv_page_pool* p, int seq) {
  return seq_ok(p, seq) ? (int)p->pages[seq].size() : SV_ERR_INVALID_ARG;
}

extern "C" const int32_t* spec_pages_block_table(const sv_page_pool* p) {
  return p ? p->table.data() : nullptr;
}

extern "C" int spec_pages_check(const sv_page_pool* p) {
  if (!p) return SV_ERR_INVALID_ARG;
  std::vector<int> seen(p->num_blocks, 0);
  for (int s = 0; s < p->max_seqs; ++s) {
    const std::vector<int>& pg = p->pages[s];
    if ((int)pg.size() > p->mbps) return SV_ERR_INVALID_ARG;
    for (int k = 0; k < p->mbps; ++k) {
      const int32_t t = p->table[(size_t)s * p->mbps + k];
      if (k < (int)pg.size() ? t != pg[k] : t != 0) return SV_ERR_INVALID_ARG;
    }
    for (int blk : pg) {
      if (blk < 0 || blk >= p->num_blocks || p->owner[blk] != s || seen[blk]++) return SV_ERR_INVALID_ARG;
    }
  }
  auto heap = p->free_heap;
  while (!heap.empty()) {
    const int blk = heap.top();
    heap.pop();
    if (blk < 0 || blk >= p->num_blocks || p->owner[blk] != -1 || seen[blk]++) return SV_ERR_INVALID_ARG;
  }
  for (int blk = 0; blk < p->num_blocks; ++blk)
    if (seen[blk] != 1) return SV_ERR_INVALID_ARG;
  return SV_OK;
}
