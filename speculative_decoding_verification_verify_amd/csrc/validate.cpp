// Optional input checks of the compute calls (SPECVERIFY_VALIDATE=1); see
// validate.h.
#include "validate.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "specverify.h"

namespace sv {

namespace {

bool fail(const char* fn, const char* what) {
  std::fprintf(stderr, "specverify: %s: %s\n", fn, what);
  return true;
}

// Device -> host copy of n elements after the stream has drained.
template <typename T>
bool fetch(const char* fn, const T* src, long long n, std::vector<T>& dst) {
  dst.resize((size_t)n);
  if (n == 0) return true;
  if (hipMemcpy(dst.data(), src, (size_t)n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) {
    fail(fn, "copying an input to the host failed");
    return false;
  }
  return true;
}

bool drain(const char* fn, hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) {
    fail(fn, "the stream reported an error before the call");
    return false;
  }
  return true;
}

}  // namespace

bool validate_on() {
  const char* v = std::getenv("SPECVERIFY_VALIDATE");
  return v && v[0] == '1' && v[1] == '\0';
}

int check_pages(const char* fn, const int32_t* block_table, const int32_t* kv_len, int B,
                int extra, int num_blocks, int max_blocks_per_seq, int max_len, hipStream_t st) {
  if (!drain(fn, st)) return SV_ERR_HIP;
  std::vector<int32_t> len, bt;
  if (!fetch(fn, kv_len, B, len) ||
      !fetch(fn, block_table, (long long)B * max_blocks_per_seq, bt))
    return SV_ERR_HIP;
  char msg[256];
  for (int b = 0; b < B; ++b) {
    const long long L = len[b];
    if (L < 0 || (max_len >= 0 && L > max_len) ||
        L + extra > (long long)SV_BLOCK_SIZE * max_blocks_per_seq) {
      std::snprintf(msg, sizeof msg, "kv_len[%d] = %lld: need 0 <= kv_len%s and kv_len + %d <= %lld",
                    b, L, max_len >= 0 ? " <= max_kv_len" : "", extra,
                    (long long)SV_BLOCK_SIZE * max_blocks_per_seq);
      fail(fn, msg);
      return SV_ERR_BAD_INPUT;
    }
    const long long pages = (L + extra + SV_BLOCK_SIZE - 1) / SV_BLOCK_SIZE;
    for (long long p = 0; p < pages; ++p) {
      const int32_t id = bt[(size_t)b * max_blocks_per_seq + p];
      if (id < 0 || id >= num_blocks) {
        std::snprintf(msg, sizeof msg, "block_table[%d][%lld] = %d outside [0, %d) (page of positions "
                      "[%lld, %lld))", b, p, id, num_blocks, p * SV_BLOCK_SIZE,
                      (p + 1) * SV_BLOCK_SIZE);
        fail(fn, msg);
        return SV_ERR_BAD_INPUT;
      }
    }
  }
  return SV_OK;
}

int check_commit(const char* fn, const int32_t* block_table, const int32_t* kv_len,
                 const int32_t* num_accepted, const int32_t* nodes, int B, int N, int num_blocks,
                 int max_blocks_per_seq, hipStream_t st) {
  if (!drain(fn, st)) return SV_ERR_HIP;
  std::vector<int32_t> len, acc, bt, nd;
  if (!fetch(fn, kv_len, B, len) || !fetch(fn, num_accepted, B, acc) ||
      !fetch(fn, block_table, (long long)B * max_blocks_per_seq, bt) ||
      (nodes && !fetch(fn, nodes, (long long)B * N, nd)))
    return SV_ERR_HIP;
  char msg[256];
  for (int b = 0; b < B; ++b) {
    const long long n = acc[b], L0 = (long long)len[b] - n - 1;
    if (n < 0 || n >= N || L0 < 0 || L0 + N > (long long)SV_BLOCK_SIZE * max_blocks_per_seq) {
      std::snprintf(msg, sizeof msg, "sequence %d: num_accepted = %lld, kv_len = %d: need 0 <= n < %d "
                    "and 0 <= kv_len - n - 1, kv_len - n - 1 + %d <= %lld", b, n, len[b], N, N,
                    (long long)SV_BLOCK_SIZE * max_blocks_per_seq);
      fail(fn, msg);
      return SV_ERR_BAD_INPUT;
    }
    for (long long p = 0; p < (L0 + N + SV_BLOCK_SIZE - 1) / SV_BLOCK_SIZE; ++p) {
      const int32_t id = bt[(size_t)b * max_blocks_per_seq + p];
      if (id < 0 || id >= num_blocks) {
        std::snprintf(msg, sizeof msg, "block_table[%d][%lld] = %d outside [0, %d)", b, p, id,
                      num_blocks);
        fail(fn, msg);
        return SV_ERR_BAD_INPUT;
      }
    }
    if (nodes) {
      for (long long j = 0; j < n; ++j) {
        const int32_t v = nd[(size_t)b * N + j];
        if (v < 0 || v >= N) {
          std::snprintf(msg, sizeof msg, "nodes[%d][%lld] = %d outside [0, %d)", b, j, v, N);
          fail(fn, msg);
          return SV_ERR_BAD_INPUT;
        }
      }
    }
  }
  return SV_OK;
}

int check_logits(const char* fn, const char* name, const void* x, long long rows, int V,
                 int dtype, hipStream_t st) {
  if (!drain(fn, st)) return SV_ERR_HIP;
  // Row blocks of about 16 MB, so the host copy stays bounded.
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  const long long per = std::max(1LL, (long long)((16u << 20) / ((size_t)V * es)));
  std::vector<unsigned char> buf;
  char msg[256];
  for (long long r0 = 0; r0 < rows; r0 += per) {
    const long long nr = std::min(per, rows - r0);
    buf.resize((size_t)nr * V * es);
    if (hipMemcpy(buf.data(), static_cast<const unsigned char*>(x) + (size_t)r0 * V * es,
                  buf.size(), hipMemcpyDeviceToHost) != hipSuccess) {
      fail(fn, "copying logits to the host failed");
      return SV_ERR_HIP;
    }
    for (long long r = 0; r < nr; ++r) {
      bool finite = false;
      for (int v = 0; v < V; ++v) {
        const size_t at = ((size_t)r * V + v) * es;
        uint32_t u;
        if (es == 2) {
          uint16_t h;
          std::memcpy(&h, &buf[at], 2);
          u = (uint32_t)h << 16;
        } else {
          std::memcpy(&u, &buf[at], 4);
        }
        const bool nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
        if (nan || u == 0x7F800000u) {
          std::snprintf(msg, sizeof msg, "%s row %lld, entry %d is %s", name, r0 + r, v,
                        nan ? "NaN" : "+inf");
          fail(fn, msg);
          return SV_ERR_BAD_INPUT;
        }
        finite = finite || u != 0xFF800000u;
      }
      if (!finite) {
        std::snprintf(msg, sizeof msg, "%s row %lld has no finite logit", name, r0 + r);
        fail(fn, msg);
        return SV_ERR_BAD_INPUT;
      }
    }
  }
  return SV_OK;
}

int check_tokens(const char* fn, const int32_t* tok, long long n, int V, int stride, int skip,
                 hipStream_t st) {
  if (!drain(fn, st)) return SV_ERR_HIP;
  std::vector<int32_t> t;
  if (!fetch(fn, tok, n, t)) return SV_ERR_HIP;
  char msg[256];
  for (long long i = 0; i < n; ++i) {
    if (i % stride < skip) continue;
    if (t[i] < 0 || t[i] >= V) {
      std::snprintf(msg, sizeof msg, "token [%lld][%lld] = %d outside [0, %d)", i / stride,
                    i % stride, t[i], V);
      fail(fn, msg);
      return SV_ERR_BAD_INPUT;
    }
  }
  return SV_OK;
}

int check_parents(const char* fn, const int32_t* parents, int B, int N, hipStream_t st) {
  if (!drain(fn, st)) return SV_ERR_HIP;
  std::vector<int32_t> p;
  if (!fetch(fn, parents, (long long)B * N, p)) return SV_ERR_HIP;
  char msg[256];
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < N; ++i) {
      const int32_t v = p[(size_t)b * N + i];
      if (i == 0 ? v != -1 : (v < 0 || v >= i)) {
        std::snprintf(msg, sizeof msg, "parents[%d][%d] = %d: %s", b, i, v,
                      i == 0 ? "the root's parent must be -1" : "a parent must precede its node");
        fail(fn, msg);
        return SV_ERR_BAD_INPUT;
      }
    }
  return SV_OK;
}

int check_floats(const char* fn, const char* name, const float* x, long long n, bool unit,
                 hipStream_t st) {
  if (!drain(fn, st)) return SV_ERR_HIP;
  std::vector<float> f;
  if (!fetch(fn, x, n, f)) return SV_ERR_HIP;
  char msg[256];
  for (long long i = 0; i < n; ++i) {
    const bool ok = unit ? (f[i] >= 0.f && f[i] < 1.f) : std::isfinite(f[i]);
    if (!ok) {
      std::snprintf(msg, sizeof msg, "%s[%lld] = %g is not %s", name, i, (double)f[i],
                    unit ? "in [0, 1)" : "finite");
      fail(fn, msg);
      return SV_ERR_BAD_INPUT;
    }
  }
  return SV_OK;
}

int finish(const char* fn, hipStream_t st, int status) {
  if (status != SV_OK) return status;
  const hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "the call's kernels failed: %s", hipGetErrorString(e));
    fail(fn, msg);
    return SV_ERR_HIP;
  }
  return SV_OK;
}

}  // namespace sv
