// Commit of the window's K/V after the verifier.
//
// Verification extends the verifier's KV cache by the window; after a
// rejection everything past the accepted prefix is wrong.  Either the window
// was written to a scratch buffer and the accepted rows are committed into
// the cache, or it was written in place and only the logical length moves
// (AI Engineering from Scratch, "Speculative decoding and EAGLE-3", "Rolling
// back the KV cache"; sglang_spec_decode README, the provisional KV layer).
// For a draft tree written in place the accepted path is scattered over the
// window slots and must be compacted (thakicloud, "speedup went from 1.4x to
// 0.8x", "Grading every branch in one pass": the surviving path is kept).
//
// k_kv_commit: grid (B, Hkv), block 256.  Surviving row j (the root, then
// the accepted nodes in path order) goes to position L0 + j.  All sources of
// one (sequence, KV head) are read into LDS before any slot is written, since
// in place a destination can be the source of a later row.

#include "common.h"
#include "validate.h"

namespace sv {

constexpr int kCommitThreads = 256;
constexpr int kCommitMaxRows = SV_MAX_K + 1;

template <typename T>
__global__ __launch_bounds__(kCommitThreads) void k_kv_commit(
    T* __restrict__ kc, T* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ nacc,
    const int32_t* __restrict__ nodes, const T* __restrict__ ks, const T* __restrict__ vs, int N,
    int Hkv, int D, int num_blocks, int mbps) {
  constexpr int X = 16 / sizeof(T);               // elements per 16-byte chunk of a key
  __shared__ T s_k[kCommitMaxRows * 128], s_v[kCommitMaxRows * 128];
  __shared__ int s_row[kCommitMaxRows];
  const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int n = nacc[b];
  if (n < 0 || n >= N) return;                    // not a verifier's output
  const int L0 = kv_len[b] - n - 1;
  if (L0 < 0) return;
  const int rows = n + 1;
  if (tid < rows) {
    int r = tid;
    if (nodes && tid > 0) r = clampi(nodes[(size_t)b * N + tid - 1], 0, N - 1);
    s_row[tid] = r;
  }
  __syncthreads();
  const int32_t* btb = bt + (size_t)b * mbps;
  const size_t page = (size_t)D * 16;
  auto kaddr = [&](int p, int d) {
    const int blk = clampi(btb[min(p >> 4, mbps - 1)], 0, num_blocks - 1);
    return ((size_t)blk * Hkv + g) * page + ((size_t)(d / X) * 16 + (p & 15)) * X + d % X;
  };
  auto vaddr = [&](int p, int d) {
    const int blk = clampi(btb[min(p >> 4, mbps - 1)], 0, num_blocks - 1);
    return ((size_t)blk * Hkv + g) * page + (size_t)d * 16 + (p & 15);
  };
  for (int e = tid; e < rows * D; e += kCommitThreads) {
    const int j = e / D, d = e - j * D;
    const int r = s_row[j];
    if (ks) {
      const size_t src = (((size_t)b * N + r) * Hkv + g) * D + d;
      s_k[e] = ks[src];
      s_v[e] = vs[src];
    } else if (r != j) {
      s_k[e] = kc[kaddr(L0 + r, d)];
      s_v[e] = vc[vaddr(L0 + r, d)];
    }
  }
  __syncthreads();
  for (int e = tid; e < rows * D; e += kCommitThreads) {
    const int j = e / D, d = e - j * D;
    if (ks || s_row[j] != j) {
      kc[kaddr(L0 + j, d)] = s_k[e];
      vc[vaddr(L0 + j, d)] = s_v[e];
    }
  }
}

}  // namespace sv

extern "C" int spec_kv_commit(void* k_cache, void* v_cache, const int32_t* block_table,
                              const int32_t* kv_len, const int32_t* num_accepted,
                              const int32_t* nodes, const void* k_src, const void* v_src, int B,
                              int N, int Hkv, int D, int block_size, int num_blocks,
                              int max_blocks_per_seq, int dtype, void* hip_stream) {
  if (B < 0 || N < 1 || Hkv < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
    return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if ((k_src == nullptr) != (v_src == nullptr)) return SV_ERR_INVALID_ARG;
  if (N > sv::kCommitMaxRows || block_size != SV_BLOCK_SIZE || (D != 64 && D != 128))
    return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!k_cache || !v_cache || !block_table || !kv_len || !num_accepted) return SV_ERR_INVALID_ARG;
  if (Hkv > 65535) return SV_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const char* fn = "spec_kv_commit";
  const bool chk = sv::validate_on();
  if (chk) {
    const int s = sv::check_commit(fn, block_table, kv_len, num_accepted, nodes, B, N, num_blocks,
                                   max_blocks_per_seq, st);
    if (s != SV_OK) return s;
  }
  // A chain written in place is already where it belongs.
  if (!nodes && !k_src) return SV_OK;
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(sv::k_kv_commit<uint16_t>, dim3(B, Hkv), dim3(sv::kCommitThreads), 0, st,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), block_table,
                       kv_len, num_accepted, nodes, static_cast<const uint16_t*>(k_src),
                       static_cast<const uint16_t*>(v_src), N, Hkv, D, num_blocks, max_blocks_per_seq);
  else
    hipLaunchKernelGGL(sv::k_kv_commit<float>, dim3(B, Hkv), dim3(sv::kCommitThreads), 0, st,
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), block_table, kv_len,
                       num_accepted, nodes, static_cast<const float*>(k_src),
                       static_cast<const float*>(v_src), N, Hkv, D, num_blocks, max_blocks_per_seq);
  const int status = hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
  return chk ? sv::finish(fn, st, status) : status;
}
