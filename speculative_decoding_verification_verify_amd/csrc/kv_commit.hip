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
// k_kv_commit: grid (B, Hkv), block 256.  Also, with pre set, the append
// mode of the window attention: all N rows from k_new / v_new into positions
// kv_len + j before the attention reads them.  Surviving row j (the root, then
// the accepted nodes in path order) goes to position L0 + j.  All sources of
// one (sequence, KV head) are read into LDS before any slot is written, since
// in place a destination can be the source of a later row.  The survivors'
// positions L0 .. L0 + n span at most two pages (n + 1 <= 17), whose block
// numbers are read once.  Sources are read as 16-byte chunks (a key's chunk
// is 16 contiguous bytes in the page, a row of k_src / v_src is contiguous);
// in place, a value row is gathered from its slot's strided entries.  Stores:
// one 16-byte chunk per (row, key chunk); for the values, each run of
// 16 / sizeof(T) consecutive slots of one coordinate that the survivors fill
// is one 16-byte store, and the slots of a run they fill only in part are
// stored one by one, so no slot outside L0 .. L0 + n is written.

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
    int Hkv, int D, int num_blocks, int mbps, int pre) {
  constexpr int X = 16 / sizeof(T);               // elements per 16-byte chunk / value run
  __shared__ __align__(16) T s_k[kCommitMaxRows * 128];
  __shared__ __align__(16) T s_v[kCommitMaxRows * 128];
  __shared__ int s_row[kCommitMaxRows];
  __shared__ int s_blk[2];
  const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int CPR = D / X;                          // 16-byte chunks per row
  // Scratch rows of a chain: row j's source is row j, known before the
  // lengths, so every row is requested with them (one round trip for both).
  const bool early = ks && !nodes;
  if (early) {
    for (int e = tid; e < N * CPR; e += kCommitThreads) {
      const int j = e / CPR, c = e - j * CPR;
      const size_t src = (((size_t)b * N + j) * Hkv + g) * D + (size_t)c * X;
      *reinterpret_cast<u32x4_t*>(s_k + j * D + c * X) = *reinterpret_cast<const u32x4_t*>(ks + src);
      *reinterpret_cast<u32x4_t*>(s_v + j * D + c * X) = *reinterpret_cast<const u32x4_t*>(vs + src);
    }
  }
  // pre: every row of the window, ahead of the verifier (L0 = kv_len).
  const int n = pre ? N - 1 : nacc[b];
  if (n < 0 || n >= N) return;                    // not a verifier's output
  const int L0 = pre ? kv_len[b] : kv_len[b] - n - 1;
  if (L0 < 0) return;
  const int rows = n + 1;
  const int pg0 = L0 >> 4;
  if (tid < rows) {
    int r = tid;
    if (nodes && tid > 0) r = clampi(nodes[(size_t)b * N + tid - 1], 0, N - 1);
    s_row[tid] = r;
  }
  if (tid < 2) s_blk[tid] = clampi(bt[(size_t)b * mbps + min(pg0 + tid, mbps - 1)], 0, num_blocks - 1);
  __syncthreads();
  const size_t page = (size_t)D * 16;
  // Slots L0 .. L0 + N - 1 (every source and destination) lie in pages pg0, pg0 + 1.
  auto pbase = [&](int p) { return ((size_t)s_blk[min((p >> 4) - pg0, 1)] * Hkv + g) * page; };
  for (int e = tid; !early && e < rows * CPR; e += kCommitThreads) {
    const int j = e / CPR, c = e - j * CPR;
    const int r = s_row[j];
    u32x4_t kv, vv;
    if (ks) {
      const size_t src = (((size_t)b * N + r) * Hkv + g) * D + (size_t)c * X;
      kv = *reinterpret_cast<const u32x4_t*>(ks + src);
      vv = *reinterpret_cast<const u32x4_t*>(vs + src);
    } else {
      const int p = L0 + r;
      const size_t pb = pbase(p);
      kv = *reinterpret_cast<const u32x4_t*>(kc + pb + ((size_t)c * 16 + (p & 15)) * X);
      T v[X];
#pragma unroll
      for (int q = 0; q < X; ++q) v[q] = vc[pb + (size_t)(c * X + q) * 16 + (p & 15)];
      vv = *reinterpret_cast<const u32x4_t*>(v);
    }
    *reinterpret_cast<u32x4_t*>(s_k + j * D + c * X) = kv;
    *reinterpret_cast<u32x4_t*>(s_v + j * D + c * X) = vv;
  }
  if (!early) __syncthreads();
  for (int e = tid; e < rows * CPR; e += kCommitThreads) {
    const int j = e / CPR, c = e - j * CPR;
    const int p = L0 + j;
    *reinterpret_cast<u32x4_t*>(kc + pbase(p) + ((size_t)c * 16 + (p & 15)) * X) =
        *reinterpret_cast<const u32x4_t*>(s_k + j * D + c * X);
  }
  // Value runs q0 .. q1 of X slots cover L0 .. L0 + n; the runs of one
  // coordinate go to adjacent threads.
  const int s1 = L0 + n, q0 = L0 / X, nq = s1 / X - q0 + 1;
  for (int e = tid; e < D * nq; e += kCommitThreads) {
    const int d = e / nq, q = q0 + e % nq;
    const int lo = max(q * X, L0), hi = min(q * X + X - 1, s1);
    const size_t vb = pbase(q * X) + (size_t)d * 16;
    if (lo == q * X && hi == q * X + X - 1) {
      T v[X];
#pragma unroll
      for (int k = 0; k < X; ++k) v[k] = s_v[(lo + k - L0) * D + d];
      *reinterpret_cast<u32x4_t*>(vc + vb + (lo & 15)) = *reinterpret_cast<const u32x4_t*>(v);
    } else {
      for (int sl = lo; sl <= hi; ++sl) vc[vb + (sl & 15)] = s_v[(sl - L0) * D + d];
    }
  }
}

hipError_t launch_window_store(void* kc, void* vc, const int32_t* bt, const int32_t* kv_len,
                               const void* kn, const void* vn, int B, int N, int Hkv, int D,
                               int num_blocks, int mbps, int dtype, hipStream_t st) {
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(k_kv_commit<uint16_t>, dim3(B, Hkv), dim3(kCommitThreads), 0, st,
                       static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), bt, kv_len, nullptr,
                       nullptr, static_cast<const uint16_t*>(kn), static_cast<const uint16_t*>(vn), N, Hkv,
                       D, num_blocks, mbps, 1);
  else
    hipLaunchKernelGGL(k_kv_commit<float>, dim3(B, Hkv), dim3(kCommitThreads), 0, st,
                       static_cast<float*>(kc), static_cast<float*>(vc), bt, kv_len, nullptr, nullptr,
                       static_cast<const float*>(kn), static_cast<const float*>(vn), N, Hkv, D,
                       num_blocks, mbps, 1);
  return hipGetLastError();
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
  // Keys, value runs and scratch rows move as 16-byte vectors.
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
       reinterpret_cast<uintptr_t>(k_src) | reinterpret_cast<uintptr_t>(v_src)) & 15)
    return SV_ERR_INVALID_ARG;
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
                       static_cast<const uint16_t*>(v_src), N, Hkv, D, num_blocks, max_blocks_per_seq, 0);
  else
    hipLaunchKernelGGL(sv::k_kv_commit<float>, dim3(B, Hkv), dim3(sv::kCommitThreads), 0, st,
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), block_table, kv_len,
                       num_accepted, nodes, static_cast<const float*>(k_src),
                       static_cast<const float*>(v_src), N, Hkv, D, num_blocks, max_blocks_per_seq, 0);
  const int status = hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
  return chk ? sv::finish(fn, st, status) : status;
}
