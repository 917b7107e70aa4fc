// Grouped-query attention of the K+1 verify positions over a paged KV cache,
// causal inside the draft window.
//
// The verifier scores x0 and the drafts d_1..d_K in one forward pass over
// prefix + drafts (AI Engineering from Scratch, "Speculative decoding and
// EAGLE-3", "Concept"; devpost "phoenix", "What it does"); decode-time
// attention is bound by reading the KV cache from memory (quickscale.ai,
// "Quand et pourquoi utiliser le speculative decoding", section 1), so the
// kernel is built to stream K and V once at full HBM bandwidth.
//
// bf16 path (k_attn_stream): a persistent grid, every workgroup resident from
// the start (one 8-wave workgroup per CU for 32-row tiles; the 64-row variant
// needs about 480 registers per lane and runs one 4-wave workgroup per CU).
// The work list is every page pair (32 keys) of every (sequence, KV head), in
// that order; each workgroup takes an equal contiguous share of it
// (stream-K), so sequences of very different lengths still keep every CU busy
// to the end.  Inside a share, each (sequence, KV head) segment is one online
// softmax over all G = Hq/Hkv query heads and all K+1 positions of that KV
// head (one or two 32-row tiles), so each K/V byte is read once.  The waves
// of a workgroup take every NW-th page pair:
//   S^T (32 keys x 32 rows) = K . Q^T   8 x v_mfma_f32_32x32x16_bf16 (D=128)
//   O^T (32 d x 32 rows)   += V^T . P^T 2 x 4 MFMAs per pair
// The MFMA key order is permuted so that the C registers of S^T are exactly
// the B operand of the P.V product (lane l holds tokens 8*(l/32)..+7 of each
// page for row l%32), and so that every K and V load is a 16-byte nontemporal
// vector with the 64 lanes of one instruction reading 512 contiguous bytes of
// each page.  No LDS is touched in the key loop; the next pair's K is
// requested right after this pair's scores and its V right after P.V, so
// loads stay in flight through the softmax.  At the end of a segment each
// wave stores its O, rescaled to the common row maximum, in its own LDS
// buffer, and the buffers are summed in fixed wave order.  A segment a
// workgroup covers entirely is written out directly; the at most two partial
// segments of a workgroup go to the workspace and k_attn_stream_combine
// merges them (log-sum-exp weights, fixed order).
//
// fp32 path (k_attn_valu): plain VALU kernel, one wave per query row; used for
// fp32 caches (the correctness configuration).

#include <algorithm>
#include <atomic>

#include "common.h"
#include "validate.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#ifndef SV_ATTN_WAVES
#define SV_ATTN_WAVES 8         // waves per workgroup of the one-tile stream kernel
#endif
// Waves per workgroup: the two-tile kernel needs about 480 registers per
// lane, so only one wave per SIMD fits and it keeps four waves.
template <int NT> constexpr int stream_waves() { return NT == 1 ? SV_ATTN_WAVES : 4; }
constexpr int kCombineThreads = 256;
constexpr int kPairKeys = 32;
constexpr int kStreamMaxWG = 1024;   // workspace is sized for this many workgroups

// Tuning knobs (compile-time).
#ifndef SV_ATTN_NT_LOADS
#define SV_ATTN_NT_LOADS 1      // nontemporal K/V loads: streamed once, keep them out of L2
#endif
#ifndef SV_ATTN_MIN_PAIRS_PER_WG
#define SV_ATTN_MIN_PAIRS_PER_WG 16
#endif
#ifndef SV_ATTN_LAZY
#define SV_ATTN_LAZY 8.0f       // rescale O only when the row max grows by > 2^8
#endif
#ifndef SV_ATTN_WAVES_1T
#define SV_ATTN_WAVES_1T 2      // waves per SIMD the one-tile kernel must fit
#endif

// Measurement build only (build.py --out ... --define SV_ATTN_TIMESTAMPS=1):
// each wave of k_attn_stream stamps the device's constant 100 MHz clock at
// its start, when its segment loop starts, and at the end of each segment's
// pair loop and of its merge; spec_attn_timestamps copies the stamps of the
// last launch to the host.  Per wave, kTsEv words: [0] start, [1] loop
// start, [2 + 2k] / [3 + 2k] pair-loop end / merge end of segment k (k < 10),
// [kTsEv - 2] waves per workgroup, [kTsEv - 1] segments.
#ifndef SV_ATTN_TIMESTAMPS
#define SV_ATTN_TIMESTAMPS 0
#endif
#if SV_ATTN_TIMESTAMPS
constexpr int kTsEv = 24;
constexpr int kTsSeg = (kTsEv - 4) / 2;
__device__ unsigned long long g_attn_ts[kStreamMaxWG * 8 * kTsEv];
#define SV_TS(slot) \
  do { if (lane == 0) tsp[slot] = __builtin_amdgcn_s_memrealtime(); } while (0)
#endif

__device__ __forceinline__ bf16x8 load_kv(const uint16_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#if SV_ATTN_NT_LOADS
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(q));
#else
  return __builtin_bit_cast(bf16x8, *q);
#endif
}

__device__ __forceinline__ void pair_blocks(int (&blk)[2], int pr, const int32_t* __restrict__ btb,
                                            int mbps, int num_blocks) {
  // Both table entries are requested before either is used (one wait).
  const int e0 = btb[min(2 * pr, mbps - 1)];
  const int e1 = btb[min(2 * pr + 1, mbps - 1)];
  blk[0] = clampi(e0, 0, num_blocks - 1);
  blk[1] = clampi(e1, 0, num_blocks - 1);
}

// K page layout [D/8][16][8]: chunk c (8 coordinates) of the 16 tokens is
// 256 contiguous bytes, so each load of a wave reads four whole 256-byte
// runs.  A measurement build with SV_K_TOKEN_MAJOR=1 reads token-major pages
// [16][D] instead through the same lanes (each load then touches 32 rows
// of 256 bytes, 32 bytes of each): it serves only to time the two layouts
// against each other, through spec_verify_attn (its window and commit
// paths still write the default layout).
#ifndef SV_K_TOKEN_MAJOR
#define SV_K_TOKEN_MAJOR 0
#endif

// K operand of a page pair: lane holds key k_tok of page k_page, chunks 2kk+hh.
template <int D>
__device__ __forceinline__ void load_k(bf16x8 (&kf)[D / 16], const int (&blk)[2],
                                       const uint16_t* __restrict__ kc, int Hkv, int g, int k_page,
                                       int k_tok, int hh) {
  const uint16_t* kpage = kc + ((size_t)(k_page ? blk[1] : blk[0]) * Hkv + g) * ((size_t)D * 16);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    kf[kk] = load_kv(kpage + (SV_K_TOKEN_MAJOR ? k_tok * D + (2 * kk + hh) * 8
                                               : ((2 * kk + hh) * 16 + k_tok) * 8));
}

// V operand of a page pair: lane holds tokens 8hh..8hh+7 of value coordinate 32j + l32.
template <int D>
__device__ __forceinline__ void load_v(bf16x8 (&vf)[2][D / 32], const int (&blk)[2],
                                       const uint16_t* __restrict__ vc, int Hkv, int g, int l32, int hh) {
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const uint16_t* vpage = vc + ((size_t)blk[sg] * Hkv + g) * ((size_t)D * 16);
#pragma unroll
    for (int j = 0; j < D / 32; ++j) vf[sg][j] = load_kv(vpage + (32 * j + l32) * 16 + 8 * hh);
  }
}

// Zero the V entries of keys past the sequence end: those slots may hold
// anything (even NaN); their probability is 0, but 0 * NaN would reach O.
template <int D>
__device__ __forceinline__ void mask_v_tail(bf16x8 (&vf)[2][D / 32], int pr, int L, int hh) {
  const int key0 = pr * kPairKeys + 8 * hh;
  if (pr * kPairKeys + kPairKeys > L) {
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key0 + sg * 16 + e >= L)
#pragma unroll
          for (int j = 0; j < D / 32; ++j) vf[sg][j][e] = (__bf16)0.f;
  }
}

// ---- Window taken from the projection output (k_new / v_new [B, K1, Hkv, D])
// instead of the cache (read mode; append mode stores the rows into their
// slots with a copy kernel first and then runs the plain kernel): the pair
// that holds window keys reads them there.

// True (wave-uniform) when pair pr of a sequence with committed length L0
// holds window keys L0 .. L0 + K1 - 1.
__device__ __forceinline__ bool pair_has_window(int pr, int L0, int K1) {
  return pr * kPairKeys < L0 + K1 && pr * kPairKeys + kPairKeys > L0;
}

// K operand of a pair with window keys: a window key's 16-byte chunks come
// from k_new (one address per lane: the chunk stride differs, 16 elements
// there, 256 in the page).
template <int D>
__device__ __forceinline__ void load_k_window(bf16x8 (&kf)[D / 16], const int (&blk)[2],
                                              const uint16_t* __restrict__ kc,
                                              const uint16_t* __restrict__ kn, int b, int K1,
                                              int Hkv, int g, int L0, int pr, int k_page, int k_tok,
                                              int hh) {
  const int i = pr * kPairKeys + k_page * 16 + k_tok - L0;
  const bool win = (unsigned)i < (unsigned)K1;
  const uint16_t* base =
      win ? kn + (((size_t)b * K1 + i) * Hkv + g) * D + hh * 8
          : kc + ((size_t)(k_page ? blk[1] : blk[0]) * Hkv + g) * ((size_t)D * 16) + (hh * 16 + k_tok) * 8;
  const int step = win ? 16 : 256;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(base + kk * step);
}

// V of the window: v_new holds the tokens of one value coordinate strided,
// so a segment's window rows are staged in LDS ([row][d], bf16) ahead of
// time, and the pair with window keys takes those tokens' entries from there.
constexpr int kWinRows = SV_MAX_K + 1;

template <int D>
__device__ __forceinline__ void window_v(bf16x8 (&vf)[2][D / 32], const uint16_t* s_win, int K1,
                                         int L0, int pr, int l32, int hh) {
#pragma unroll
  for (int sg = 0; sg < 2; ++sg)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = pr * kPairKeys + sg * 16 + 8 * hh + e - L0;
      if ((unsigned)i < (unsigned)K1) {
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
          vf[sg][j][e] = __builtin_bit_cast(__bf16, s_win[i * D + 32 * j + l32]);
      }
    }
}

// Scores of one page pair for tile nt, window-causal mask, online-softmax
// update of (m, l, O) and the bf16 probabilities for the P.V product.
template <int D, int NT>
__device__ __forceinline__ void score_pair(const bf16x8 (&kf)[D / 16], int pr, int hh, int nt,
                                           const bf16x8 (&qf)[NT][D / 16], const uint32_t (&am)[NT],
                                           int L0, float sl2, f32x16 (&o)[NT][D / 32],
                                           float (&m_run)[NT], float (&l_run)[NT], bf16x8 (&pf)[2]) {
  constexpr int KK = D / 16, DT = D / 32;
  const int key0 = pr * kPairKeys + 8 * hh;     // key of reg r: key0 + (r>>3)*16 + (r&7)
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[nt][kk], s, 0, 0, 0);
  float mx = -INFINITY;
  // Prefix keys (< L0) are visible; window key L0 + j is visible iff bit j of
  // the row's ancestor set is set (a chain's row i has bits 0..i); later keys
  // have no bit.  One 8-bit word per run of 8 consecutive keys.
#pragma unroll
  for (int grp = 0; grp < 2; ++grp) {
    const int j0 = key0 + grp * 16 - L0;
    uint32_t vb;
    if (j0 >= 32) vb = 0u;
    else if (j0 >= 0) vb = (am[nt] >> j0) & 0xFFu;
    else if (j0 <= -8) vb = 0xFFu;
    else vb = (((1u << -j0) - 1u) | (am[nt] << -j0)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = grp * 8 + e;
      const float v = ((vb >> e) & 1u) ? s[r] * sl2 : -INFINITY;
      s[r] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // Lazy rescaling: keep the running reference unless the row max grows by
  // more than SV_ATTN_LAZY (so p <= 2^SV_ATTN_LAZY); O / l is unchanged.
  const bool need = mx > m_run[nt] + SV_ATTN_LAZY;
  if (__ballot(need)) {
    const float m_new = need ? mx : m_run[nt];
    const float alpha = need ? exp2_dev(m_run[nt] - m_new) : 1.f;
    l_run[nt] *= alpha;
    m_run[nt] = m_new;
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nt][j][r] *= alpha;
  }
  const float m_use = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = exp2_dev(s[r] - m_use);
    rs += s[r];
  }
  rs += __shfl_xor(rs, 32, 64);
  l_run[nt] += rs;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[sg][e] = (__bf16)s[8 * sg + e];
}

template <int D, int NT>
__device__ __forceinline__ void pv_pair(const bf16x8 (&vf)[2][D / 32], int nt, const bf16x8 (&pf)[2],
                                        f32x16 (&o)[NT][D / 32]) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
      o[nt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[sg][j], pf[sg], o[nt][j], 0, 0, 0);
}

// Page pairs of a sequence with committed length L0, capped by the grid's
// max_kv_len.
__device__ __forceinline__ int npairs_from_len(int L0, int K1, int np_cap) {
  const int L = L0 + K1;
  return min(np_cap, max(1, (L + kPairKeys - 1) / kPairKeys));
}
__device__ __forceinline__ int npairs_of(const int32_t* __restrict__ kv_len, int b, int K1, int np_cap) {
  return npairs_from_len(kv_len[b], K1, np_cap);
}

// Block-wide sum of one value per thread (fixed order; all threads get it).
template <int NTH>
__device__ __forceinline__ long long block_sum_ll(long long v, long long* s_red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) t += s_red[w];
  return t;
}

// The sequence b holding work item u and the index of its first item,
// Hkv * sum_{b' < b} npairs(b').  All threads return the same values.
template <int NTH>
__device__ void locate_work(const int32_t* __restrict__ kv_len, int B, int K1, int np_cap, int Hkv,
                            long long u, int& b_out, long long& off_out, long long* s_wsum,
                            long long* s_res, int* s_found) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __syncthreads();
  if (tid == 0) { s_found[0] = B; s_res[0] = 0; }
  long long carry = 0;
  for (int base = 0; base < B; base += NTH) {
    const int b = base + tid;
    const long long v = (b < B) ? (long long)npairs_of(kv_len, b, K1, np_cap) * Hkv : 0;
    long long incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    __syncthreads();
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    long long ex = carry + incl - v;
    for (int ww = 0; ww < wave; ++ww) ex += s_wsum[ww];
    if (b < B && ex <= u && u < ex + v) { s_found[0] = b; s_res[0] = ex; }
    long long tile = 0;
#pragma unroll
    for (int ww = 0; ww < NTH / 64; ++ww) tile += s_wsum[ww];
    carry += tile;
    __syncthreads();
    if (s_found[0] < B) break;
  }
  b_out = s_found[0];
  off_out = s_res[0];
  __syncthreads();
}

__host__ __device__ inline long long stream_start(int w, long long U, int W) { return (long long)w * U / W; }

// Work item u belongs to the last workgroup whose share starts at or before u.
__host__ __device__ inline int stream_owner(long long u, long long U, int W) {
  return (int)(((u + 1) * W - 1) / U);
}

// One (sequence, KV head) piece of a workgroup's share: pairs [p_lo, p_hi)
// of sequence b, KV head g.  Wave-uniform.
struct Seg {
  int b, g, np, off, p_lo, p_hi, end, slot, L0;
  bool full;
};

// The window rows of segment s that lie in its pairs [p_lo, p_hi) (the rest
// belong to another workgroup's share), as dwords (two d's of one row):
// loaded by window_rows_load into registers, then written by
// window_rows_store to the LDS stage.
template <int D, int NTH>
struct WinStage {
  static constexpr int N = (kWinRows * D / 2 + NTH - 1) / NTH;   // dwords per thread
  typedef uint32_t Regs[N];
};

template <int D, int NTH>
__device__ __forceinline__ void window_rows_load(typename WinStage<D, NTH>::Regs& reg, const Seg& s, int K1,
                                                 int Hkv, const uint16_t* __restrict__ vn, int tid) {
  const int i_lo = max(0, s.p_lo * kPairKeys - s.L0), i_hi = min(K1, s.p_hi * kPairKeys - s.L0);
#pragma unroll
  for (int r = 0; r < WinStage<D, NTH>::N; ++r) {
    const int e = i_lo * (D / 2) + tid + r * NTH;
    reg[r] = 0u;
    if (e < i_hi * (D / 2)) {
      const int i = e / (D / 2), d = 2 * (e - i * (D / 2));
      reg[r] = *reinterpret_cast<const uint32_t*>(vn + (((size_t)s.b * K1 + i) * Hkv + s.g) * D + d);
    }
  }
}

template <int D, int NTH>
__device__ __forceinline__ void window_rows_store(const typename WinStage<D, NTH>::Regs& reg, const Seg& s,
                                                  int K1, uint16_t* s_win, int tid) {
  const int i_lo = max(0, s.p_lo * kPairKeys - s.L0), i_hi = min(K1, s.p_hi * kPairKeys - s.L0);
#pragma unroll
  for (int r = 0; r < WinStage<D, NTH>::N; ++r) {
    const int e = i_lo * (D / 2) + tid + r * NTH;
    if (e < i_hi * (D / 2)) {
      const int i = e / (D / 2), d = 2 * (e - i * (D / 2));
      *reinterpret_cast<uint32_t*>(s_win + i * D + d) = reg[r];
    }
  }
}


// The piece after s in the share that ends at u1, if any.
__device__ __forceinline__ bool next_segment(const Seg& s, Seg& n, int u1, int B, int Hkv, int K1,
                                             int np_cap, const int32_t* __restrict__ kv_len) {
  n = s;
  if (s.end >= u1) return false;
  int nb = s.b, ng = s.g + 1, off = s.off, np = s.np;
  if (ng == Hkv) {
    ng = 0;
    off += s.np * Hkv;
    if (++nb >= B) return false;
    np = npairs_of(kv_len, nb, K1, np_cap);
  }
  n.b = nb;
  n.g = ng;
  n.off = off;
  n.np = np;
  n.p_lo = 0;
  n.end = min(u1, off + (ng + 1) * np);
  n.p_hi = n.end - (off + ng * np);
  n.slot = 1;
  n.full = (n.p_hi == np);
  n.L0 = kv_len[nb];
  return true;
}

// Q operand (B of S^T = K Q^T) of a piece: lane holds Q[row = nt*32 + l32]
// [kk*16 + hh*8 .. +8]; rows past G*(K+1) are zero.  am = the row's window
// node's ancestor-or-self set: from anc[b][i] for a tree, bits 0..i for the
// chain (anc == nullptr).
template <int D, int NT>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[NT][D / 16], uint32_t (&am)[NT],
                                       const uint16_t* __restrict__ q,
                                       const uint32_t* __restrict__ anc, const Seg& s, int K1,
                                       int Hq, int G, int rows, int l32, int hh) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = nt * 32 + l32;
    const bool valid = row < rows;
    const int hq = valid ? row / K1 : 0;
    const int i = valid ? row - hq * K1 : K1 - 1;
    am[nt] = (anc && valid) ? anc[(size_t)s.b * K1 + i] : ((2u << i) - 1u);
    const uint16_t* qp = q + (((size_t)s.b * K1 + i) * Hq + (size_t)s.g * G + hq) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (valid) {
        qf[nt][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hh * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[nt][kk][e] = (__bf16)0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 stream-K kernel.  grid (W), block 256.
// Partial slots: opart[((w * 2 + slot) * ROWS + row) * D + d] (fp32, scaled to
// the slot's max) and ml[(w * 2 + slot) * ROWS + row] = (max, sum), scores in
// base-2 units.  Slot 0: the segment that starts the workgroup's share;
// slot 1: a segment that starts later and runs past its end.
// ---------------------------------------------------------------------------
template <int D, int NT, bool WIN>
__global__ __launch_bounds__(64 * stream_waves<NT>(), NT == 1 ? SV_ATTN_WAVES_1T * 4 / stream_waves<NT>() : 1) void k_attn_stream(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ kv_len,
    const uint32_t* __restrict__ anc, uint16_t* __restrict__ out,
    int B, int K1, int Hq, int Hkv, int num_blocks, int mbps, int np_cap, float sl2, int W,
    float* __restrict__ opart, float2* __restrict__ ml, const uint16_t* __restrict__ kn,
    const uint16_t* __restrict__ vn) {
  constexpr int KK = D / 16;         // MFMA k-steps for S
  constexpr int DT = D / 32;         // d tiles for O
  constexpr int ROWS = 32 * NT;
  constexpr int OPAD = D + 4;        // LDS row stride (floats)
  constexpr int NW = stream_waves<NT>();
  constexpr int kStreamThreads = 64 * NW;
  constexpr int TPR = kStreamThreads / 32;   // epilogue threads per output row
  constexpr int DPT = D / TPR;               // output d's per thread in the epilogue
  __shared__ float s_o[NW][32][OPAD];        // one buffer per wave for the segment merge
  __shared__ uint16_t s_win[WIN ? 2 : 1][WIN ? kWinRows * D : 1];   // window V stage, double buffered
  __shared__ float s_m[NW][32], s_l[NW][32];
  __shared__ long long s_red[NW];
  __shared__ long long s_res[1];
  __shared__ int s_found[3];
  __shared__ int s_wsum[NW];

  const int w = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar pair indices
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = Hq / Hkv;
  const int rows = G * K1;
#if SV_ATTN_TIMESTAMPS
  unsigned long long* tsp = g_attn_ts + ((size_t)w * NW + wave) * kTsEv;
  int tsk = 0;
  SV_TS(0);
  if (lane == 0) { tsp[kTsEv - 2] = NW; tsp[kTsEv - 1] = 0ull; }
#endif

  // The share [u0, u1) needs the total work U, and its first item's
  // sequence b with that sequence's first item off_b.  The host bounds the
  // work list below 2^30 items, so these fit int; values that come back
  // through LDS are made wave-uniform (scalar registers).
  int U, u0, u1, b, off_b, L0b;
  if (B <= kStreamThreads) {
    // One read of kv_len and one block scan give all of it.
    const int kvb = tid < B ? kv_len[tid] : 0;
    const int v = tid < B ? npairs_from_len(kvb, K1, np_cap) * Hkv : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane == 63) s_wsum[tid >> 6] = incl;
    if (tid == 0) s_found[0] = B;
    __syncthreads();
    int ex = incl - v, tot = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      ex += (ww < (tid >> 6)) ? s_wsum[ww] : 0;
      tot += s_wsum[ww];
    }
    U = __builtin_amdgcn_readfirstlane(tot);
    u0 = (int)stream_start(w, U, W);
    u1 = (int)stream_start(w + 1, U, W);
    if (tid < B && ex <= u0 && u0 < ex + v) { s_found[0] = tid; s_found[1] = ex; s_found[2] = kvb; }
    __syncthreads();
    if (u0 >= u1) return;
    b = __builtin_amdgcn_readfirstlane(s_found[0]);
    off_b = __builtin_amdgcn_readfirstlane(s_found[1]);
    L0b = __builtin_amdgcn_readfirstlane(s_found[2]);
  } else {
    long long tot = 0;
    for (int bb = tid; bb < B; bb += kStreamThreads) tot += (long long)npairs_of(kv_len, bb, K1, np_cap) * Hkv;
    U = __builtin_amdgcn_readfirstlane((int)block_sum_ll<kStreamThreads>(tot, s_red));
    u0 = (int)stream_start(w, U, W);
    u1 = (int)stream_start(w + 1, U, W);
    if (u0 >= u1) return;
    long long off;
    locate_work<kStreamThreads>(kv_len, B, K1, np_cap, Hkv, u0, b, off, s_red, s_res, s_found);
    b = __builtin_amdgcn_readfirstlane(b);
    off_b = __builtin_amdgcn_readfirstlane((int)off);
    L0b = b < B ? kv_len[b] : 0;
  }
  if (b >= B) return;                       // u0 < U always finds a sequence
  // K operand row of this lane: MFMA key mk = l32 -> page mk>>4, token below.
  const int k_page = l32 >> 4;
  const int k_tok = 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);

  // The share's first segment.
  Seg cur;
  cur.b = b;
  cur.np = npairs_from_len(L0b, K1, np_cap);     // L0b is kv_len[b], already read
  cur.g = (u0 - off_b) / cur.np;
  cur.off = off_b;
  cur.p_lo = (u0 - off_b) - cur.g * cur.np;
  cur.end = min(u1, off_b + (cur.g + 1) * cur.np);
  cur.p_hi = cur.p_lo + (cur.end - u0);
  cur.slot = 0;
  cur.full = (cur.p_lo == 0) && (cur.p_hi == cur.np);
  cur.L0 = L0b;

  // Wave v takes pairs p_lo + v, p_lo + v + NW, ... of each piece.
  // First K/V as early as possible: page table, then the pages, then Q.
  bf16x8 kf[KK];
  bf16x8 vf[2][DT];
  // (A pair with window keys taken from k_new / v_new is loaded by the loop
  // that runs it.)
  int pr = cur.p_lo + wave;
  if (pr < cur.p_hi && !(WIN && pair_has_window(pr, cur.L0, K1))) {
    int blk[2];
    pair_blocks(blk, pr, bt + (size_t)cur.b * mbps, mbps, num_blocks);
    load_k<D>(kf, blk, kc, Hkv, cur.g, k_page, k_tok, hh);
    load_v<D>(vf, blk, vc, Hkv, cur.g, l32, hh);
  }
  bf16x8 qf[NT][KK];
  uint32_t am[NT];
  load_q<D, NT>(qf, am, q, anc, cur, K1, Hq, G, rows, l32, hh);
  int wbuf = 0;                                    // stage of the current segment's window
  if (WIN) {
    uint32_t stg[WinStage<D, kStreamThreads>::N];
    window_rows_load<D, kStreamThreads>(stg, cur, K1, Hkv, vn, tid);
    window_rows_store<D, kStreamThreads>(stg, cur, K1, s_win[0], tid);
  }
  __syncthreads();
#if SV_ATTN_TIMESTAMPS
  SV_TS(1);
#endif

  while (true) {
    Seg nxt;
    const bool has_next = next_segment(cur, nxt, u1, B, Hkv, K1, np_cap, kv_len);
    const int nxt_first = nxt.p_lo + wave;        // this wave's first pair of nxt
    const bool nxt_mine = has_next && nxt_first < nxt.p_hi;
    // ... and whether that pair holds window keys from k_new / v_new: then
    // it is not prefetched here.
    const bool nxt_win = WIN && nxt_mine && pair_has_window(nxt_first, nxt.L0, K1);

    f32x16 o[NT][DT];
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = -INFINITY;
      l_run[nt] = 0.f;
#pragma unroll
      for (int j = 0; j < DT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nt][j][r] = 0.f;
    }

    // Staggered pipeline over this wave's pairs (4 apart): the next pair's K
    // is requested right after this pair's scores and its V right after P.V.
    // After the last pair of the segment, the "next pair" is this wave's
    // first pair of the next segment, so its loads fly during the merge.
    // With the window taken from k_new / v_new, the pairs that hold window
    // keys (from L0 / 32 on: the last one or two of the sequence) run after
    // the others in a loop of their own that also makes their loads, so the
    // main loop keeps the plain kernel's register budget.
    const int32_t* btb = bt + (size_t)cur.b * mbps;
    const int L = cur.L0 + K1;
    const int p_main = WIN ? min(cur.p_hi, max(cur.p_lo, cur.L0 / kPairKeys)) : cur.p_hi;
    bool prefetched = false;
    while (pr < p_main) {
      const int nx = pr + NW;
      const bool in_seg = nx < p_main;
      const bool cross = !in_seg && nx >= cur.p_hi && nxt_mine && !nxt_win;
      int nblk[2] = {0, 0};
      if (in_seg) pair_blocks(nblk, nx, btb, mbps, num_blocks);
      else if (cross) pair_blocks(nblk, nxt_first, bt + (size_t)nxt.b * mbps, mbps, num_blocks);
      const int ng = cross ? nxt.g : cur.g;
      bf16x8 pf[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        score_pair<D, NT>(kf, pr, hh, nt, qf, am, cur.L0, sl2, o, m_run, l_run, pf[nt]);
      if (in_seg || cross) load_k<D>(kf, nblk, kc, Hkv, ng, k_page, k_tok, hh);
      mask_v_tail<D>(vf, pr, L, hh);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pv_pair<D, NT>(vf, nt, pf[nt], o);
      if (in_seg || cross) load_v<D>(vf, nblk, vc, Hkv, ng, l32, hh);
      prefetched |= cross;
      pr = (in_seg || nx < cur.p_hi) ? nx : cur.p_hi;
    }
    if (WIN) {
      // This wave's window pairs, each loaded here: K from k_new for the
      // window keys, V from the staged rows.
      for (; pr < cur.p_hi; pr += NW) {
        int blk[2];
        pair_blocks(blk, pr, btb, mbps, num_blocks);
        load_k_window<D>(kf, blk, kc, kn, cur.b, K1, Hkv, cur.g, cur.L0, pr, k_page, k_tok, hh);
        load_v<D>(vf, blk, vc, Hkv, cur.g, l32, hh);
        bf16x8 pf[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          score_pair<D, NT>(kf, pr, hh, nt, qf, am, cur.L0, sl2, o, m_run, l_run, pf[nt]);
        window_v<D>(vf, s_win[wbuf], K1, cur.L0, pr, l32, hh);
        mask_v_tail<D>(vf, pr, L, hh);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pv_pair<D, NT>(vf, nt, pf[nt], o);
      }
    }
    if (nxt_mine && !prefetched && !nxt_win) {     // no pair of mine in cur
      int nblk[2];
      pair_blocks(nblk, nxt_first, bt + (size_t)nxt.b * mbps, mbps, num_blocks);
      load_k<D>(kf, nblk, kc, Hkv, nxt.g, k_page, k_tok, hh);
      load_v<D>(vf, nblk, vc, Hkv, nxt.g, l32, hh);
    }

#if SV_ATTN_TIMESTAMPS
    if (tsk < kTsSeg) SV_TS(2 + 2 * tsk);
#endif
    // The next segment's window rows, staged before this segment's merge
    // (whose barrier orders them before their use).  Requested only after
    // the pair loop: held across it, they would push the loop past the
    // register budget.
    if (WIN && has_next) {
      uint32_t stg[WinStage<D, kStreamThreads>::N];
      window_rows_load<D, kStreamThreads>(stg, nxt, K1, Hkv, vn, tid);
      window_rows_store<D, kStreamThreads>(stg, nxt, K1, s_win[wbuf ^ 1], tid);
    }

    // Merge the 4 waves one 32-row tile at a time: each wave stores its O,
    // rescaled to the common row max, in its own LDS buffer; the sum over
    // waves is taken in fixed order 0..3.  Then the output rows (whole
    // segment) or the partial are written.
    const size_t part_base = ((size_t)w * 2 + cur.slot) * ROWS;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (lane < 32) { s_m[wave][l32] = m_run[nt]; s_l[wave][l32] = l_run[nt]; }
      __syncthreads();
      float mall = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) mall = fmaxf(mall, s_m[ww][l32]);
      const float f = exp2_dev(m_run[nt] - ((mall == -INFINITY) ? 0.f : mall));
#pragma unroll
      for (int j = 0; j < DT; ++j)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          // regs 4qd..4qd+3 hold d = 32j + 8qd + 4hh + 0..3
          *reinterpret_cast<float4*>(&s_o[wave][l32][32 * j + 8 * qd + 4 * hh]) =
              make_float4(o[nt][j][4 * qd] * f, o[nt][j][4 * qd + 1] * f,
                          o[nt][j][4 * qd + 2] * f, o[nt][j][4 * qd + 3] * f);
        }
      __syncthreads();
      const int row_l = tid / TPR;
      const int d0 = (tid % TPR) * DPT;
      const int row = nt * 32 + row_l;
      float mrow = s_m[0][row_l];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) mrow = fmaxf(mrow, s_m[ww][row_l]);
      const float mu = (mrow == -INFINITY) ? 0.f : mrow;
      float lsum = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) lsum += s_l[ww][row_l] * exp2_dev(s_m[ww][row_l] - mu);
      float acc[DPT];
#pragma unroll
      for (int e = 0; e < DPT; e += 4) {
        float4 v = *reinterpret_cast<const float4*>(&s_o[0][row_l][d0 + e]);
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
          const float4 a = *reinterpret_cast<const float4*>(&s_o[ww][row_l][d0 + e]);
          v.x = a.x + v.x; v.y = a.y + v.y; v.z = a.z + v.z; v.w = a.w + v.w;
        }
        acc[e] = v.x; acc[e + 1] = v.y; acc[e + 2] = v.z; acc[e + 3] = v.w;
      }
      if (row < rows) {
        if (cur.full) {
          const int hq = row / K1, i = row - hq * K1;
          uint16_t* op = out + (((size_t)cur.b * K1 + i) * Hq + (size_t)cur.g * G + hq) * D + d0;
          const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
          for (int e = 0; e < DPT; e += 2) {
            const __bf16 lo = (__bf16)(acc[e] * inv);
            const __bf16 hi = (__bf16)(acc[e + 1] * inv);
            const uint32_t wd = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            *reinterpret_cast<uint32_t*>(op + e) = wd;
          }
        } else {
          float* pp = opart + (part_base + row) * D + d0;
#pragma unroll
          for (int e = 0; e < DPT; e += 4)
            *reinterpret_cast<float4*>(pp + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
          if (tid % TPR == 0) ml[part_base + row] = make_float2(mrow, lsum);
        }
      }
      __syncthreads();
    }

#if SV_ATTN_TIMESTAMPS
    if (tsk < kTsSeg) SV_TS(3 + 2 * tsk);
    ++tsk;
    if (lane == 0) tsp[kTsEv - 1] = tsk;
#endif
    if (!has_next) break;
    cur = nxt;
    wbuf ^= 1;
    // Q of the new segment (the loads of its first pair are already in flight).
    load_q<D, NT>(qf, am, q, anc, cur, K1, Hq, G, rows, l32, hh);
    pr = cur.p_lo + wave;
  }
}

// ---------------------------------------------------------------------------
// Merge of the segments that span several workgroups.  grid (Hkv, B, z),
// block 256: TPR threads per row, each with D / TPR of the coordinates,
// 256 / TPR rows per block pass; the z blocks of a segment take every z-th
// group of rows.  Two shapes: with enough segments to fill the chip (short
// spans of partials) 8 threads per row, all rows in one pass, z = 1; with
// few segments (long spans) D/4 threads per row and the rows spread over
// blocks.  One pass over the partials in share order with a running
// maximum: each thread requests the next NB partials before it adds the
// current ones, rescales its sums when a batch raises the maximum and adds
// the batch in order, so the result does not depend on the launch shape.
// ---------------------------------------------------------------------------
template <int D, int NT, int TPR, int NB>
__global__ __launch_bounds__(kCombineThreads) void k_attn_stream_combine(
    const float* __restrict__ opart, const float2* __restrict__ ml, const int32_t* __restrict__ kv_len,
    uint16_t* __restrict__ out, int B, int K1, int Hq, int Hkv, int np_cap, int W) {
  constexpr int ROWS = 32 * NT;
  constexpr int DPT = D / TPR;                  // coordinates per thread
  constexpr int NV = DPT / 4;                   // float4 per partial per thread
  constexpr int RPB = kCombineThreads / TPR;
  static_assert(DPT % 4 == 0, "whole float4 per thread");
  __shared__ long long s_red[kCombineThreads / 64];
  __shared__ int s_slot[kStreamMaxWG];
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  long long tot = 0, before = 0;
  for (int bb = tid; bb < B; bb += kCombineThreads) {
    const long long v = (long long)npairs_of(kv_len, bb, K1, np_cap) * Hkv;
    tot += v;
    if (bb < b) before += v;
  }
  const long long U = block_sum_ll<kCombineThreads>(tot, s_red);
  const long long off_b = block_sum_ll<kCombineThreads>(before, s_red);
  const int np = npairs_of(kv_len, b, K1, np_cap);
  const long long ua = off_b + (long long)g * np, ub = ua + np;
  const int wa = stream_owner(ua, U, W), wb = stream_owner(ub - 1, U, W);
  if (wa == wb) return;                       // written whole by its workgroup
  const int G = Hq / Hkv;
  const int rows = G * K1;
  const int d0 = (tid % TPR) * DPT;
  // The partial slot of each share of the segment (slot 1 for a first share
  // that starts inside it), -1 for an empty share.
  const int nparts = wb - wa + 1;
  for (int k = tid; k < nparts; k += kCombineThreads) {
    const int ww = wa + k;
    const long long s0 = stream_start(ww, U, W);
    s_slot[k] = s0 >= stream_start(ww + 1, U, W) ? -1 : ww * 2 + ((k == 0 && s0 != ua) ? 1 : 0);
  }
  __syncthreads();
  for (int row = blockIdx.z * RPB + tid / TPR; row < rows; row += gridDim.z * RPB) {
    float m = -INFINITY, lsum = 0.f;
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
    // Batches of NB partials in two register buffers; the next batch is
    // requested before the current one is added.
    float2 sa[NB], sb[NB];
    float4 va[NB][NV], vb[NB][NV];
    auto fetch = [&](int k0, float2 (&st)[NB], float4 (&v)[NB][NV]) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        st[j].x = -INFINITY;                      // weight 0 unless loaded below
        const int sl = k0 + j < nparts ? s_slot[k0 + j] : -1;
        if (sl >= 0) {
          const size_t ix = (size_t)sl * ROWS + row;
          st[j] = ml[ix];
          const float4* pp = reinterpret_cast<const float4*>(opart + ix * D + d0);
#pragma unroll
          for (int q = 0; q < NV; ++q) v[j][q] = pp[q];
        }
      }
    };
    auto add = [&](const float2 (&st)[NB], const float4 (&v)[NB][NV]) {
      float mb = m;
#pragma unroll
      for (int j = 0; j < NB; ++j) mb = fmaxf(mb, st[j].x);
      if (mb > m) {                               // a larger maximum: rescale the sums
        const float r = exp2_dev(m - mb);         // 0 while nothing was added
        lsum *= r;
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] *= r;
        m = mb;
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (st[j].x == -INFINITY) continue;       // empty share, or no visible key
        const float f = exp2_dev(st[j].x - m);
        lsum += st[j].y * f;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
          acc[4 * q] += v[j][q].x * f; acc[4 * q + 1] += v[j][q].y * f;
          acc[4 * q + 2] += v[j][q].z * f; acc[4 * q + 3] += v[j][q].w * f;
        }
      }
    };
    fetch(0, sa, va);
    for (int k0 = 0; k0 < nparts; k0 += 2 * NB) {
      if (k0 + NB < nparts) fetch(k0 + NB, sb, vb);
      add(sa, va);
      if (k0 + NB >= nparts) break;
      if (k0 + 2 * NB < nparts) fetch(k0 + 2 * NB, sa, va);
      add(sb, vb);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int hq = row / K1, i = row - hq * K1;
    uint16_t* op = out + (((size_t)b * K1 + i) * Hq + (size_t)g * G + hq) * D + d0;
#pragma unroll
    for (int e = 0; e < DPT; e += 4) {
      const __bf16 o0 = (__bf16)(acc[e] * inv), o1 = (__bf16)(acc[e + 1] * inv);
      const __bf16 o2 = (__bf16)(acc[e + 2] * inv), o3 = (__bf16)(acc[e + 3] * inv);
      const uint32_t w01 = (uint32_t)__builtin_bit_cast(uint16_t, o0) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, o1) << 16);
      const uint32_t w23 = (uint32_t)__builtin_bit_cast(uint16_t, o2) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, o3) << 16);
      *reinterpret_cast<uint2*>(op + e) = make_uint2(w01, w23);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: grid (K1, Hq, B), block 64 (one wave per query row).
// k_cache [NB, Hkv, D/4, 16, 4], v_cache [NB, Hkv, D, 16].  With kn / vn the
// window keys are read from there (never from the cache).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_attn_valu(
    const float* __restrict__ q, float* __restrict__ kc, float* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ kv_len,
    const uint32_t* __restrict__ anc, float* __restrict__ out,
    int K1, int Hq, int Hkv, int D, int num_blocks, int mbps, float sl2,
    const float* __restrict__ kn, const float* __restrict__ vn) {
  __shared__ float s_q[256];
  __shared__ float s_p[64];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = h / (Hq / Hkv);
  const int L0 = kv_len[b];
  const int t = L0 + i;                           // last key that can be visible
  const uint32_t am = anc ? anc[(size_t)b * K1 + i] : ((2u << i) - 1u);
  const float* qp = q + (((size_t)b * K1 + i) * Hq + h) * D;
  for (int d = lane; d < D; d += 64) s_q[d] = qp[d];
  __syncthreads();
  const int32_t* btb = bt + (size_t)b * mbps;
  const size_t page = (size_t)D * 16;
  float m_run = -INFINITY, l_run = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};              // d = lane + 64 * c
  for (int j0 = 0; j0 <= t; j0 += 64) {
    const int j = j0 + lane;
    float sc = -INFINITY;
    const unsigned jw = (unsigned)(j - L0);
    if (j <= t && (jw >= 32u || ((am >> jw) & 1u))) {
      float acc = 0.f;
      if (kn && j >= L0) {
        const float* kp = kn + (((size_t)b * K1 + (j - L0)) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) acc += s_q[d] * kp[d];
      } else {
        const int blk = clampi(btb[min(j >> 4, mbps - 1)], 0, num_blocks - 1);
        const float* kp = kc + ((size_t)blk * Hkv + g) * page;
        const int tok = j & 15;
        for (int d = 0; d < D; ++d) acc += s_q[d] * kp[((d >> 2) * 16 + tok) * 4 + (d & 3)];
      }
      sc = acc * sl2;
    }
    float mx = sc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_dev(m_run - m_new);
    const float p = exp2_dev(sc - m_new);
    const float ps = wave_sum(p);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    s_p[lane] = p;
    __syncthreads();
    for (int c = 0; c < 4; ++c) o[c] *= alpha;
    const int nk = min(64, t + 1 - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const int jk = j0 + jj;
      const float pj = s_p[jj];
      if (kn && jk >= L0) {
        const float* vp = vn + (((size_t)b * K1 + (jk - L0)) * Hkv + g) * D;
        for (int c = 0; c < 4; ++c) {
          const int d = lane + 64 * c;
          if (d < D) o[c] += pj * vp[d];
        }
      } else {
        const int blk = clampi(btb[min(jk >> 4, mbps - 1)], 0, num_blocks - 1);
        const float* vp = vc + ((size_t)blk * Hkv + g) * page;
        for (int c = 0; c < 4; ++c) {
          const int d = lane + 64 * c;
          if (d < D) o[c] += pj * vp[d * 16 + (jk & 15)];
        }
      }
    }
    __syncthreads();
  }
  float* op = out + (((size_t)b * K1 + i) * Hq + h) * D;
  for (int c = 0; c < 4; ++c) {
    const int d = lane + 64 * c;
    if (d < D) op[d] = o[c] / l_run;
  }
}

static inline int attn_tiles(int G, int K1) { return (G * K1 + 31) / 32; }

struct AttnPlan {
  int w_max, tiles, np_cap;
  bool too_big;
  size_t opart_bytes, ml_bytes;
};

// The workspace depends on the arguments only: partial slots for the largest
// grid these arguments can get.  The grid itself also depends on the device.
static inline AttnPlan attn_plan(int B, int K, int Hq, int Hkv, int D, int max_kv_len) {
  AttnPlan p{};
  const int K1 = K + 1;
  p.tiles = attn_tiles(Hq / Hkv, K1);
  p.np_cap = (max_kv_len + K1 + kPairKeys - 1) / kPairKeys;
  const long long u_max = (long long)B * Hkv * p.np_cap;
  p.too_big = u_max >= (1LL << 30);
  const long long w_max = std::max<long long>(
      1, std::min<long long>(u_max / SV_ATTN_MIN_PAIRS_PER_WG, kStreamMaxWG));
  p.w_max = (int)w_max;
  const size_t slots = w_max > 1 ? (size_t)w_max * 2 * 32 * p.tiles : 0;
  p.opart_bytes = (slots * D * sizeof(float) + 255) & ~(size_t)255;
  p.ml_bytes = (slots * sizeof(float2) + 255) & ~(size_t)255;
  return p;
}

// Workgroups of k_attn_stream<D, NT> that are resident on one CU at once
// (queried once per process; every caller stores the same value).
template <int D, int NT, bool WIN>
static int stream_blocks_per_cu() {
  static std::atomic<int> cached{0};
  int nb = cached.load(std::memory_order_relaxed);
  if (nb > 0) return nb;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&k_attn_stream<D, NT, WIN>),
                                                   64 * stream_waves<NT>(), 0) != hipSuccess || nb <= 0)
    nb = 1;
  cached.store(nb, std::memory_order_relaxed);
  return nb;
}

// Window source: kn / vn == nullptr means the window is already in the cache.
struct WindowArgs {
  const void* kn;
  const void* vn;
  int store;
};

template <int D, int NT, bool WIN>
static hipError_t launch_stream_t(const void* q, void* kc, void* vc, const int32_t* bt,
                                  const int32_t* kv_len, const uint32_t* anc, void* out, int B, int K1,
                                  int Hq, int Hkv, int num_blocks, int mbps, float sl2,
                                  const AttnPlan& p, char* ws, const WindowArgs& win, hipStream_t st) {
  // Persistent grid: every workgroup resident from the start.
  const int W = (int)std::min<long long>(
      p.w_max, (long long)stream_blocks_per_cu<D, NT, WIN>() * std::max(1, device_cus()));
  float* opart = reinterpret_cast<float*>(ws);
  float2* ml = reinterpret_cast<float2*>(ws + p.opart_bytes);
  hipLaunchKernelGGL((k_attn_stream<D, NT, WIN>), dim3(W), dim3(64 * stream_waves<NT>()), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<uint16_t*>(kc),
                     static_cast<uint16_t*>(vc), bt, kv_len, anc, static_cast<uint16_t*>(out), B,
                     K1, Hq, Hkv, num_blocks, mbps, p.np_cap, sl2, W, opart, ml,
                     static_cast<const uint16_t*>(win.kn), static_cast<const uint16_t*>(win.vn));
  if (W > 1) {
    const int rows = (Hq / Hkv) * K1;
    if ((long long)B * Hkv >= device_cus()) {
      hipLaunchKernelGGL((k_attn_stream_combine<D, NT, 8, 2>), dim3(Hkv, B, 1), dim3(kCombineThreads),
                         0, st, opart, ml, kv_len, static_cast<uint16_t*>(out), B, K1, Hq, Hkv,
                         p.np_cap, W);
    } else {
      // Few segments, each spread over many workgroups: rows over blocks too.
      constexpr int rpb = kCombineThreads / (D / 4);
      hipLaunchKernelGGL((k_attn_stream_combine<D, NT, D / 4, 8>), dim3(Hkv, B, (rows + rpb - 1) / rpb),
                         dim3(kCombineThreads), 0, st, opart, ml, kv_len, static_cast<uint16_t*>(out), B,
                         K1, Hq, Hkv, p.np_cap, W);
    }
  }
  return hipGetLastError();
}

template <int D, int NT>
static hipError_t launch_stream(const void* q, void* kc, void* vc, const int32_t* bt,
                                const int32_t* kv_len, const uint32_t* anc, void* out, int B, int K1,
                                int Hq, int Hkv, int num_blocks, int mbps, float sl2,
                                const AttnPlan& p, char* ws, const WindowArgs& win, hipStream_t st) {
  return win.kn ? launch_stream_t<D, NT, true>(q, kc, vc, bt, kv_len, anc, out, B, K1, Hq, Hkv,
                                               num_blocks, mbps, sl2, p, ws, win, st)
                : launch_stream_t<D, NT, false>(q, kc, vc, bt, kv_len, anc, out, B, K1, Hq, Hkv,
                                                num_blocks, mbps, sl2, p, ws, win, st);
}

}  // namespace sv

#if SV_ATTN_TIMESTAMPS
// The stamps of the last k_attn_stream launch (see SV_ATTN_TIMESTAMPS):
// copies min(bytes, their size) bytes to host memory; returns the size.
extern "C" size_t spec_attn_timestamps(void* host, size_t bytes) {
  const size_t n = sizeof(sv::g_attn_ts);
  if (host && bytes) {
    if (hipDeviceSynchronize() != hipSuccess) return 0;
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(sv::g_attn_ts), bytes < n ? bytes : n, 0,
                            hipMemcpyDeviceToHost) != hipSuccess)
      return 0;
  }
  return n;
}
#endif

extern "C" size_t spec_verify_attn_workspace_bytes(int B, int K, int Hq, int Hkv, int D,
                                                   int max_kv_len) {
  if (B <= 0 || K < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_kv_len < 0) return 0;
  const sv::AttnPlan p = sv::attn_plan(B, K, Hq, Hkv, D, max_kv_len);
  return p.opart_bytes + p.ml_bytes;
}

namespace sv {

static int verify_attn_impl(const void* q, void* k_cache, void* v_cache,
                            const int32_t* block_table, const int32_t* kv_len, const uint32_t* anc,
                            void* out, int B, int K, int Hq, int Hkv, int D, int block_size,
                            int num_blocks, int max_blocks_per_seq, int max_kv_len, float scale,
                            int dtype, void* workspace, size_t workspace_bytes, void* hip_stream,
                            const WindowArgs& win, const char* fn) {
  if (B < 0 || K < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_kv_len < 0 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (K > SV_MAX_K || block_size != SV_BLOCK_SIZE || (D != 64 && D != 128) || Hq % Hkv != 0 ||
      (Hq / Hkv) * (K + 1) > 64)
    return SV_ERR_UNSUPPORTED;
  if ((long long)max_kv_len + K + 1 > (long long)max_blocks_per_seq * SV_BLOCK_SIZE)
    return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!q || !k_cache || !v_cache || !block_table || !kv_len || !out) return SV_ERR_INVALID_ARG;
  if ((win.kn == nullptr) != (win.vn == nullptr)) return SV_ERR_INVALID_ARG;
  // The append copy moves 16-byte vectors (either dtype).
  if (win.kn && win.store &&
      ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
        reinterpret_cast<uintptr_t>(win.kn) | reinterpret_cast<uintptr_t>(win.vn)) & 15))
    return SV_ERR_INVALID_ARG;
  if (B > 65535 || Hkv > 65535) return SV_ERR_UNSUPPORTED;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  const float sl2 = sc * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int K1 = K + 1;
  const AttnPlan p = attn_plan(B, K, Hq, Hkv, D, max_kv_len);
  if (dtype == SV_BF16) {
    if (p.too_big) return SV_ERR_UNSUPPORTED;
    if (p.w_max > 1) {
      if (!workspace) return SV_ERR_INVALID_ARG;
      if (workspace_bytes < p.opart_bytes + p.ml_bytes) return SV_ERR_WORKSPACE;
      if (reinterpret_cast<uintptr_t>(workspace) & 255) return SV_ERR_INVALID_ARG;
    }
    const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                         reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out) |
                         reinterpret_cast<uintptr_t>(win.kn) | reinterpret_cast<uintptr_t>(win.vn);
    if (al & 15) return SV_ERR_INVALID_ARG;
  }
  const bool chk = validate_on();
  if (chk) {
    const int s = check_pages(fn, block_table, kv_len, B, K1, num_blocks, max_blocks_per_seq,
                              max_kv_len, st);
    if (s != SV_OK) return s;
  }
  hipError_t e;
  WindowArgs win_r = win;
  if (win.kn && win.store) {
    // Append: the window rows go into their slots first (one small copy
    // kernel), and the attention then reads the whole window from the cache.
    e = launch_window_store(k_cache, v_cache, block_table, kv_len, win.kn, win.vn, B, K1, Hkv, D,
                            num_blocks, max_blocks_per_seq, dtype, st);
    if (e != hipSuccess) return chk ? finish(fn, st, SV_ERR_HIP) : SV_ERR_HIP;
    win_r = WindowArgs{nullptr, nullptr, 0};
  }
  if (dtype == SV_F32) {
    hipLaunchKernelGGL(k_attn_valu, dim3(K1, Hq, B), dim3(64), 0, st,
                       static_cast<const float*>(q), static_cast<float*>(k_cache),
                       static_cast<float*>(v_cache), block_table, kv_len, anc,
                       static_cast<float*>(out), K1, Hq, Hkv, D, num_blocks, max_blocks_per_seq, sl2,
                       static_cast<const float*>(win_r.kn), static_cast<const float*>(win_r.vn));
    e = hipGetLastError();
  } else {
    char* ws = static_cast<char*>(workspace);
    if (D == 128) {
      e = p.tiles == 1 ? launch_stream<128, 1>(q, k_cache, v_cache, block_table, kv_len, anc, out, B,
                                               K1, Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, win_r, st)
                       : launch_stream<128, 2>(q, k_cache, v_cache, block_table, kv_len, anc, out, B,
                                               K1, Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, win_r, st);
    } else {
      e = p.tiles == 1 ? launch_stream<64, 1>(q, k_cache, v_cache, block_table, kv_len, anc, out, B,
                                              K1, Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, win_r, st)
                       : launch_stream<64, 2>(q, k_cache, v_cache, block_table, kv_len, anc, out, B,
                                              K1, Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, win_r, st);
    }
  }
  const int status = e == hipSuccess ? SV_OK : SV_ERR_HIP;
  return chk ? finish(fn, st, status) : status;
}

}  // namespace sv

extern "C" int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* kv_len, void* out, int B,
                                int K, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_kv_len, float scale, int dtype,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
  return sv::verify_attn_impl(q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), block_table,
                              kv_len, nullptr, out, B, K, Hq, Hkv,
                              D, block_size, num_blocks, max_blocks_per_seq, max_kv_len, scale, dtype,
                              workspace, workspace_bytes, hip_stream,
                              sv::WindowArgs{nullptr, nullptr, 0}, "spec_verify_attn");
}

extern "C" int spec_verify_attn_tree(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* kv_len,
                                     const uint32_t* anc, void* out, int B, int N, int Hq, int Hkv,
                                     int D, int block_size, int num_blocks, int max_blocks_per_seq,
                                     int max_kv_len, float scale, int dtype, void* workspace,
                                     size_t workspace_bytes, void* hip_stream) {
  if (B > 0 && !anc) return SV_ERR_INVALID_ARG;
  if (N < 2) return SV_ERR_INVALID_ARG;
  return sv::verify_attn_impl(q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), block_table,
                              kv_len, anc, out, B, N - 1, Hq, Hkv,
                              D, block_size, num_blocks, max_blocks_per_seq, max_kv_len, scale, dtype,
                              workspace, workspace_bytes, hip_stream,
                              sv::WindowArgs{nullptr, nullptr, 0}, "spec_verify_attn_tree");
}

extern "C" int spec_verify_attn_window(const void* q, const void* k_new, const void* v_new,
                                       void* k_cache, void* v_cache, const int32_t* block_table,
                                       const int32_t* kv_len, const uint32_t* anc, void* out, int B,
                                       int N, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                       int max_blocks_per_seq, int max_kv_len, float scale, int dtype,
                                       int mode, void* workspace, size_t workspace_bytes,
                                       void* hip_stream) {
  if (N < 2) return SV_ERR_INVALID_ARG;
  if (mode != SV_WINDOW_READ && mode != SV_WINDOW_APPEND) return SV_ERR_INVALID_ARG;
  if (B > 0 && (!k_new || !v_new)) return SV_ERR_INVALID_ARG;
  return sv::verify_attn_impl(q, k_cache, v_cache, block_table, kv_len, anc, out, B, N - 1, Hq, Hkv, D,
                              block_size, num_blocks, max_blocks_per_seq, max_kv_len, scale, dtype,
                              workspace, workspace_bytes, hip_stream,
                              sv::WindowArgs{k_new, v_new, mode == SV_WINDOW_APPEND ? 1 : 0},
                              "spec_verify_attn_window");
}
